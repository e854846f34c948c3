"""GPU parity of the LM-head pass with the selector's rank projection riding
along (dflash_lm_topk_proj) and of the edge scores from that projection
(dflash_candidate_edges_hp): ids and logits bit-identical to dflash_lm_topk,
hp against the oracle's hidden_projection, edges against the oracle's
DFlash2BeamCandidateSelector scores."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import assert_close, check_edges

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _check_hp(hp, H, Wp, what):
    ref = O.rank_projection(H, Wp)
    assert_close(hp, ref, what)
    # fp32 sums of exact bf16 products: far inside the value tolerance
    err = np.abs(hp.astype(np.float64) - ref).max()
    assert err <= 1e-4 * max(1.0, np.abs(ref).max()), f"{what}: max |hp - ref| = {err:.3g}"


def _fused_vs_plain(B, d, k, s, c, what):
    from tests.gpu_common import dev_bf16, say
    H, W, Wp = dev_bf16(d["H"]), dev_bf16(d["W"]), dev_bf16(d["Wp"])
    ids0, lg0 = B.lm_topk(H, W, k, s, c)
    ids1, lg1, hp = B.lm_topk_proj(H, W, k, s, c, Wp)
    assert np.array_equal(ids0.cpu().numpy(), ids1.cpu().numpy()), f"{what}: ids differ from dflash_lm_topk"
    assert np.array_equal(lg0.cpu().numpy().view(np.uint32), lg1.cpu().numpy().view(np.uint32)), \
        f"{what}: logits differ from dflash_lm_topk"
    hp_h = hp.cpu().numpy()
    _check_hp(hp_h, d["H"], d["Wp"], what)
    say(f"[fused {what}] ids/logits identical, hp ok")
    return ids1, lg1, hp


@pytest.mark.parametrize("T,V,Hd,k,R", [
    # W_proj's rows in extra tiles of group 0:
    (512, 32768, 2048, 8, 64),     # mid-like (V % 256 == 0)
    (300, 5000, 520, 16, 48),      # ragged rows and vocabulary, Hd % 64 != 0, R % 32 != 0
    (64, 4096, 256, 4, 144),       # 128-wide tiles: two projection tiles
    (8, 1000, 64, 1, 16),          # one row tile, k = 1
    # W_proj's rows in the free columns of the last vocabulary tile:
    (2048, 8320, 136, 16, 128),    # 256-wide tiles, V % 256 = 128, R fills the free half exactly
    (300, 5056, 520, 16, 64),      # 128-wide tiles, V % 128 = 64, Hd % 64 != 0
    (64, 4160, 256, 4, 48),        # 128-wide tiles, V % 128 = 64, R < the free columns
])
def test_fused_shapes(B, T, V, Hd, k, R):
    rng = np.random.default_rng(T + V + R)
    bf = lambda shape, sg: WL.to_bf16_bits((rng.standard_normal(shape) * sg).astype(np.float32))
    d = dict(H=bf((T, Hd), 1.0), W=bf((V, Hd), 0.02), Wp=bf((R, Hd), 0.02))
    _fused_vs_plain(B, d, k, 0.5, 30.0, f"shape {T, V, Hd, k, R}")


def test_fused_full_workload_then_edges(B):
    from tests.gpu_common import candidate, dev, dev_bf16
    d = candidate("full")
    Rq, S, k = d["requests"], d["steps"], d["top_k"]
    ids, lg, hp = _fused_vs_plain(B, d, k, d["multiplier"], d["softcap"], "full")
    # edges from the fused projection, on the step's own candidates
    P, Sc = dev_bf16(d["P"]), dev_bf16(d["S"])
    anchor = dev(d["anchor"])
    E = B.candidate_edges_hp(P, Sc, ids.view(Rq, S, k), lg.view(Rq, S, k), hp, anchor).cpu().numpy()
    ids_h, lg_h = ids.cpu().numpy().reshape(Rq, S, k), lg.cpu().numpy().reshape(Rq, S, k)
    ref = O.candidate_edges(d["P"], d["S"], ids_h, lg_h, d["H"], d["Wp"], d["anchor"])
    check_edges(E, ref, lg_h, "full, edges from the fused projection")
    # and the same as the two-kernel path on the same inputs
    E2 = B.candidate_edges(P, Sc, ids.view(Rq, S, k), lg.view(Rq, S, k), dev_bf16(d["H"]), dev_bf16(d["Wp"]),
                           anchor).cpu().numpy()
    assert_close(E, E2, "full, fused vs two-kernel edges")


@pytest.mark.parametrize("Rq,S,k,V,R", [
    (32, 8, 8, 32768, 64),         # mid-like
    (16, 16, 32, 262144, 256),     # large-like: k = 32, rank 256
    (5, 3, 20, 700, 48),           # k in (16, 32], R % 32 != 0
])
def test_edges_hp_shapes(B, Rq, S, k, V, R):
    from tests.gpu_common import dev, dev_bf16
    rng = np.random.default_rng(Rq * 100 + R)
    bf = lambda shape, sg: WL.to_bf16_bits((rng.standard_normal(shape) * sg).astype(np.float32))
    P, Sc = bf((V, R), 0.5), bf((V, R), 0.5)
    ids = np.stack([rng.choice(V, k, replace=False) for _ in range(Rq * S)]).reshape(Rq, S, k).astype(np.int32)
    U = rng.standard_normal((Rq, S, k)).astype(np.float32)
    anchor = rng.integers(0, V, Rq).astype(np.int32)
    hp = rng.standard_normal((Rq * S, R)).astype(np.float32)
    E = B.candidate_edges_hp(dev_bf16(P), dev_bf16(Sc), dev(ids), dev(U), dev(hp), dev(anchor)).cpu().numpy()
    ref = O.candidate_edges_from_hp(P, Sc, ids, U, hp, anchor)
    check_edges(E, ref, U, f"edges from hp {Rq, S, k, V, R}")
