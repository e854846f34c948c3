"""GPU parity of dflash_candidate_edges against the oracle
(DFlash2BeamCandidateSelector edge scores [requests, steps, top_k, top_k])."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import check_edges

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _gpu_edges(B, d):
    from tests.gpu_common import dev, dev_bf16
    E = B.candidate_edges(dev_bf16(d["P"]), dev_bf16(d["S"]), dev(d["ids"]), dev(d["U"]),
                          dev_bf16(d["H"]), dev_bf16(d["Wp"]), dev(d["anchor"]))
    return E.cpu().numpy()


def _ref(d):
    return O.candidate_edges(d["P"], d["S"], d["ids"], d["U"], d["H"], d["Wp"], d["anchor"])


def _amplified(d, seed):
    """Codebooks drawn N(0, 1) so the bilinear term dominates the unary logit."""
    V, R = d["P"].shape
    e = dict(d)
    e["P"] = WL.bf16_normal(seed, 20, (V, R))
    e["S"] = WL.bf16_normal(seed, 21, (V, R))
    return e


@pytest.mark.parametrize("name", ["tiny", "mid", "full"])
def test_workload_all_rows(B, name):
    from tests.gpu_common import candidate, say
    d = candidate(name) if name == "full" else WL.candidate_inputs(name)
    E = _gpu_edges(B, d)
    check_edges(E, _ref(d), d["U"], name)
    a = _amplified(d, 700 + len(name))
    Ea = _gpu_edges(B, a)
    check_edges(Ea, _ref(a), a["U"], name + " amplified")
    say(f"[edges {name}] max|dE|={np.abs(E - _ref(d)).max():.3g}")


def test_large_workload_subset(B):
    d = WL.candidate_inputs("large", requests=96)
    E = _gpu_edges(B, d)
    check_edges(E, _ref(d), d["U"], "large")


def test_large_full_size_all_requests(B):
    """The large configuration at its full 512 x 16 rows, the launch the
    benchmark times (two K slices of the projection, the k = 32 / rank 256
    bilinear tile); the oracle checks every request, 64 at a time."""
    from tests.gpu_common import say
    d = WL.candidate_inputs("large")
    Rq, S = d["requests"], d["steps"]
    E = _gpu_edges(B, d)
    assert E.shape == d["ids"].shape + (d["top_k"],)
    hp = O.rank_projection(d["H"], d["Wp"]).reshape(Rq, S, -1)
    worst = 0.0
    for r0 in range(0, Rq, 64):
        req = np.arange(r0, min(Rq, r0 + 64))
        ref = O.candidate_edges_from_hp(d["P"], d["S"], d["ids"][req], d["U"][req],
                                        hp[req].reshape(len(req) * S, -1), d["anchor"][req])
        check_edges(E[req], ref, d["U"][req], f"large, full size, requests {r0}..{req[-1]}")
        worst = max(worst, float(np.abs(E[req] - ref).max()))
    say(f"[edges large full size] {Rq} requests, max|dE|={worst:.3g}")


@pytest.mark.parametrize("Rq,S,k,V,R,Hd", [
    (3, 5, 3, 100, 16, 24),       # k < 16, R = 16 (4-wide lane chunks), Hd % 64 != 0
    (5, 2, 20, 300, 48, 520),     # k in (16, 32], R % 32 != 0
    (2, 3, 40, 500, 256, 64),     # k in (32, 64], R = 256
    (1, 1, 1, 10, 32, 8),         # one request, one step, k = 1
    (77, 3, 16, 2000, 128, 4104), # ragged row count for the projection tiles
    (32, 16, 16, 5000, 128, 1000),  # 8 row blocks x 4 slices, Hd % 64 != 0
    (20, 7, 11, 3000, 48, 264),     # ragged rows, rank % 32 != 0, a short last slice
    (64, 16, 16, 7000, 80, 512),    # 16 row blocks, rank 80
    (2, 4, 4, 1024, 16, 256),       # rank 16, one row block
])
def test_shapes(B, Rq, S, k, V, R, Hd):
    rng = np.random.default_rng(Rq * 1000 + k)
    bf = lambda shape, s: WL.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))
    d = dict(P=bf((V, R), 0.5), S=bf((V, R), 0.5), H=bf((Rq * S, Hd), 1.0), Wp=bf((R, Hd), 0.1),
             ids=np.stack([rng.choice(V, k, replace=False) for _ in range(Rq * S)]).reshape(Rq, S, k).astype(np.int32),
             U=rng.standard_normal((Rq, S, k)).astype(np.float32),
             anchor=rng.integers(0, V, Rq).astype(np.int32))
    check_edges(_gpu_edges(B, d), _ref(d), d["U"], f"shape {Rq, S, k, V, R, Hd}")


def test_zero_codebooks_give_unary(B):
    d = WL.candidate_inputs("mid")
    d = dict(d, P=np.zeros_like(d["P"]))
    E = _gpu_edges(B, d)
    assert np.array_equal(E, np.broadcast_to(d["U"][:, :, None, :], E.shape))


def test_deterministic(B):
    d = WL.candidate_inputs("mid")
    assert np.array_equal(_gpu_edges(B, d).view(np.uint32), _gpu_edges(B, d).view(np.uint32))

