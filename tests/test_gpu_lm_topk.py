"""GPU parity of dflash_lm_topk against the oracle (compute_candidates of the
DFlash2 drafter: LM head, output multiplier, soft cap, per-position top-k)."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import check_topk_rows, check_topk_summaries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _run(B, H, W, k, s, c):
    from tests.gpu_common import dev_bf16
    ids, vals = B.lm_topk(dev_bf16(H), dev_bf16(W), k, s, c)
    return ids.cpu().numpy(), vals.cpu().numpy()


def _check(B, H, W, k, s, c, rows=None, label=""):
    from tests.gpu_common import say
    gids, gvals = _run(B, H, W, k, s, c)
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    keys = O.lm_logit_keys(H, W, s, c, rows=rows)
    exact, near = check_topk_rows(gids[rows], gvals[rows], keys, k, label=label)
    say(f"[lm_topk {label}] rows={len(rows)} exact={exact} near={near}")
    return gids, gvals


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_small_workloads_all_rows(B, name):
    d = WL.candidate_inputs(name)
    _check(B, d["H"], d["W"], d["top_k"], d["multiplier"], d["softcap"], label=name)


def _random_case(seed, T, V, Hd, sigma_w):
    rng = np.random.default_rng(seed)
    H = WL.to_bf16_bits(rng.standard_normal((T, Hd), dtype=np.float32))
    W = WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32) * np.float32(sigma_w))
    return H, W


@pytest.mark.parametrize("T,V,Hd,k,s,c", [
    (300, 5000, 200, 7, 0.75, 5.0),     # ragged in every dimension, cap well inside tanh's bend
    (1, 777, 8, 1, 1.0, 0.0),           # one row, k = 1, a single K chunk
    (37, 4099, 72, 64, 2.0, 30.0),      # k = 64, V just past a tile
    (513, 20000, 136, 16, 0.5, 30.0),   # three row tiles, two partial
    # 256-row tiles with 64-entry lists (k in (32, 64])
    (2048, 8320, 72, 64, 0.75, 20.0),   # 8 row tiles x 32 groups of 256-column tiles, a K tail
    (1024, 16640, 128, 48, 1.0, 30.0),  # 4 row tiles x 64 groups of 256-column tiles
    (100, 9000, 256, 48, 1.0, 30.0),    # one row tile of 128-column tiles (nontemporal W, rotated K order)
    (300, 20000, 200, 40, 0.5, 0.0),    # two row tiles of 128-column tiles, no cap
])
def test_ragged_shapes(B, T, V, Hd, k, s, c):
    H, W = _random_case(T * 7 + V, T, V, Hd, 0.2)
    _check(B, H, W, k, s, c, label=f"T{T} V{V} Hd{Hd} k{k}")


def test_one_hot_exact_at_full_vocab(B):
    """One-hot hidden states make every logit an LM-head weight exactly on both
    sides, so all ids must match the oracle bit for bit."""
    d = WL.candidate_inputs("full", requests=4)
    W = d["W"]
    T, Hd = 64, W.shape[1]
    rng = np.random.default_rng(9)
    H = np.zeros((T, Hd), np.uint16)
    H[np.arange(T), rng.integers(0, Hd, T)] = 0x3F80
    k = d["top_k"]
    gids, gvals = _run(B, H, W, k, 1.0, 0.0)
    keys = O.lm_logit_keys(H, W, 1.0, 0.0)
    rids, rvals = O.topk_from_keys(keys, k)
    assert np.array_equal(gids, rids)
    assert np.array_equal(gvals, rvals)
    # a power-of-two multiplier keeps the logits exact as well
    gids, gvals = _run(B, H, W, k, 0.5, 0.0)
    rids, rvals = O.topk_from_keys(O.lm_logit_keys(H, W, 0.5, 0.0), k)
    assert np.array_equal(gids, rids) and np.array_equal(gvals, rvals)


def _golden_all_rows(B, d, name):
    """Every golden row of workload ``name`` (tests/golden/topk_<name>.npz,
    written from the oracle by make_topk_goldens.py) against the GPU's top-k of
    the whole workload, in the launch configuration the benchmark times."""
    from tests.gpu_common import say
    from tests.golden.make_topk_goldens import input_digest, load
    rows, summ, k, V, digest = load(name)
    assert input_digest(d) == digest, f"{name}: the seeded inputs are not the bits the goldens were made from"
    assert k == d["top_k"] and V == d["vocab"]
    gids, gvals = _run(B, d["H"], d["W"], k, d["multiplier"], d["softcap"])
    exact, near = check_topk_summaries(gids[rows], gvals[rows], summ, k, V, label=name)
    say(f"[lm_topk {name} golden] rows={len(rows)} exact={exact} near={near}")
    return gids, gvals


def test_full_workload_all_rows(B):
    """All 4096 rows of the 256 x 16 workload against the oracle's goldens."""
    from tests.gpu_common import candidate
    d = candidate("full")
    gids, gvals = _golden_all_rows(B, d, "full")
    # deterministic: a second call gives the same bits
    gids2, gvals2 = _run(B, d["H"], d["W"], d["top_k"], d["multiplier"], d["softcap"])
    assert np.array_equal(gids, gids2) and np.array_equal(gvals.view(np.uint32), gvals2.view(np.uint32))


def test_large_vocab_tie_heavy_golden_requests(B):
    """The large configuration at its full 8192 rows (the launch the benchmark
    times): 32 row tiles, k = 32, a tie-heavy LM head; 32 whole requests, one in
    every 256-row tile, against the oracle's goldens."""
    _golden_all_rows(B, WL.candidate_inputs("large"), "large")


@pytest.fixture(scope="module")
def full_inputs():
    from tests.gpu_common import candidate
    return candidate("full")


def _full_rows_vs_golden(B, d, r0, T, label):
    """Rows r0 .. r0 + T - 1 of the full workload as a launch of their own,
    every row against the oracle's goldens."""
    from tests.gpu_common import say
    from tests.golden.make_topk_goldens import load
    rows, summ, k, V, _ = load("full")
    assert np.array_equal(rows, np.arange(len(rows)))
    H = np.ascontiguousarray(d["H"][r0:r0 + T])
    gids, gvals = _run(B, H, d["W"], k, d["multiplier"], d["softcap"])
    exact, near = check_topk_summaries(gids, gvals, summ[r0:r0 + T], k, V, label=label)
    say(f"[lm_topk {label}] rows={T} exact={exact} near={near}")


@pytest.mark.parametrize("T", [16, 33, 64])
def test_skinny_rows_full_vocab(B, full_inputs, T):
    """Up to 16 rows the head streams W (the bandwidth regime), up to 64 it runs
    64-row tiles: every row of the full vocabulary's product against the
    oracle's goldens, 16 / 33 (a ragged tile) / 64."""
    _full_rows_vs_golden(B, full_inputs, (T * 37) % 1000, T, f"skinny T{T}")


@pytest.mark.parametrize("T,V,Hd,k,s,c", [
    # up to 32 rows (k <= 16 above 16 rows) with Hd / 256 a power of two up to 16:
    # the streaming kernel, each wave reading Hd / 256 KB of every tile
    (1, 777, 256, 1, 1.0, 0.0),        # one row, 1 load per wave per tile, a ragged last tile
    (5, 4099, 512, 8, 0.75, 20.0),     # 2 loads
    (16, 70001, 1024, 32, 1.0, 30.0),  # 4 loads, k = 32, 256 groups: the two-stage merge
    (16, 20000, 2048, 64, 0.5, 30.0),  # 8 loads, k = 64
    (13, 1000, 4096, 16, 2.0, 5.0),    # 16 loads, fewer tiles than CUs
    (24, 9000, 4096, 16, 0.75, 20.0),  # 17-32 rows: two 16-row blocks of hidden rows
    (32, 70001, 1024, 8, 1.0, 30.0),   # 32 rows, 4 loads
    (17, 3000, 512, 16, 0.75, 5.0),    # one row in the second hidden block
    (3, 5, 256, 4, 1.0, 0.0),          # a vocabulary smaller than one tile
    (2, 291, 256, 16, 1.0, 30.0),      # 19 groups: the ranking merge with a 3-entry last list
    (20, 5000, 2048, 32, 0.5, 30.0),   # 17-32 rows with k > 16: the 64-row tile
    # other hidden sizes take the 64-row tile
    (9, 3000, 1536, 8, 1.0, 30.0),     # Hd / 256 = 6
    (7, 5000, 384, 8, 0.75, 20.0),     # Hd % 256 != 0
])
def test_streaming_rows(B, T, V, Hd, k, s, c):
    H, W = _random_case(T * 31 + V + Hd, T, V, Hd, 0.1)
    gids, gvals = _check(B, H, W, k, s, c, label=f"streaming T{T} V{V} Hd{Hd} k{k}")
    # deterministic: a second call gives the same bits
    gids2, gvals2 = _run(B, H, W, k, s, c)
    assert np.array_equal(gids, gids2) and np.array_equal(gvals.view(np.uint32), gvals2.view(np.uint32))


@pytest.mark.parametrize("T,V,Hd,k", [
    (50, 70001, 1000, 8),    # 64-row tile with a K tail and a ragged vocabulary
    (64, 300, 64, 64),       # fewer columns than groups: one tile per group, k = 64
])
def test_skinny_ragged(B, T, V, Hd, k):
    H, W = _random_case(T + V + Hd, T, V, Hd, 0.1)
    _check(B, H, W, k, 0.75, 20.0, label=f"skinny T{T} V{V} Hd{Hd} k{k}")


@pytest.mark.parametrize("T,V,Hd,k", [
    (200, 40000, 256, 16),  # one row tile, 256 groups of 128 columns: the ranking merge
    (200, 40000, 256, 32),  # the same with k = 32: the two-stage merge of 16-list blocks
    (16, 40000, 256, 8),    # the streaming kernel, 256 groups: the ranking merge
])
def test_exact_ties_many_groups(B, T, V, Hd, k):
    """Integer-valued logits (H and W in {-1, 0, 1}, multiplier 1, no cap): the
    keys are exact on both sides and tie everywhere, so merging more than 16
    groups must order equal keys by id exactly as the oracle does: every row
    is an exactly-equal row."""
    from tests.gpu_common import say
    rng = np.random.default_rng(T * 3 + V + k)
    H = WL.to_bf16_bits(rng.integers(-1, 2, (T, Hd)).astype(np.float32))
    W = WL.to_bf16_bits(rng.integers(-1, 2, (V, Hd)).astype(np.float32))
    gids, gvals = _run(B, H, W, k, 1.0, 0.0)
    keys = O.lm_logit_keys(H, W, 1.0, 0.0)
    exact, near = check_topk_rows(gids, gvals, keys, k, label=f"ties T{T} k{k}")
    say(f"[lm_topk ties T{T} V{V} k{k}] rows={T} exact={exact} near={near}")
    assert exact == T
    # the rows do tie across the cut: at some row, ids outside the list share the k-th key
    rr = np.arange(T)
    kth = keys[rr, gids[:, -1]]
    at_kth = (keys == kth[:, None]).sum(axis=1)
    in_list = (keys[rr[:, None], gids] == kth[:, None]).sum(axis=1)
    assert (at_kth > in_list).any()


def test_256_rows_full_vocab(B, full_inputs):
    """256 rows over the full vocabulary (one row tile, 256 groups of 256
    columns, the ranking merge): the benchmark's bandwidth-regime launch, every
    row against the oracle's goldens."""
    _full_rows_vs_golden(B, full_inputs, 0, 256, "256 rows full vocab")
