"""The LM-head top-k goldens (tests/golden/topk_{full,large}.npz) against the
oracle they were written from, and the top-k row checker the GPU tests apply
to them (compute_candidates: top-k ids and their logits; ties by lower id)."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.golden.make_topk_goldens import golden_rows, input_digest, load
from tests.parity import ATOL, RTOL, check_topk_summaries, topk_row_summary


@pytest.mark.parametrize("name", ["full", "large"])
def test_golden_structure(name):
    rows, summ, k, V, _ = load(name)
    assert np.array_equal(rows, golden_rows(name))
    assert k == WL.CONFIGS[name]["top_k"] and V == WL.CONFIGS[name]["vocab"]
    for ids, keys in summ:
        assert len(ids) >= k and len(set(ids.tolist())) == len(ids)
        assert np.all((ids >= 0) & (ids < V))
        # sorted by (key desc, id asc); everything past the k-th within tolerance below it
        for a in range(len(ids) - 1):
            assert keys[a] > keys[a + 1] or (keys[a] == keys[a + 1] and ids[a] < ids[a + 1])
        kth = keys[k - 1]
        assert np.all(keys[k:] >= kth - (ATOL + RTOL * abs(kth)))


@pytest.mark.parametrize("name,nrows", [("full", 3), ("large", 2)])
def test_golden_rows_recomputed(name, nrows):
    """The generator still makes the same bits, and a few rows recomputed from
    the oracle give the stored summaries exactly (the k-th key's neighbourhood
    included)."""
    rows, summ, k, V, digest = load(name)
    d = WL.candidate_inputs(name)
    assert input_digest(d) == digest
    pick = np.linspace(0, len(rows) - 1, nrows).astype(int)
    keys = O.lm_logit_keys(d["H"], d["W"], d["multiplier"], d["softcap"], rows=rows[pick])
    ids, vals = O.topk_from_keys(keys, k)
    for j, i in enumerate(pick):
        sid, sval = topk_row_summary(keys[j], k)
        assert np.array_equal(sid, summ[i][0]) and np.array_equal(sval, summ[i][1])
        assert np.array_equal(ids[j], summ[i][0][:k])


def _summary_case():
    # keys of one row: ids 0..9, a clear top 3 (ids 7, 2, 5), then a near tie at
    # the k-th place (ids 1 and 8 within the tolerance of each other)
    vals = np.array([0.1, 1.50, 3.0, 0.2, 0.3, 2.5, 0.0, 4.0, 1.49, -1.0])
    keys = O.f64_to_bf16(vals)
    return keys, O.bf16_to_f64(keys)


def test_checker_accepts_exact_and_near_rows():
    keys, v = _summary_case()
    k = 4
    summ = [topk_row_summary(keys, k)]
    exact_ids = summ[0][0][:k]
    exact, near = check_topk_summaries([exact_ids], [v[exact_ids]], summ, k, 10)
    assert (exact, near) == (1, 0)
    # swapping the near-tied k-th id is a valid top-k within tolerance
    alt = np.array([7, 2, 5, 8] if exact_ids[3] == 1 else [7, 2, 5, 1])
    exact, near = check_topk_summaries([alt], [v[alt]], summ, k, 10, max_near_frac=1.0)
    assert (exact, near) == (0, 1)


def test_checker_rejects_a_missing_clear_winner():
    keys, v = _summary_case()
    k = 4
    summ = [topk_row_summary(keys, k)]
    # drop id 5 (2.5, far above the k-th) and keep both near-tied ids
    bad = np.array([7, 2, 1, 8]) if v[1] >= v[8] else np.array([7, 2, 8, 1])
    with pytest.raises(AssertionError, match="missing"):
        check_topk_summaries([bad], [v[bad]], summ, k, 10, max_near_frac=1.0)


def test_checker_rejects_an_id_far_below_the_kth():
    keys, v = _summary_case()
    k = 4
    summ = [topk_row_summary(keys, k)]
    bad = np.array([7, 2, 5, 4])  # id 4 (0.3) is far below the k-th (1.49)
    with pytest.raises(AssertionError, match="below the k-th"):
        check_topk_summaries([bad], [v[bad]], summ, k, 10, max_near_frac=1.0)
