"""Pins of the oracle's LM-head top-k (``compute_candidates`` of the DFlash2
drafter, vLLM ``DFlash2BeamForCausalLM``; logits processor with
``scale=output_multiplier`` and ``soft_cap=final_logit_softcapping``).

Each pin ties the oracle to something other than itself: exact one-hot
products, an independent heap selection, a hand-worked tie example
(tests/golden), the Taylor series of the cap, brute-force dot products.
"""
import heapq
import json
import math
import os

import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_of(values):
    return O.f64_to_bf16(np.asarray(values, dtype=np.float64))


def test_bf16_rounding_known_patterns():
    # fp32 bit patterns -> expected bf16 (round to nearest, ties to even)
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F808000: 0x3F80,  # halfway, lower is even -> down
        0x3F818000: 0x3F82,  # halfway, lower is odd -> up
        0x3F808001: 0x3F81,  # just above halfway -> up
        0x3F807FFF: 0x3F80,  # just below halfway -> down
        0xBF818000: 0xBF82,  # negative, halfway odd -> away (magnitude up)
        0x7F7FFFFF: 0x7F80,  # max finite fp32 rounds to +inf in bf16
        0x00000000: 0x0000,
        0x80000000: 0x8000,
    }
    u = np.array(list(cases), dtype=np.uint32)
    got = O.f32_to_bf16(u.view(np.float32))
    assert [int(x) for x in got] == list(cases.values())
    nan = O.f32_to_bf16(np.array([0x7FC00001], dtype=np.uint32).view(np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0
    # widening is exact
    b = np.arange(0, 0x7F80, 97, dtype=np.uint16)
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(b)), b)


def _one_hot_rows(T, Hd, cols):
    H = np.zeros((T, Hd), dtype=np.uint16)
    H[np.arange(T), cols] = 0x3F80  # bf16 1.0
    return H


def test_one_hot_logits_are_lm_head_columns():
    """H[t] = e_j makes every logit a weight W[v, j] exactly (s = 1, no cap)."""
    rng = np.random.default_rng(0)
    V, Hd, T = 4096, 64, 6
    W = WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32))
    cols = rng.integers(0, Hd, T)
    keys = O.lm_logit_keys(_one_hot_rows(T, Hd, cols), W, 1.0, 0.0)
    expect = W[:, cols].T
    # -0 and +0 are one value; compare values
    assert np.array_equal(O.bf16_to_f64(keys), O.bf16_to_f64(expect))


def test_multiplier_power_of_two_is_exact():
    rng = np.random.default_rng(1)
    V, Hd = 512, 32
    W = WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32))
    H = _one_hot_rows(3, Hd, [0, 5, 31])
    keys = O.lm_logit_keys(H, W, 0.25, 0.0)
    assert np.array_equal(O.bf16_to_f64(keys), 0.25 * O.bf16_to_f64(W[:, [0, 5, 31]].T))


def _heap_topk(vals, k):
    """Independent selection: heapq over (value, -id)."""
    best = heapq.nlargest(k, ((float(v), -i) for i, v in enumerate(vals)))
    return [-i for _, i in best], [v for v, _ in best]


def test_topk_matches_heap_selection_on_tie_heavy_keys():
    rng = np.random.default_rng(2)
    T, V, k = 16, 3000, 32
    # keys from a set of 11 values: many ties at and across the k-th place
    levels = _bits_of(np.linspace(-1, 4, 11))
    keys = levels[rng.integers(0, 11, (T, V))]
    keys[0, :] = levels[3]  # a row where everything ties
    ids, vals = O.topk_from_keys(keys, k)
    for t in range(T):
        hid, hval = _heap_topk(O.bf16_to_f64(keys[t]), k)
        assert list(ids[t]) == hid
        assert np.array_equal(vals[t], np.asarray(hval, dtype=np.float32))
    assert list(ids[0]) == list(range(k))


def test_signed_zero_ties_by_id():
    keys = np.array([[0x8000, 0x0000, 0x8000, 0xBF80]], dtype=np.uint16)  # -0, +0, -0, -1
    ids, vals = O.topk_from_keys(keys, 3)
    assert list(ids[0]) == [0, 1, 2]


def test_golden_tie_example():
    with open(os.path.join(GOLDEN, "topk_ties.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        keys = _bits_of(case["logits"])[None, :]
        ids, vals = O.topk_from_keys(keys, case["k"])
        assert list(ids[0]) == case["ids"], case
        assert list(vals[0].astype(float)) == case["values"], case


def test_softcap_series_and_order():
    """One-hot rows make the raw logit a chosen weight w.  With multiplier s and
    cap c the key is bf16(c tanh(s w / c)): checked against the Taylor series
    x - x^3/(3c^2) + 2x^5/(15c^4) (x = s w, |x/c| <= 0.15, remainder < 1e-8),
    which the other order, s c tanh(w / c), misses by far more than a bf16 ulp."""
    ws = np.array([8.0, -8.0, 4.5, 2.0, -0.75, 0.125, 0.0], dtype=np.float32)
    Hd = len(ws)
    W = WL.to_bf16_bits(np.diag(ws))           # W[v, v] = ws[v]
    H = _one_hot_rows(Hd, Hd, np.arange(Hd))   # logit[t, t] = ws[t]
    s, c = 0.5, 30.0
    keys = O.lm_logit_keys(H, W, s, c)
    got = O.bf16_to_f64(np.diag(keys))
    x = s * ws.astype(np.float64)
    series = x - x**3 / (3 * c * c) + 2 * x**5 / (15 * c**4)
    assert np.array_equal(got, O.bf16_to_f64(_bits_of(series)))
    other = s * c * np.tanh(ws.astype(np.float64) / c)
    assert not np.array_equal(O.bf16_to_f64(_bits_of(other)), got)
    # odd, monotone, bounded by the cap
    xs = np.linspace(-200, 200, 801)
    W2 = WL.to_bf16_bits(xs.astype(np.float32)[:, None])
    H2 = np.full((1, 1), 0x3F80, dtype=np.uint16)
    v = O.bf16_to_f64(O.lm_logit_keys(H2, W2, 1.0, c))[0]
    assert np.all(np.diff(v) >= 0) and np.all(np.abs(v) <= c)
    assert np.array_equal(v, -v[::-1])


def test_no_cap_when_softcap_nonpositive():
    rng = np.random.default_rng(3)
    W = WL.to_bf16_bits(rng.standard_normal((64, 8), dtype=np.float32) * 20)
    H = _one_hot_rows(8, 8, np.arange(8))
    for c in (0.0, -1.0):
        keys = O.lm_logit_keys(H, W, 1.0, c)
        assert np.array_equal(O.bf16_to_f64(keys), O.bf16_to_f64(W.T))


def test_brute_force_dot_products():
    """Python-loop dot products (float64, sequential) give the same keys."""
    rng = np.random.default_rng(4)
    T, V, Hd = 3, 40, 24
    H = WL.to_bf16_bits(rng.standard_normal((T, Hd), dtype=np.float32))
    W = WL.to_bf16_bits(rng.standard_normal((V, Hd), dtype=np.float32) * 0.1)
    s, c = 0.75, 2.0
    keys = O.lm_logit_keys(H, W, s, c)
    hf = [[float(np.frombuffer(np.uint32(int(b) << 16).tobytes(), np.float32)[0]) for b in row] for row in H]
    wf = [[float(np.frombuffer(np.uint32(int(b) << 16).tobytes(), np.float32)[0]) for b in row] for row in W]
    for t in range(T):
        for v in range(V):
            acc = 0.0
            for j in range(Hd):
                acc += hf[t][j] * wf[v][j]
            x = c * math.tanh(s * acc / c)
            assert keys[t, v] == _bits_of([x])[0]


def test_rows_subset_equals_full():
    d = WL.candidate_inputs("tiny")
    k = d["top_k"]
    ids, vals = O.lm_topk(d["H"], d["W"], k, d["multiplier"], d["softcap"])
    ids2, vals2 = O.lm_topk(d["H"], d["W"], k, d["multiplier"], d["softcap"], rows=[5, 1])
    assert np.array_equal(ids[[5, 1]], ids2) and np.array_equal(vals[[5, 1]], vals2)
    # sorted by (value desc, id asc) and distinct
    for t in range(ids.shape[0]):
        assert len(set(ids[t])) == k
        for a in range(k - 1):
            assert vals[t, a] > vals[t, a + 1] or (vals[t, a] == vals[t, a + 1] and ids[t, a] < ids[t, a + 1])
