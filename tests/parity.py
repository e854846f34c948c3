"""Acceptance rules shared by the GPU parity tests (HIP path vs the oracle).

Values (logits, edges, q/k outputs, attention): |gpu - ref| <= 1e-2 + 1e-2 |ref|
elementwise (bf16 inputs, fp32 accumulation).  Integer results (ids, written
cache slots, V payloads) are compared bit for bit, ids under the rule that the
logits they rank are exactly equal on both sides.
"""
from __future__ import annotations

import numpy as np

from oracle import dflash_oracle as O

ATOL = 1e-2
RTOL = 1e-2


def within_tol(got, ref, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(got - ref) <= atol + rtol * np.abs(ref)


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    ok = within_tol(got, ref, atol, rtol)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        g = np.asarray(got, np.float64)
        r = np.asarray(ref, np.float64)
        detail = ", ".join(f"{tuple(i)}: gpu={g[tuple(i)]:.6g} ref={r[tuple(i)]:.6g}" for i in idx)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; {detail}")


def topk_row_summary(key_row, k, atol=ATOL, rtol=RTOL):
    """The oracle's ranking of one row near its k-th place: every id whose key is
    at least the k-th key minus the tolerance, sorted by (key desc, id asc), and
    their keys (float64).  The first k entries are the oracle's top-k.

    key_row: the oracle's bf16 keys of the row (uint16 bits, all V of them).
    """
    vals = O.bf16_to_f64(key_row)
    kth = -np.partition(-vals, k - 1)[k - 1]
    near = np.nonzero(vals >= kth - (atol + rtol * abs(kth)))[0]
    order = np.lexsort((near, -vals[near]))
    return near[order].astype(np.int64), vals[near[order]]


def check_topk_summaries(gids, gvals, summaries, k, V, max_near_frac=0.05, label=""):
    """Check GPU top-k rows against the oracle's row summaries (``topk_row_summary``).

    A row whose GPU values equal the oracle's keys at the GPU ids and equal the
    oracle's top-k values is an exactly-equal row: its ids must match the
    oracle's bit for bit, in order.  Any other row (an fp32 accumulation-order
    difference moved a key across a bf16 rounding boundary) must still be a valid
    top-k within tolerance: every GPU id's oracle key is at least the k-th key
    minus the tolerance (so it is in the summary), its value is within tolerance
    of that key, and every id whose oracle key beats the k-th by more than the
    tolerance is in the GPU list.  Returns (exact_rows, near_rows).
    """
    exact = near = 0
    for t, (sid, sval) in enumerate(summaries):
        gi = np.asarray(gids[t], np.int64)
        gv = np.asarray(gvals[t], np.float64)
        assert np.all((gi >= 0) & (gi < V)), f"{label} row {t}: id out of range"
        assert len(set(gi.tolist())) == k, f"{label} row {t}: repeated ids"
        # sorted by (value desc, id asc) on the GPU's own values
        for a in range(k - 1):
            assert gv[a] > gv[a + 1] or (gv[a] == gv[a + 1] and gi[a] < gi[a + 1]), f"{label} row {t}: order"
        pos = {int(i): j for j, i in enumerate(sid)}
        missing = [int(i) for i in gi if int(i) not in pos]
        assert not missing, f"{label} row {t}: ids {missing[:5]} lie below the k-th logit by more than the tolerance"
        at = sval[[pos[int(i)] for i in gi]]
        assert within_tol(gv, at).all(), f"{label} row {t}: values far from the oracle's logits at the same ids"
        rv = sval[:k]
        if np.array_equal(gv, at) and np.array_equal(gv, rv):
            assert np.array_equal(gi, sid[:k]), (
                f"{label} row {t}: exactly-equal logits but ids differ: gpu {gi.tolist()} oracle {sid[:k].tolist()}")
            exact += 1
        else:
            kth = rv[-1]
            must = sid[sval > kth + (ATOL + RTOL * abs(kth))]
            lost = np.setdiff1d(must, gi)
            assert lost.size == 0, (
                f"{label} row {t}: ids {lost[:5].tolist()} beat the k-th logit by more than the tolerance "
                "but are missing")
            near += 1
    n = len(summaries)
    assert near <= max(2, int(max_near_frac * n)), f"{label}: {near} of {n} rows differ from the oracle"
    return exact, near


def check_topk_rows(gids, gvals, keys, k, max_near_frac=0.05, label=""):
    """``check_topk_summaries`` with the summaries taken from the oracle's full
    keys ``[n, V]`` of the checked rows."""
    summaries = [topk_row_summary(keys[t], k) for t in range(keys.shape[0])]
    return check_topk_summaries(gids, gvals, summaries, k, keys.shape[1], max_near_frac, label)


def bf16_ulp(x):
    """Spacing of the bf16 numbers at |x|: 2^(e - 7) for |x| in [2^e, 2^(e+1)),
    and the subnormal spacing 2^-133 below 2^-126."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


# The attention kernel's fp32 output before its one bf16 rounding differs from
# the exact softmax average by far less than this: each weight is carried as two
# bf16 parts (2^-16 relative), scores and sums are fp32 (2^-24 per rounding,
# a few hundred roundings per output whose errors do not line up), so the
# expected error is ~1e-6 for these N(0, 1) values; 2^-14 leaves a wide margin
# yet sits below one ulp at the typical output (|o| ~ 0.02: ulp 2^-13).
ATTN_PRE_ROUND = 2.0 ** -14


def check_attention(got, ref, what, pre_round=ATTN_PRE_ROUND):
    """Attention outputs (float64 of the bf16 bits) against the oracle's: the
    value tolerance, and every output within one bf16 ulp of the oracle's plus
    the kernel's pre-rounding error (both sides round once to bf16, so two
    roundings apart they differ by at most one ulp).  Returns (outputs equal,
    outputs one ulp apart or less, total)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    assert_close(g, r, what)
    d = np.abs(g - r)
    bound = bf16_ulp(np.maximum(np.abs(g), np.abs(r))) + pre_round
    bad = d > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: gpu={g[tuple(i)]:.6g} ref={r[tuple(i)]:.6g}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {d.size} outputs more than one bf16 ulp "
                             f"(+{pre_round:.3g}) from the oracle; {detail}")
    return int((d == 0).sum()), int((d <= bf16_ulp(np.maximum(np.abs(g), np.abs(r)))).sum()), d.size


def check_edges(E, ref, U, what="edges"):
    """Values within tolerance, the bilinear residual E - U within 1% of its
    per-(request, step) maximum, and p = 0 rows identical across predecessors."""
    assert_close(E, ref, what)
    Rg = E.astype(np.float64) - U[:, :, None, :]
    Rr = ref.astype(np.float64) - U[:, :, None, :]
    scale = np.abs(Rr).max(axis=(2, 3), keepdims=True)
    bad = np.abs(Rg - Rr) > 1e-2 * scale + 1e-6
    assert not bad.any(), f"{what}: residual mismatch at {np.argwhere(bad)[:3].tolist()}"
    assert np.all(E[:, 0] == E[:, 0, :1]), f"{what}: p = 0 rows differ across predecessors"
