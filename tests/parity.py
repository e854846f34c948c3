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


def check_topk_rows(gids, gvals, keys, ref_ids, ref_vals, k, max_near_frac=0.05):
    """Check GPU top-k rows against the oracle's full keys of the same rows.

    keys: oracle bf16 keys [n, V] of the checked rows; ref_ids / ref_vals: the
    oracle's top-k of those rows.  A row whose GPU values equal the oracle's
    keys at the GPU ids and equal the oracle's top-k values is an exactly-equal
    row: its ids must match the oracle's bit for bit, in order.  Any other row
    (an fp32 accumulation-order difference moved a key across a bf16 rounding
    boundary) must still be a valid top-k within tolerance.  Returns
    (exact_rows, near_rows).
    """
    n, V = keys.shape
    exact = near = 0
    for t in range(n):
        ok_vals = O.bf16_to_f64(keys[t])
        gi = np.asarray(gids[t], np.int64)
        gv = np.asarray(gvals[t], np.float64)
        assert np.all((gi >= 0) & (gi < V)), f"row {t}: id out of range"
        assert len(set(gi.tolist())) == k, f"row {t}: repeated ids"
        at = ok_vals[gi]
        assert within_tol(gv, at).all(), f"row {t}: values far from the oracle's logits at the same ids"
        # sorted by (value desc, id asc) on the GPU's own values
        for a in range(k - 1):
            assert gv[a] > gv[a + 1] or (gv[a] == gv[a + 1] and gi[a] < gi[a + 1]), f"row {t}: order"
        rv = np.asarray(ref_vals[t], np.float64)
        if np.array_equal(gv, at) and np.array_equal(gv, rv):
            assert np.array_equal(gi, ref_ids[t]), (
                f"row {t}: exactly-equal logits but ids differ: gpu {gi.tolist()} oracle {list(ref_ids[t])}")
            exact += 1
        else:
            kth = rv[-1]
            assert np.all(at >= kth - (ATOL + RTOL * abs(kth))), f"row {t}: an id far below the k-th logit"
            near += 1
    assert near <= max(2, int(max_near_frac * n)), f"{near} of {n} rows differ from the oracle"
    return exact, near


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
