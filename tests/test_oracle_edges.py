"""Pins of the oracle's candidate-selector edge scores
(``DFlash2BeamCandidateSelector``: score = candidate's own logit +
<predecessor[q] * h_p, successor[c]>, h_p = the hidden state projected to the
codebook rank, the first position's predecessor = the anchor token; output
``[requests, steps, top_k (predecessor), top_k]``).
"""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL


def _case(Rq=2, St=4, k=4, V=64, Hd=32, R=8, seed=0, sigma=0.5):
    rng = np.random.default_rng(seed)
    bf = lambda shape, s=1.0: WL.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))
    d = dict(P=bf((V, R), sigma), S=bf((V, R), sigma), H=bf((Rq * St, Hd)),
             Wp=bf((R, Hd), sigma),
             ids=np.stack([np.stack([rng.choice(V, k, replace=False) for _ in range(St)])
                           for _ in range(Rq)]).astype(np.int32),
             U=rng.standard_normal((Rq, St, k)).astype(np.float32),
             anchor=rng.integers(0, V, Rq).astype(np.int32))
    return d


def _E(d, **over):
    x = dict(d, **over)
    return O.candidate_edges(x["P"], x["S"], x["ids"], x["U"], x["H"], x["Wp"], x["anchor"])


def test_zero_codebooks_give_unary_broadcast():
    d = _case()
    z = np.zeros_like(d["P"])
    E = _E(d, P=z)
    assert np.array_equal(E, np.broadcast_to(d["U"][:, :, None, :], E.shape))
    E = _E(d, S=z)
    assert np.array_equal(E, np.broadcast_to(d["U"][:, :, None, :], E.shape))


def test_anchor_is_first_predecessor_and_replicated():
    d = _case(seed=1)
    E = _E(d)
    # identical across q at p = 0 (bit-exact)
    assert np.all(E[:, 0, :, :] == E[:, 0, :1, :])
    # changing ids at the last step must not touch step 0..St-1 predecessors of p=0
    ids2 = d["ids"].copy()
    ids2[:, -1, :] = (ids2[:, -1, :] + 1) % d["P"].shape[0]
    E2 = _E(d, ids=ids2)
    assert np.array_equal(E2[:, 0], E[:, 0])
    # changing the anchor changes only p = 0
    E3 = _E(d, anchor=(d["anchor"] + 7) % d["P"].shape[0])
    assert np.array_equal(E3[:, 1:], E[:, 1:]) and not np.array_equal(E3[:, 0], E[:, 0])


def test_identity_codebooks_closed_form():
    """R = V and P = S = I: the bilinear term is h_p[pred_q] when pred_q equals
    the candidate id c, else 0 -- which fixes which id is the predecessor and
    which the candidate, and the one-step shift."""
    V = R = 16
    Rq, St, k, Hd = 2, 3, 4, 8
    rng = np.random.default_rng(2)
    eye = WL.to_bf16_bits(np.eye(V, dtype=np.float32))
    H = WL.to_bf16_bits(rng.standard_normal((Rq * St, Hd)).astype(np.float32))
    Wp = WL.to_bf16_bits(rng.standard_normal((R, Hd)).astype(np.float32))
    # ids chosen so that some candidates equal some predecessors
    ids = np.array([[[1, 2, 3, 4], [3, 1, 5, 6], [6, 7, 3, 0]],
                    [[9, 8, 7, 6], [8, 9, 10, 11], [12, 11, 9, 8]]], dtype=np.int32)
    anchor = np.array([2, 7], dtype=np.int32)
    U = np.zeros((Rq, St, k), dtype=np.float32)
    E = O.candidate_edges(eye, eye, ids, U, H, Wp, anchor).astype(np.float64)
    hf = O.bf16_to_f64(H).reshape(Rq, St, Hd)
    wf = O.bf16_to_f64(Wp)
    for r in range(Rq):
        for p in range(St):
            hp = [sum(wf[i, j] * hf[r, p, j] for j in range(Hd)) for i in range(R)]
            for q in range(k):
                pred = int(anchor[r]) if p == 0 else int(ids[r, p - 1, q])
                for c in range(k):
                    want = hp[pred] if pred == int(ids[r, p, c]) else 0.0
                    assert E[r, p, q, c] == pytest.approx(want, rel=1e-6, abs=1e-6)
    # some nonzero entries exist (the pin is not vacuous)
    assert np.count_nonzero(E) >= 4


def test_bilinear_in_codebooks_linear_in_h():
    d = _case(seed=3, V=32, R=8)
    U = d["U"]
    base = lambda **o: _E(d, **o).astype(np.float64) - U[:, :, None, :]
    rng = np.random.default_rng(4)
    tol = 1e-5 * np.abs(base()).max() + 1e-6
    S2 = WL.to_bf16_bits(rng.standard_normal(d["S"].shape).astype(np.float32))
    combS = WL.to_bf16_bits((O.bf16_to_f64(d["S"]) + O.bf16_to_f64(S2)).astype(np.float32))
    if np.array_equal(O.bf16_to_f64(combS), O.bf16_to_f64(d["S"]) + O.bf16_to_f64(S2)):
        assert np.max(np.abs(base(S=combS) - base() - base(S=S2))) <= tol
    # linear in h: doubling h doubles the residual exactly (power of two)
    H2 = WL.to_bf16_bits((2.0 * O.bf16_to_f64(d["H"])).astype(np.float32))
    assert np.max(np.abs(base(H=H2) - 2.0 * base())) <= tol


def test_bilinearity_with_exact_sums():
    """Codebooks on a coarse grid so that P1 + P2 is exact in bf16."""
    rng = np.random.default_rng(5)
    d = _case(seed=6, V=32, R=8)
    grid = lambda: WL.to_bf16_bits((rng.integers(-8, 9, d["P"].shape) / 8).astype(np.float32))
    P1, P2 = grid(), grid()
    Ps = WL.to_bf16_bits((O.bf16_to_f64(P1) + O.bf16_to_f64(P2)).astype(np.float32))
    assert np.array_equal(O.bf16_to_f64(Ps), O.bf16_to_f64(P1) + O.bf16_to_f64(P2))
    U = d["U"][:, :, None, :]
    r = lambda P: _E(d, P=P).astype(np.float64) - U
    lhs, rhs = r(Ps), r(P1) + r(P2)
    assert np.max(np.abs(lhs - rhs)) <= 1e-5 * np.abs(rhs).max() + 1e-6


def test_rank_one_scalar():
    """R = k = 1: E = u + P[pred] * (Wp . h) * S[id]."""
    rng = np.random.default_rng(7)
    V, Hd = 10, 6
    P = WL.to_bf16_bits(rng.standard_normal((V, 1)).astype(np.float32))
    S = WL.to_bf16_bits(rng.standard_normal((V, 1)).astype(np.float32))
    Wp = WL.to_bf16_bits(rng.standard_normal((1, Hd)).astype(np.float32))
    H = WL.to_bf16_bits(rng.standard_normal((3, Hd)).astype(np.float32))
    ids = np.array([[[4], [7], [1]]], dtype=np.int32)
    U = np.array([[[0.5], [-1.0], [2.0]]], dtype=np.float32)
    anchor = np.array([9], dtype=np.int32)
    E = O.candidate_edges(P, S, ids, U, H, Wp, anchor)
    pf, sf = O.bf16_to_f64(P)[:, 0], O.bf16_to_f64(S)[:, 0]
    hp = O.bf16_to_f64(H) @ O.bf16_to_f64(Wp)[0]
    preds = [9, 4, 7]
    for p in range(3):
        want = float(U[0, p, 0]) + pf[preds[p]] * hp[p] * sf[ids[0, p, 0]]
        assert float(E[0, p, 0, 0]) == pytest.approx(want, rel=1e-6)


def test_brute_force_loops_tiny_workload():
    d = WL.candidate_inputs("tiny")
    E = _E(d).astype(np.float64)
    Pf, Sf = O.bf16_to_f64(d["P"]), O.bf16_to_f64(d["S"])
    Hf, Wf = O.bf16_to_f64(d["H"]), O.bf16_to_f64(d["Wp"])
    Rq, St, k = d["ids"].shape
    R, Hd = Wf.shape
    for r in range(Rq):
        for p in range(St):
            t = r * St + p
            hp = [sum(Wf[i, j] * Hf[t, j] for j in range(Hd)) for i in range(R)]
            for q in range(k):
                pred = d["anchor"][r] if p == 0 else d["ids"][r, p - 1, q]
                for c in range(k):
                    cid = d["ids"][r, p, c]
                    acc = float(d["U"][r, p, c])
                    bil = sum(Pf[pred, i] * hp[i] * Sf[cid, i] for i in range(R))
                    assert E[r, p, q, c] == pytest.approx(acc + bil, rel=1e-6, abs=1e-7)


def test_rank_projection_selects_hidden_columns():
    # W_proj rows that are unit vectors pick columns of H exactly (a closed form
    # that a transposed operand or a dropped term would break)
    rng = np.random.default_rng(5)
    T, Hd, R = 6, 40, 8
    H = WL.to_bf16_bits(rng.standard_normal((T, Hd)).astype(np.float32))
    cols = rng.choice(Hd, R, replace=False)
    Wp = np.zeros((R, Hd), dtype=np.float32)
    Wp[np.arange(R), cols] = 1.0
    Wp[3, cols[5]] = 2.0                      # one row sums two columns
    hp = O.rank_projection(H, WL.to_bf16_bits(Wp))
    Hf = O.bf16_to_f64(H)
    want = Hf[:, cols].copy()
    want[:, 3] += 2.0 * Hf[:, cols[5]]
    assert hp.shape == (T, R)
    assert np.array_equal(hp, want)


def test_rank_projection_brute_force():
    d = _case(Rq=1, St=3, Hd=24, R=5, seed=11)
    hp = O.rank_projection(d["H"], d["Wp"])
    Hf, Wf = O.bf16_to_f64(d["H"]), O.bf16_to_f64(d["Wp"])
    for t in range(3):
        for i in range(5):
            assert hp[t, i] == pytest.approx(sum(Wf[i, j] * Hf[t, j] for j in range(24)), rel=1e-12)


def test_edges_from_hp_matches_edges_and_brute_force():
    d = _case(Rq=2, St=3, k=3, V=40, Hd=16, R=8, seed=12)
    hp = O.rank_projection(d["H"], d["Wp"])
    E = O.candidate_edges_from_hp(d["P"], d["S"], d["ids"], d["U"], hp, d["anchor"])
    assert np.array_equal(E, _E(d))
    # a given hp that no H could give: the brute-force bilinear form on it
    rng = np.random.default_rng(13)
    hq = rng.standard_normal(hp.shape)
    E2 = O.candidate_edges_from_hp(d["P"], d["S"], d["ids"], d["U"], hq, d["anchor"]).astype(np.float64)
    Pf, Sf = O.bf16_to_f64(d["P"]), O.bf16_to_f64(d["S"])
    for r in range(2):
        for p in range(3):
            for q in range(3):
                pred = d["anchor"][r] if p == 0 else d["ids"][r, p - 1, q]
                for c in range(3):
                    want = float(d["U"][r, p, c]) + sum(Pf[pred, i] * hq[r * 3 + p, i] * Sf[d["ids"][r, p, c], i]
                                                        for i in range(8))
                    assert E2[r, p, q, c] == pytest.approx(want, rel=1e-6, abs=1e-7)
