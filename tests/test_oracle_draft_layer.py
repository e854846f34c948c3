"""Pins of the oracle's draft-layer projections (DFlash2BeamAttention: the
bias-free ``qkv_proj`` and ``o_proj`` linears) and of the whole attention
sublayer they wrap."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL


def _bf(x):
    return WL.to_bf16_bits(np.asarray(x, np.float32))


def test_linear_integer_sums_round_once_to_bf16():
    # small integers: the exact sums are integers; bf16 keeps 8 significant
    # bits, so 257 rounds to 256 (tie to even), 259 to 260, 255 stays
    X = _bf([[1.0] * 257, [1.0] * 255 + [2.0, 2.0]])
    W = _bf(np.ones((2, 257)))
    W[1, :] = _bf(np.r_[np.ones(255), [2.0, 0.0]])
    Y = O.bf16_to_f64(O.linear(X, W))
    assert Y[0, 0] == 256.0          # 257 -> 256
    assert Y[0, 1] == 256.0          # 255 + 2 = 257 -> 256
    assert Y[1, 0] == 260.0          # 255 + 4 = 259 -> 260
    assert Y[1, 1] == 260.0          # 255 + 4 = 259 -> 260


def test_linear_selector_rows_copy_columns():
    rng = np.random.default_rng(7)
    X = _bf(rng.standard_normal((6, 40)))
    cols = rng.integers(0, 40, 24)
    W = np.zeros((24, 40), np.float32)
    W[np.arange(24), cols] = 1.0
    assert np.array_equal(O.linear(X, _bf(W)), X[:, cols])


def test_linear_brute_force():
    rng = np.random.default_rng(8)
    X, W = _bf(rng.standard_normal((3, 9))), _bf(rng.standard_normal((4, 9)) * 0.3)
    Y = O.bf16_to_f64(O.linear(X, W))
    Xf, Wf = O.bf16_to_f64(X), O.bf16_to_f64(W)
    for m in range(3):
        for n in range(4):
            assert Y[m, n] == pytest.approx(sum(Xf[m, k] * Wf[n, k] for k in range(9)), rel=2 ** -8)


def test_draft_attention_with_identity_projections_is_the_attention_path():
    # hidden size = (Hq + 2 Hkv) D and W_qkv = I: qkv is the hidden row; with
    # W_o = I (Hq D columns) the sublayer's output is the attention output
    a = WL.attention_inputs("attn", requests=2)
    Hq, Hkv, D = 4, 2, 128
    Lq = a["query_len"]
    rng = np.random.default_rng(9)
    T = 2 * Lq
    hid = (Hq + 2 * Hkv) * D
    hidden = _bf(rng.standard_normal((T, hid)))
    cache = a["cache"][:, :Hkv]
    Wqkv = _bf(np.eye(hid))
    Wo = _bf(np.eye(Hq * D))
    out, c2 = O.draft_attention(hidden, Wqkv, Wo, Hq, Hkv, D, a["q_w"], a["k_w"], a["eps"], a["positions"],
                                a["theta"], a["slots"], cache, a["block_tables"], a["seq_lens"], Lq,
                                a["block_size"], a["window"])
    q, _, c_ref = O.qk_norm_rope_cache(hidden, Hq, Hkv, D, a["q_w"], a["k_w"], a["eps"], a["positions"], a["theta"],
                                       a["slots"], cache, a["block_size"])
    o = O.block_attn(q, c_ref, a["block_tables"], a["seq_lens"], Lq, Hq, Hkv, D, a["block_size"], a["window"],
                     D ** -0.5)
    assert np.array_equal(c2, c_ref)
    assert np.array_equal(out, np.asarray(o).reshape(T, Hq * D))
