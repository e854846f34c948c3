"""Pins of the oracle's RoPE options (the fused q/k op and store_context_kv
take head_dim, rotary_dim and is_neox_style, and the cos/sin cache the pages
use is bf16): GPT-J pairing, partial rotary dim, bf16 table."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL

D, THETA, EPS = 128, 1e6, 1e-6


def _one_hot_head(idx, val=2.0, Hq=1, Hkv=1, T=1):
    x = np.zeros((T, (Hq + 2 * Hkv) * D), np.float32)
    x[:, idx] = val
    return WL.to_bf16_bits(x)


def _ones():
    return WL.to_bf16_bits(np.ones(D, np.float32))


@pytest.mark.parametrize("neox", [True, False])
def test_pairing_of_a_one_hot_head(neox):
    # y = e_0 * sqrt(D) (unit-RMS norm of a one-hot vector); rotation by angle
    # index 0 moves it into its pair partner: D/2 for NeoX, 1 for GPT-J
    pos = np.array([5])
    q, _, _ = O.qk_norm_rope_cache(_one_hot_head(0), 1, 1, D, _ones(), _ones(), EPS, pos, THETA, neox=neox)
    y = O.bf16_to_f64(q[0, 0])
    r = np.sqrt(D) / np.sqrt(1 + EPS * D / 4.0)  # val^2 / D mean square, val = 2
    partner = D // 2 if neox else 1
    nz = sorted(np.flatnonzero(y).tolist())
    assert nz == sorted({0, partner})
    assert y[0] == pytest.approx(r * np.cos(5.0), rel=2 ** -7)
    assert y[partner] == pytest.approx(r * np.sin(5.0), rel=2 ** -7)


@pytest.mark.parametrize("neox", [True, False])
def test_partial_rotary_angle_uses_the_rotary_dim(neox):
    # element 2 (GPT-J: angle index 1) or 1 (NeoX: angle index 1) turns by
    # pos * theta^(-2/rot), rot = 32; its partner is 3 (GPT-J) or 1 + 16 (NeoX)
    rot, p = 32, 700
    idx = 1 if neox else 2
    partner = idx + rot // 2 if neox else idx + 1
    q, _, _ = O.qk_norm_rope_cache(_one_hot_head(idx), 1, 1, D, _ones(), _ones(), EPS, np.array([p]), THETA,
                                   rotary_dim=rot, neox=neox)
    y = O.bf16_to_f64(q[0, 0])
    ang = p * THETA ** (-2.0 / rot)
    r = np.sqrt(D) / np.sqrt(1 + EPS * D / 4.0)
    assert sorted(np.flatnonzero(y).tolist()) == sorted([idx, partner])
    assert y[idx] == pytest.approx(r * np.cos(ang), rel=2 ** -7, abs=1e-3)
    assert y[partner] == pytest.approx(r * np.sin(ang), rel=2 ** -7, abs=1e-3)


@pytest.mark.parametrize("neox", [True, False])
def test_partial_rotary_leaves_the_tail_as_normed(neox):
    rng = np.random.default_rng(4)
    T, rot = 6, 64
    x = WL.to_bf16_bits(rng.standard_normal((T, 3 * D)).astype(np.float32))
    w = WL.to_bf16_bits((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    pos = rng.integers(1, 4000, T)
    q, k, _ = O.qk_norm_rope_cache(x, 1, 1, D, w, w, EPS, pos, THETA, rotary_dim=rot, neox=neox)
    q0, k0, _ = O.qk_norm_rope_cache(x, 1, 1, D, w, w, EPS, np.zeros(T, np.int64), THETA, rotary_dim=rot, neox=neox)
    assert np.array_equal(q[..., rot:], q0[..., rot:])
    assert np.array_equal(k[..., rot:], k0[..., rot:])
    assert not np.array_equal(q[..., :rot], q0[..., :rot])
    # position 0 is the identity: the plain norm
    assert np.array_equal(q0[:, 0], O.rms_norm(x[:, :D], w, EPS))


@pytest.mark.parametrize("neox", [True, False])
def test_rotation_preserves_each_pair_norm(neox):
    rng = np.random.default_rng(5)
    T = 8
    x = WL.to_bf16_bits(rng.standard_normal((T, 3 * D)).astype(np.float32))
    pos = rng.integers(0, 8000, T)
    q, _, _ = O.qk_norm_rope_cache(x, 1, 1, D, _ones(), _ones(), EPS, pos, THETA, neox=neox)
    q0, _, _ = O.qk_norm_rope_cache(x, 1, 1, D, _ones(), _ones(), EPS, np.zeros(T, np.int64), THETA, neox=neox)
    a, b = O.bf16_to_f64(q[:, 0]), O.bf16_to_f64(q0[:, 0])
    if neox:
        na, nb = a[:, :D // 2] ** 2 + a[:, D // 2:] ** 2, b[:, :D // 2] ** 2 + b[:, D // 2:] ** 2
    else:
        na, nb = a[:, 0::2] ** 2 + a[:, 1::2] ** 2, b[:, 0::2] ** 2 + b[:, 1::2] ** 2
    assert np.allclose(na, nb, rtol=2 ** -6, atol=1e-4)


def test_bf16_table_values_and_identity_at_zero():
    pos = np.array([0, 1, 77, 8191])
    c, s = O.rope_cos_sin(pos, D, THETA, "bf16")
    cf, sf = O.rope_cos_sin(pos, D, THETA, "f64")
    # every value is a bf16 number within half a bf16 ulp (<= 2^-8 relative) of the exact one
    assert np.array_equal(O.bf16_to_f64(O.f64_to_bf16(c)), c)
    assert np.all(np.abs(c - cf) <= 2 ** -8 * np.abs(cf) + 1e-30)
    assert np.all(np.abs(s - sf) <= 2 ** -8 * np.abs(sf) + 1e-30)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    rng = np.random.default_rng(6)
    x = WL.to_bf16_bits(rng.standard_normal((1, 3 * D)).astype(np.float32))
    a, _, _ = O.qk_norm_rope_cache(x, 1, 1, D, _ones(), _ones(), EPS, np.array([0]), THETA, table="bf16")
    b, _, _ = O.qk_norm_rope_cache(x, 1, 1, D, _ones(), _ones(), EPS, np.array([0]), THETA)
    assert np.array_equal(a, b)


def test_store_context_kv_variants_equal_the_draft_layer_k_path():
    rng = np.random.default_rng(7)
    n, L, Hkv = 5, 2, 2
    kv = WL.to_bf16_bits(rng.standard_normal((n, L, 2, Hkv, D)).astype(np.float32))
    kw = WL.to_bf16_bits((1 + 0.1 * rng.standard_normal((L, D))).astype(np.float32))
    pos = rng.integers(0, 3000, n)
    slots = rng.permutation(64)[:n].astype(np.int64)
    caches = [np.zeros((16, Hkv, 4, 2 * D), np.uint16) for _ in range(L)]
    for opts in (dict(neox=False), dict(rotary_dim=64), dict(rotary_dim=32, neox=False, table="bf16")):
        out = O.store_context_kv(kv, kw, EPS, pos, THETA, slots, caches, 4, **opts)
        for l in range(L):
            qkv = np.concatenate([kv[:, l, 0].reshape(n, -1), kv[:, l, 1].reshape(n, -1)], axis=1)
            _, _, ref = O.qk_norm_rope_cache(qkv, 0, Hkv, D, kw[l], kw[l], EPS, pos, THETA, slots, caches[l], 4,
                                             **opts)
            assert np.array_equal(out[l], ref), opts
