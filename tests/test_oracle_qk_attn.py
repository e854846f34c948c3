"""Pins of the oracle's draft-layer q/k RMSNorm + NeoX RoPE + cache write and
of its non-causal sliding-window block attention (vLLM
``DFlash2BeamAttention``: per-head ``q_norm``/``k_norm`` RMSNorm, ``get_rope``
with ``is_neox_style=True``, a slot-mapped K/V cache write, then attention of the
query block over the cache with scale ``head_dim ** -0.5``, every layer
non-causal sliding-window).
"""
import math

import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL

ONE = np.uint16(0x3F80)


def _bf(rng, shape, s=1.0):
    return WL.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


def test_rmsnorm_unit_rms_before_weight():
    rng = np.random.default_rng(0)
    T, Hq, Hkv, D = 5, 2, 1, 64
    qkv = _bf(rng, (T, (Hq + 2 * Hkv) * D), 3.0)
    w = np.full(D, ONE, dtype=np.uint16)
    eps = 1e-6
    q, k, _ = O.qk_norm_rope_cache(qkv, Hq, Hkv, D, w, w, eps, np.zeros(T, np.int64), 1e6)
    x = O.bf16_to_f64(qkv).reshape(T, Hq + 2 * Hkv, D)
    for t in range(T):
        for h in range(Hq):
            ms = np.mean(x[t, h] ** 2)
            rms = math.sqrt(np.mean(O.bf16_to_f64(q[t, h]) ** 2))
            assert rms == pytest.approx(math.sqrt(ms / (ms + eps)), rel=2e-3)  # bf16 output


def test_rmsnorm_weight_is_plain_scale():
    """Weight w (not 1 + w): w = 2 doubles a w = 1 output exactly."""
    rng = np.random.default_rng(1)
    T, D = 3, 32
    qkv = _bf(rng, (T, 3 * D))
    one = np.full(D, ONE, np.uint16)
    two = np.full(D, np.uint16(0x4000), np.uint16)
    q1, k1, _ = O.qk_norm_rope_cache(qkv, 1, 1, D, one, one, 1e-6, np.full(T, 7), 1e4)
    q2, k2, _ = O.qk_norm_rope_cache(qkv, 1, 1, D, two, one, 1e-6, np.full(T, 7), 1e4)
    assert np.array_equal(O.bf16_to_f64(q2), 2 * O.bf16_to_f64(q1))
    assert np.array_equal(k2, k1)


def test_rope_position_zero_is_identity_and_pair_norm_preserved():
    rng = np.random.default_rng(2)
    T, Hq, Hkv, D = 6, 3, 1, 128
    qkv = _bf(rng, (T, (Hq + 2 * Hkv) * D))
    w = _bf(rng, (D,), 0.1)
    w = WL.to_bf16_bits(O.bf16_to_f64(w).astype(np.float32) + 1)
    pos0 = np.zeros(T, np.int64)
    q0, k0, _ = O.qk_norm_rope_cache(qkv, Hq, Hkv, D, w, w, 1e-6, pos0, 1e6)
    # position 0: plain normalised x * w, rounded once
    x = O.bf16_to_f64(qkv).reshape(T, -1, D)
    wf = O.bf16_to_f64(w)
    want = x[:, :Hq] / np.sqrt(np.mean(x[:, :Hq] ** 2, -1, keepdims=True) + 1e-6) * wf
    assert np.array_equal(q0, O.f64_to_bf16(want))
    # pair norm (i, i + D/2) preserved at any position
    pos = np.array([1, 5, 100, 4095, 8191, 123456], np.int64)
    q, k, _ = O.qk_norm_rope_cache(qkv, Hq, Hkv, D, w, w, 1e-6, pos, 1e6)
    a = O.bf16_to_f64(q0)
    b = O.bf16_to_f64(q)
    na = a[..., : D // 2] ** 2 + a[..., D // 2:] ** 2
    nb = b[..., : D // 2] ** 2 + b[..., D // 2:] ** 2
    assert np.allclose(nb, na, rtol=2e-2, atol=1e-4)  # bf16 outputs on both sides


def test_rope_neox_pairing_and_angle():
    """A unit vector e_i rotates into (cos a, sin a) on the pair (i, i + D/2),
    a = pos * theta^(-2i/D); nothing leaks into other coordinates (GPT-J style
    pairing (2i, 2i+1) would)."""
    D, theta = 16, 10000.0
    for i in (0, 3, 7):
        row = np.zeros((1, 3 * D), np.float32)
        row[0, i] = 1.0
        row[0, D + i] = 1.0
        qkv = WL.to_bf16_bits(row)
        w = np.full(D, ONE, np.uint16)
        pos = np.array([9], np.int64)
        q, k, _ = O.qk_norm_rope_cache(qkv, 1, 1, D, w, w, 0.0, pos, theta)
        y = O.bf16_to_f64(q[0, 0])
        a = 9 * theta ** (-2 * i / D)
        r = math.sqrt(D)  # rms norm of e_i scales it to sqrt(D)
        want = np.zeros(D)
        want[i] = r * math.cos(a)
        want[i + D // 2] = r * math.sin(a)
        assert np.allclose(y, want, rtol=4e-3, atol=4e-3 * r)
        assert np.array_equal(q[0, 0], k[0, 0])


def test_cache_write_sentinel():
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D, bs, nblk = 12, 2, 2, 32, 4, 8
    qkv = _bf(rng, (T, (Hq + 2 * Hkv) * D))
    w = np.full(D, ONE, np.uint16)
    slots = rng.permutation(nblk * bs)[:T].astype(np.int64)
    slots[[2, 7, 11]] = -1
    cache = np.full((nblk, Hkv, bs, 2 * D), 0xFFFF, np.uint16)
    pos = rng.integers(0, 100, T)
    q, k, c2 = O.qk_norm_rope_cache(qkv, Hq, Hkv, D, w, w, 1e-6, pos, 1e4, slots, cache, bs)
    changed = np.zeros(nblk * bs, bool)
    v = qkv.reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:]
    for t in range(T):
        s = slots[t]
        if s < 0:
            continue
        changed[s] = True
        b, o = divmod(s, bs)
        assert np.array_equal(c2[b, :, o, D:], v[t])      # V bits unchanged
        assert np.array_equal(c2[b, :, o, :D], k[t])      # K' as returned
    flat = c2.transpose(0, 2, 1, 3).reshape(nblk * bs, -1)
    assert np.all(flat[~changed] == 0xFFFF)
    assert changed.sum() == T - 3
    # no cache: nothing returned
    _, _, none = O.qk_norm_rope_cache(qkv, Hq, Hkv, D, w, w, 1e-6, pos, 1e4)
    assert none is None


# ---------------------------------------------------------------- attention
def _paged(rng, seq_lens, Hkv, D, bs):
    nb = [(L + bs - 1) // bs for L in seq_lens]
    perm = rng.permutation(sum(nb)).astype(np.int32)
    tables = np.zeros((len(seq_lens), max(nb)), np.int32)
    off = 0
    for r, n in enumerate(nb):
        tables[r, :n] = perm[off:off + n]
        off += n
    cache = _bf(rng, (sum(nb), Hkv, bs, 2 * D))
    return cache, tables


def _brute_attention(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, window, scale):
    """Pure-Python loops over every (request, head, query, key)."""
    Rq = len(seq_lens)
    out = np.zeros((Rq * Lq, Hq, D))
    qf = O.bf16_to_f64(q)
    for r in range(Rq):
        L = int(seq_lens[r])
        for i in range(Lq):
            pos = L - Lq + i
            for h in range(Hq):
                kh = h // (Hq // Hkv)
                scores, vals = [], []
                for j in range(L):
                    if j < pos - window + 1:
                        continue
                    row = cache[tables[r, j // bs], kh, j % bs]
                    kv = O.bf16_to_f64(row)
                    scores.append(sum(qf[r * Lq + i, h, d] * kv[d] for d in range(D)) * scale)
                    vals.append(kv[D:])
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                z = sum(e)
                out[r * Lq + i, h] = sum(ej / z * v for ej, v in zip(e, vals))
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(4)
    Lq, Hq, Hkv, D, bs, window = 3, 4, 2, 8, 4, 5
    seq_lens = np.array([3, 7, 12], np.int32)  # first request: block only
    cache, tables = _paged(rng, seq_lens, Hkv, D, bs)
    q = _bf(rng, (len(seq_lens) * Lq, Hq, D))
    scale = D ** -0.5
    got = O.bf16_to_f64(O.block_attn(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, window, scale))
    want = _brute_attention(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, window, scale)
    assert np.array_equal(got, O.bf16_to_f64(O.f64_to_bf16(want))) or \
        np.allclose(got, want, rtol=8e-3, atol=1e-6)


def test_attention_one_visible_key_returns_its_value():
    rng = np.random.default_rng(5)
    Lq, Hq, Hkv, D, bs = 1, 2, 1, 16, 4
    seq_lens = np.array([9], np.int32)
    cache, tables = _paged(rng, seq_lens, Hkv, D, bs)
    q = _bf(rng, (1, Hq, D))
    o = O.block_attn(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, 1, D ** -0.5)
    v = cache[tables[0, 8 // bs], 0, 8 % bs, D:]
    assert np.array_equal(o[0, 0], v) and np.array_equal(o[0, 1], v)


def test_attention_equal_keys_give_mean_value():
    rng = np.random.default_rng(6)
    Lq, Hq, Hkv, D, bs, window = 4, 2, 2, 8, 4, 6
    seq_lens = np.array([14], np.int32)
    cache, tables = _paged(rng, seq_lens, Hkv, D, bs)
    cache[..., :D] = cache[0, 0, 0, :D]  # every key the same
    q = _bf(rng, (Lq, Hq, D))
    o = O.bf16_to_f64(O.block_attn(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, window, 0.3))
    L = 14
    for i in range(Lq):
        pos = L - Lq + i
        keys = range(max(0, pos - window + 1), L)
        for h in range(Hq):
            vm = np.mean([O.bf16_to_f64(cache[tables[0, j // bs], h, j % bs, D:]) for j in keys], axis=0)
            assert np.allclose(o[i, h], vm, rtol=8e-3, atol=1e-6)


def test_attention_wide_window_is_full_noncausal():
    """window >= seq_len: every query sees every key of its request, so all
    queries of one head with equal q give equal outputs."""
    rng = np.random.default_rng(7)
    Lq, Hq, Hkv, D, bs = 4, 2, 1, 8, 4
    seq_lens = np.array([10], np.int32)
    cache, tables = _paged(rng, seq_lens, Hkv, D, bs)
    q = np.broadcast_to(_bf(rng, (1, Hq, D)), (Lq, Hq, D)).copy()
    o = O.block_attn(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, 10, D ** -0.5)
    assert np.all(o == o[:1])
    o_small = O.block_attn(q, cache, tables, seq_lens, Lq, Hq, Hkv, D, bs, 3, D ** -0.5)
    assert not np.all(o_small == o_small[:1])  # with a window, queries differ


def test_window_bounds_reading():
    # query i at seq_len - Lq + i; the window keeps `window` keys at or before it
    assert O.attention_window(100, 16, 0, 2048) == (0, 100)
    assert O.attention_window(5000, 16, 0, 2048) == (5000 - 16 - 2047, 5000)
    assert O.attention_window(5000, 16, 15, 2048) == (5000 - 1 - 2047, 5000)
