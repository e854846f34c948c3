"""Pins of the oracle's context K/V precompute (DFlash2BeamModel
``precompute_and_store_context_kv``: ``hidden_norm`` RMSNorm of the context
states, one linear against every draft layer's stacked K/V rows, then
``store_context_kv``: each layer's K-norm and RoPE on K, K and V written to that
layer's cache)."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL


def _bf(rng, shape, s=1.0):
    return WL.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


def test_rms_norm_constant_row_closed_form():
    d, c, eps = 64, 3.0, 1e-6
    x = WL.to_bf16_bits(np.full((2, d), c, np.float32))
    w = WL.to_bf16_bits(np.linspace(0.5, 1.5, d).astype(np.float32))
    y = O.bf16_to_f64(O.rms_norm(x, w, eps))
    want = c / np.sqrt(c * c + eps) * O.bf16_to_f64(w)
    assert np.allclose(y, want, rtol=2 ** -8)


def test_rms_norm_brute_force_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = _bf(rng, (3, 40))
    w = _bf(rng, (40,), 0.5)
    y = O.bf16_to_f64(O.rms_norm(x, w, 1e-6))
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    for r in range(3):
        ms = sum(v * v for v in xf[r]) / 40
        for i in range(40):
            assert y[r, i] == pytest.approx(xf[r, i] / np.sqrt(ms + 1e-6) * wf[i], rel=2 ** -8, abs=1e-30)
    # a power-of-two scale of the row changes nothing (eps negligible)
    y2 = O.rms_norm(WL.to_bf16_bits((xf * 4.0).astype(np.float32)), w, 1e-12)
    assert np.array_equal(y2, O.rms_norm(x, w, 1e-12))


def test_context_kv_layout_with_selector_rows():
    # rows of W_ctx that are unit vectors copy columns of the normed states: each
    # (layer, K/V, head, dim) output lands where the [num_ctx, L, 2, Hkv, D] view says
    rng = np.random.default_rng(2)
    n, hid, L, Hkv, D = 5, 48, 2, 2, 4
    ctx = _bf(rng, (n, hid))
    w = _bf(rng, (hid,), 0.3)
    rows = L * 2 * Hkv * D
    cols = rng.integers(0, hid, rows)
    W = np.zeros((rows, hid), np.float32)
    W[np.arange(rows), cols] = 1.0
    kv = O.context_kv(ctx, w, 1e-6, WL.to_bf16_bits(W), L, Hkv, D)
    normed = O.rms_norm(ctx, w, 1e-6)
    assert kv.shape == (n, L, 2, Hkv, D)
    flat = kv.reshape(n, rows)
    assert np.array_equal(flat, normed[:, cols])
    l, j, h, dd = 1, 1, 0, 3
    assert np.array_equal(kv[:, l, j, h, dd], normed[:, cols[((l * 2 + j) * Hkv + h) * D + dd]])


def test_context_kv_brute_force():
    rng = np.random.default_rng(3)
    n, hid, L, Hkv, D = 2, 16, 1, 1, 4
    ctx, w, W = _bf(rng, (n, hid)), _bf(rng, (hid,), 0.5), _bf(rng, (L * 2 * Hkv * D, hid), 0.3)
    kv = O.bf16_to_f64(O.context_kv(ctx, w, 1e-6, W, L, Hkv, D)).reshape(n, -1)
    normed, Wf = O.bf16_to_f64(O.rms_norm(ctx, w, 1e-6)), O.bf16_to_f64(W)
    for t in range(n):
        for o in range(L * 2 * Hkv * D):
            assert kv[t, o] == pytest.approx(sum(normed[t, j] * Wf[o, j] for j in range(hid)), rel=2 ** -8)


def _store_case(L=2, n=6, Hkv=2, D=8, nblk=4, bs=4, seed=4):
    rng = np.random.default_rng(seed)
    kv = _bf(rng, (n, L, 2, Hkv, D))
    kw = WL.to_bf16_bits((1 + 0.1 * rng.standard_normal((L, D))).astype(np.float32))
    pos = rng.integers(0, 500, n)
    slots = rng.permutation(nblk * bs)[:n].astype(np.int64)
    slots[2] = -1
    caches = [_bf(rng, (nblk, Hkv, bs, 2 * D)) for _ in range(L)]
    return kv, kw, pos, slots, caches


def test_store_context_kv_equals_the_draft_layer_k_path():
    # for each layer, the same as qk_norm_rope_cache's K path (no q heads) on that
    # layer's K and V with its K-norm weight
    kv, kw, pos, slots, caches = _store_case()
    out = O.store_context_kv(kv, kw, 1e-6, pos, 1e6, slots, caches, 4)
    n, L, _, Hkv, D = kv.shape
    for l in range(L):
        qkv = np.concatenate([kv[:, l, 0].reshape(n, Hkv * D), kv[:, l, 1].reshape(n, Hkv * D)], axis=1)
        _, _, ref = O.qk_norm_rope_cache(qkv, 0, Hkv, D, kw[l], kw[l], 1e-6, pos, 1e6, slots, caches[l], 4)
        assert np.array_equal(out[l], ref)


def test_store_context_kv_skips_padding_and_copies_v_bits():
    kv, kw, pos, slots, caches = _store_case()
    out = O.store_context_kv(kv, kw, 1e-6, pos, 1e6, slots, caches, 4)
    written = np.zeros(caches[0].shape[0] * caches[0].shape[2], bool)
    for t, s in enumerate(slots):
        if s >= 0:
            b, o = divmod(int(s), 4)
            written[s] = True
            for l in range(2):
                assert np.array_equal(out[l][b, :, o, 8:], kv[t, l, 1])
    for l in range(2):
        for s in np.flatnonzero(~written):
            b, o = divmod(int(s), 4)
            assert np.array_equal(out[l][b, :, o], caches[l][b, :, o])


def test_store_context_kv_position_zero_is_norm_only():
    kv, kw, pos, slots, caches = _store_case()
    pos = np.zeros_like(pos)
    out = O.store_context_kv(kv, kw, 1e-6, pos, 1e6, slots, caches, 4)
    t = 0
    b, o = divmod(int(slots[t]), 4)
    for l in range(2):
        assert np.array_equal(out[l][b, :, o, :8], O.rms_norm(kv[t, l, 0], kw[l], 1e-6))
