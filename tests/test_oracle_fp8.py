"""Pins of the oracle's fp8 cache arithmetic: OCP E4M3 ("fn") and E5M2 codes by
their definitions, round to nearest with ties to the even code and saturation,
and the fp8 variants of the cache writers and of the attention."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL


@pytest.mark.parametrize("fmt,x,code", [
    ("e4m3", 1.0, 0x38), ("e4m3", -2.0, 0xC0), ("e4m3", 448.0, 0x7E), ("e4m3", 2.0 ** -6, 0x08),
    ("e4m3", 2.0 ** -9, 0x01), ("e4m3", 7 * 2.0 ** -9, 0x07), ("e4m3", 0.0, 0x00), ("e4m3", 1000.0, 0x7E),
    ("e4m3", -1e9, 0xFE), ("e4m3", 1.0625, 0x38), ("e4m3", 1.1875, 0x3A), ("e4m3", 1.5 * 2.0 ** -9, 0x02),
    ("e4m3", 0.5 * 2.0 ** -9, 0x00), ("e4m3", 0.51 * 2.0 ** -9, 0x01), ("e4m3", 460.0, 0x7E),
    ("e5m2", 1.0, 0x3C), ("e5m2", 57344.0, 0x7B), ("e5m2", 2.0 ** -14, 0x04), ("e5m2", 2.0 ** -16, 0x01),
    ("e5m2", 1e6, 0x7B), ("e5m2", 1.125, 0x3C), ("e5m2", 1.375, 0x3E), ("e5m2", -0.75, 0xBA),
])
def test_known_codes(fmt, x, code):
    assert int(O.f64_to_fp8(np.array([x]), fmt)[0]) == code
    if abs(x) <= (448 if fmt == "e4m3" else 57344) and code not in (0x00,):
        v = O.fp8_to_f64(np.array([code], np.uint8), fmt)[0]
        assert abs(v - x) <= abs(x) * 2 ** -3 + 2.0 ** -10  # relative step, or half the subnormal step


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_code_round_trips(fmt):
    codes = np.arange(256, dtype=np.uint8)
    v = O.fp8_to_f64(codes, fmt)
    ok = np.isfinite(v)
    assert np.array_equal(O.f64_to_fp8(v[ok], fmt), codes[ok])
    assert ok.sum() == (254 if fmt == "e4m3" else 248)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rounding_is_nearest_and_monotone(fmt):
    x = np.linspace(-600 if fmt == "e4m3" else -70000, 600 if fmt == "e4m3" else 70000, 20001)
    x = np.concatenate([x, np.geomspace(1e-7, 10, 4001), -np.geomspace(1e-7, 10, 4001)])
    x.sort()
    c = O.f64_to_fp8(x, fmt)
    v = O.fp8_to_f64(c, fmt)
    assert np.all(np.diff(v) >= 0)                       # monotone
    _, table = O._fp8_positive_table(fmt)
    a = np.abs(x)
    inside = a <= table[-1]
    # no finite value is strictly closer than the chosen one
    d = np.abs(np.abs(v) - a)
    best = np.min(np.abs(table[None, :] - a[inside][:, None]), axis=1)
    assert np.all(d[inside] <= best + 1e-300)
    assert np.all(np.abs(v[~inside]) == table[-1])      # saturation


def test_scaled_conversion_divides_in_fp32():
    bits = WL.to_bf16_bits(np.array([2.0, -3.0, 0.1], np.float32))
    c = O.bf16_to_fp8_scaled(bits, 0.5, "e4m3")
    assert c[0] == O.f64_to_fp8(np.array([4.0]), "e4m3")[0] == 0x48
    assert c[1] == 0xC8 | 0x04      # -6.0 = -1.5 * 2^2
    q = np.float32(O.bf16_to_f64(bits[2:])[0]) / np.float32(0.5)
    assert c[2] == O.f64_to_fp8(np.array([float(q)]), "e4m3")[0]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_attention_equals_attention_on_the_dequantised_cache(fmt):
    # e4m3 / e5m2 values times a power of two are bf16 numbers: the fp8 path
    # must equal the bf16 path on the decoded cache exactly
    rng = np.random.default_rng(3)
    D, bs, Lq, Hq, Hkv = 128, 16, 4, 2, 1
    seq = np.array([40, 60], np.int32)
    tables = rng.permutation(8).astype(np.int32).reshape(2, 4)
    q = WL.to_bf16_bits(rng.standard_normal((2 * Lq, Hq, D)).astype(np.float32))
    codes = rng.integers(0, 256, size=(8, Hkv, bs, 2 * D), dtype=np.uint8)
    bad = ~np.isfinite(O.fp8_to_f64(codes, fmt))
    codes[bad] = 0x30
    ks, vs = 0.5, 2.0
    dec = O.fp8_to_f64(codes, fmt)
    dec[..., :D] *= ks
    dec[..., D:] *= vs
    bf = O.f64_to_bf16(dec)
    assert np.array_equal(O.bf16_to_f64(bf), dec)
    args = (q, None, tables, seq, Lq, Hq, Hkv, D, bs, 50, D ** -0.5)
    o8 = O.block_attn(args[0], codes, *args[2:], cache_fp8=fmt, k_scale=ks, v_scale=vs)
    o16 = O.block_attn(args[0], bf, *args[2:])
    assert np.array_equal(o8, o16)


def test_fp8_writers_store_the_bf16_values_quantised():
    rng = np.random.default_rng(4)
    n, L, Hkv, D = 5, 2, 2, 128
    kv = WL.to_bf16_bits(rng.standard_normal((n, L, 2, Hkv, D)).astype(np.float32))
    kw = WL.to_bf16_bits((1 + 0.1 * rng.standard_normal((L, D))).astype(np.float32))
    pos = rng.integers(0, 3000, n)
    slots = rng.permutation(64)[:n].astype(np.int64)
    slots[1] = -1
    ks, vs = np.array([0.25, 0.5]), np.array([0.125, 1.0])
    c16 = O.store_context_kv(kv, kw, 1e-6, pos, 1e6, slots, [np.zeros((16, Hkv, 4, 2 * D), np.uint16)] * L, 4)
    c8 = O.store_context_kv(kv, kw, 1e-6, pos, 1e6, slots, [np.zeros((16, Hkv, 4, 2 * D), np.uint8)] * L, 4,
                            cache_fp8="e4m3", k_scale=ks, v_scale=vs)
    for l in range(L):
        for t in range(n):
            if slots[t] < 0:
                continue
            b, o = divmod(int(slots[t]), 4)
            assert np.array_equal(c8[l][b, :, o, :D], O.bf16_to_fp8_scaled(c16[l][b, :, o, :D], ks[l], "e4m3"))
            assert np.array_equal(c8[l][b, :, o, D:], O.bf16_to_fp8_scaled(kv[t, l, 1], vs[l], "e4m3"))
    # the draft layer's writer: the same rule on k_out and the V input
    d = WL.qk_inputs("mid")
    Tq = 20
    qkv = d["qkv"][:Tq]
    cache8 = np.zeros((d["num_blocks"], d["hkv"], d["block_size"], 2 * D), np.uint8)
    q, k, c = O.qk_norm_rope_cache(qkv, d["hq"], d["hkv"], D, d["q_w"], d["k_w"], d["eps"], d["positions"][:Tq],
                                   d["theta"], d["slots"][:Tq], cache8, d["block_size"], cache_fp8="e5m2",
                                   k_scale=0.5, v_scale=0.25)
    v_in = qkv.reshape(Tq, d["hq"] + 2 * d["hkv"], D)[:, d["hq"] + d["hkv"]:]
    for t in range(Tq):
        b, o = divmod(int(d["slots"][t]), d["block_size"])
        assert np.array_equal(c[b, :, o, :D], O.bf16_to_fp8_scaled(k[t], 0.5, "e5m2"))
        assert np.array_equal(c[b, :, o, D:], O.bf16_to_fp8_scaled(v_in[t], 0.25, "e5m2"))
