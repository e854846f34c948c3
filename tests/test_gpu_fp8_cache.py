"""GPU parity of the fp8 K/V cache paths (E4M3fn / E5M2 with per-layer
scales): the draft layer's fused q/k write and the context K/V precompute store
the bf16 values their bf16 caches would hold, divided by the scale and rounded
to fp8; the codes must match the oracle's bit for bit on the same bf16 values."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import assert_close, check_attention

pytestmark = pytest.mark.gpu

SENT = 0x7F  # a NaN code in both formats: never written for finite values


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


@pytest.mark.parametrize("fmt,ks,vs", [("e4m3", 0.05, 0.02), ("e5m2", 0.5, 0.25), ("e4m3", 1.0, 1.0)])
def test_qk_fp8_cache_write(B, fmt, ks, vs):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.qk_inputs("mid", pad_fraction=0.1)
    D, Hq, Hkv = d["head_dim"], d["hq"], d["hkv"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    shape = (d["num_blocks"], Hkv, d["block_size"], 2 * D)
    cache = torch.full(shape, SENT, dtype=torch.uint8, device="cuda")
    sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
    q, k = B.qk_norm_rope_cache(dev_bf16(d["qkv"]), Hq, Hkv, D, dev_bf16(d["q_w"]), dev_bf16(d["k_w"]), d["eps"],
                                dev(d["positions"]), cs, dev(d["slots"]), cache, cache_fp8=fmt, kv_scale=sc)
    torch.cuda.synchronize()
    gk, gc = host_bf16(k), cache.cpu().numpy()
    v_in = d["qkv"].reshape(-1, Hq + 2 * Hkv, D)[:, Hq + Hkv:]
    want = np.full(shape, SENT, np.uint8)
    for t, s in enumerate(d["slots"]):
        if s < 0:
            continue
        b, o = divmod(int(s), d["block_size"])
        want[b, :, o, :D] = O.bf16_to_fp8_scaled(gk[t], ks, fmt)
        want[b, :, o, D:] = O.bf16_to_fp8_scaled(v_in[t], vs, fmt)
    assert np.array_equal(gc, want), f"{fmt}: {int((gc != want).sum())} codes differ"
    # and the oracle's own path, within its k_out rounding differences
    rq, rk, rc = O.qk_norm_rope_cache(d["qkv"], Hq, Hkv, D, d["q_w"], d["k_w"], d["eps"], d["positions"],
                                      d["theta"], d["slots"], np.full(shape, SENT, np.uint8), d["block_size"],
                                      cache_fp8=fmt, k_scale=ks, v_scale=vs)
    assert_close(O.bf16_to_f64(gk), O.bf16_to_f64(rk), fmt + " k_out")
    same_k = np.zeros(shape[:3], bool)
    for t, s in enumerate(d["slots"]):
        if s >= 0 and np.array_equal(gk[t], rk[t]):
            b, o = divmod(int(s), d["block_size"])
            same_k[b, :, o] = True
    assert np.array_equal(gc[same_k], rc[same_k])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_context_kv_fp8_store(B, fmt):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.context_kv_inputs("ctx_small", pad_fraction=0.1)
    L, D, Hkv = d["layers"], d["head_dim"], d["hkv"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    shape = (d["num_blocks"], Hkv, d["block_size"], 2 * D)
    scales = np.array([[0.04, 0.01], [0.5, 2.0]], np.float32)[:L]
    args = (dev_bf16(d["ctx_states"]), dev_bf16(d["hidden_norm_w"]), d["eps"], dev_bf16(d["W_kv"]), L, Hkv, D,
            dev_bf16(d["k_norm_w"]), d["eps"], dev(d["positions"]), cs, dev(d["slots"]))
    c16 = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    kv = B.context_kv(*args, c16, want_kv=True)
    c8 = [torch.full(shape, SENT, dtype=torch.uint8, device="cuda") for _ in range(L)]
    B.context_kv(*args, c8, cache_fp8=fmt, kv_scales=torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    kvh = host_bf16(kv)
    for l in range(L):
        g16, g8 = host_bf16(c16[l]), c8[l].cpu().numpy()
        want = np.full(shape, SENT, np.uint8)
        for t, s in enumerate(d["slots"]):
            if s < 0:
                continue
            b, o = divmod(int(s), d["block_size"])
            want[b, :, o, :D] = O.bf16_to_fp8_scaled(g16[b, :, o, :D], scales[l, 0], fmt)
            want[b, :, o, D:] = O.bf16_to_fp8_scaled(kvh[t, l, 1], scales[l, 1], fmt)
        assert np.array_equal(g8, want), f"{fmt} layer {l}: {int((g8 != want).sum())} codes differ"


def _codes(cache, D, ks, vs, fmt):
    c = np.empty(cache.shape, np.uint8)
    c[..., :D] = O.bf16_to_fp8_scaled(cache[..., :D], ks, fmt)
    c[..., D:] = O.bf16_to_fp8_scaled(cache[..., D:], vs, fmt)
    return c


@pytest.mark.parametrize("fmt,ks,vs", [("e4m3", 0.015, 0.01), ("e5m2", 0.5, 0.25)])
def test_block_attn_fp8_cache(B, fmt, ks, vs):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16, say
    a = WL.attention_inputs("attn", requests=8)
    D = a["head_dim"]
    codes = _codes(a["cache"], D, ks, vs, fmt)
    sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
    o = B.block_attn(dev_bf16(a["q"]), dev(codes), dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"],
                     a["window"], cache_fp8=fmt, kv_scale=sc)
    torch.cuda.synchronize()
    ref = O.block_attn(a["q"], codes, a["block_tables"], a["seq_lens"], a["query_len"], a["hq"], a["hkv"], D,
                       a["block_size"], a["window"], D ** -0.5, cache_fp8=fmt, k_scale=ks, v_scale=vs)
    g, r = O.bf16_to_f64(host_bf16(o)), O.bf16_to_f64(ref)
    same, one_ulp, n = check_attention(g, r, f"fp8 {fmt} attention")
    rel = np.abs(g - r).max() / np.sqrt(np.mean(r * r))
    say(f"[attn fp8 {fmt}] equal {same} / within 1 ulp {one_ulp} / {n}; max|d|/rms(ref) = {rel:.3g}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_block_attn_fp8_equals_bf16_on_the_decoded_cache(B, fmt):
    # power-of-two scales: code value * scale is a bf16 number and the scale
    # multiplications are exact, so the fp8 path must give the bf16 path's bits
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    a = WL.attention_inputs("attn", requests=6)
    D = a["head_dim"]
    ks, vs = 0.0078125, 0.0625
    codes = _codes(a["cache"], D, ks, vs, fmt)
    dec = O.fp8_to_f64(codes, fmt)
    dec[..., :D] *= ks
    dec[..., D:] *= vs
    bf = O.f64_to_bf16(dec)
    sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
    args = (dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"], a["window"])
    o8 = B.block_attn(dev_bf16(a["q"]), dev(codes), *args, cache_fp8=fmt, kv_scale=sc)
    o16 = B.block_attn(dev_bf16(a["q"]), dev_bf16(bf), *args)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(o8), host_bf16(o16))


def test_draft_layer_with_an_fp8_cache(B):
    # the draft layer's own block written fp8 by the fused q/k op, then read by
    # the attention, against the oracle's same pipeline
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    fmt, ks, vs = "e4m3", 0.015, 0.01
    a = WL.attention_inputs("attn", requests=6)
    D = a["head_dim"]
    codes = _codes(a["cache"], D, ks, vs, fmt)
    cs = B.rope_cos_sin(a["max_pos"], D, a["theta"], "cuda")
    cache = dev(codes)
    sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
    q, _ = B.qk_norm_rope_cache(dev_bf16(a["qkv"]), a["hq"], a["hkv"], D, dev_bf16(a["q_w"]), dev_bf16(a["k_w"]),
                                a["eps"], dev(a["positions"]), cs, dev(a["slots"]), cache, want_k=False,
                                cache_fp8=fmt, kv_scale=sc)
    o = B.block_attn(q, cache, dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"], a["window"],
                     cache_fp8=fmt, kv_scale=sc)
    torch.cuda.synchronize()
    rq, _, rc = O.qk_norm_rope_cache(a["qkv"], a["hq"], a["hkv"], D, a["q_w"], a["k_w"], a["eps"], a["positions"],
                                     a["theta"], a["slots"], codes, a["block_size"], cache_fp8=fmt, k_scale=ks,
                                     v_scale=vs)
    ro = O.block_attn(rq, rc, a["block_tables"], a["seq_lens"], a["query_len"], a["hq"], a["hkv"], D,
                      a["block_size"], a["window"], D ** -0.5, cache_fp8=fmt, k_scale=ks, v_scale=vs)
    g, r = O.bf16_to_f64(host_bf16(o)), O.bf16_to_f64(ro)
    # the two sides' q differ by rounding in a few elements: see the bf16 pipeline test
    check_attention(g, r, "draft layer over an fp8 cache", pre_round=2.0 ** -10)


def test_context_kv_fp8_with_rope_options(B):
    # fp8 store combined with GPT-J pairing, a partial rotary dim and a bf16 table:
    # the codes are the quantised bf16 cache of the same options
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.context_kv_inputs("ctx_small")
    L, D, Hkv, rot = d["layers"], d["head_dim"], d["hkv"], 48
    cs = B.rope_cos_sin(d["max_pos"], rot, d["theta"], "cuda", dtype=torch.bfloat16)
    shape = (d["num_blocks"], Hkv, d["block_size"], 2 * D)
    scales = torch.tensor([[0.03, 0.02], [0.06, 0.04]], dtype=torch.float32, device="cuda")[:L]
    args = (dev_bf16(d["ctx_states"]), dev_bf16(d["hidden_norm_w"]), d["eps"], dev_bf16(d["W_kv"]), L, Hkv, D,
            dev_bf16(d["k_norm_w"]), d["eps"], dev(d["positions"]), cs, dev(d["slots"]))
    c16 = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    B.context_kv(*args, c16, rotary_dim=rot, is_neox=False)
    c8 = [torch.full(shape, SENT, dtype=torch.uint8, device="cuda") for _ in range(L)]
    B.context_kv(*args, c8, rotary_dim=rot, is_neox=False, cache_fp8="e5m2", kv_scales=scales)
    torch.cuda.synchronize()
    sc = scales.cpu().numpy()
    for l in range(L):
        g16, g8 = host_bf16(c16[l]), c8[l].cpu().numpy()
        w = np.any(g8 != SENT, axis=-1)
        assert np.array_equal(w, np.any(g16 != 0, axis=-1))
        assert np.array_equal(g8[..., :D][w], O.bf16_to_fp8_scaled(g16[..., :D][w], sc[l, 0], "e5m2"))
        assert np.array_equal(g8[..., D:][w], O.bf16_to_fp8_scaled(g16[..., D:][w], sc[l, 1], "e5m2"))


def test_plain_context_kv_and_attention_equal_the_ex_defaults(B):
    import ctypes
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    d = WL.context_kv_inputs("ctx_small")
    L, D, Hkv = d["layers"], d["head_dim"], d["hkv"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    shape = (d["num_blocks"], Hkv, d["block_size"], 2 * D)
    x, hw, Wkv, kw = dev_bf16(d["ctx_states"]), dev_bf16(d["hidden_norm_w"]), dev_bf16(d["W_kv"]), dev_bf16(d["k_norm_w"])
    pos, slots = dev(d["positions"]), dev(d["slots"])
    c1 = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    B.context_kv(x, hw, d["eps"], Wkv, L, Hkv, D, kw, d["eps"], pos, cs, slots, c1)
    c2 = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    n, Hd = x.shape
    ws = torch.empty(B.context_kv_workspace_size(n, Hd), dtype=torch.uint8, device="cuda")
    ptrs = (ctypes.c_void_p * L)(*[c.data_ptr() for c in c2])
    st = B.lib().dflash_context_kv(x.data_ptr(), hw.data_ptr(), d["eps"], Wkv.data_ptr(), n, Hd, L, Hkv, D, kw.data_ptr(), d["eps"],
           pos.data_ptr(), cs.data_ptr(), cs.shape[0], slots.data_ptr(), ctypes.cast(ptrs, ctypes.c_void_p),
           shape[0], shape[2], None, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    for l in range(L):
        assert np.array_equal(host_bf16(c1[l]), host_bf16(c2[l]))
    # attention: the plain call against the binding's _ex call
    a = WL.attention_inputs("attn", requests=3)
    q, cache = dev_bf16(a["q"]), dev_bf16(a["cache"])
    tables, seq = dev(a["block_tables"]), dev(a["seq_lens"])
    o1 = B.block_attn(q, cache, tables, seq, a["query_len"], a["window"])
    o2 = torch.empty_like(o1)
    st = B.lib().dflash_block_attn(q.data_ptr(), cache.data_ptr(), cache.shape[0], tables.data_ptr(), tables.shape[1],
                                   seq.data_ptr(), seq.shape[0], a["query_len"], a["hq"], a["hkv"], D, 16,
                                   a["window"], D ** -0.5, o2.data_ptr(), None, 0,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and np.array_equal(host_bf16(o1), host_bf16(o2))


def test_block_attn_fp8_full_size_equals_bf16_on_the_decoded_cache(B):
    """The attention workload at its full 128 requests over an E4M3 cache (the
    launch the benchmark times): with power-of-two scales the fp8 path must
    give the bf16 path's bits on the decoded cache, and the bf16 path is
    checked against the oracle at this size elsewhere.  Codes and decoded
    values come from torch's own fp8 casts, not from this library."""
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    a = WL.attention_inputs("attn")
    D = a["head_dim"]
    ks, vs = 0.03125, 0.03125  # |K| <= sqrt(128) and |V| < 14 stay below 448 * scale
    c = dev_bf16(a["cache"]).float()
    c[..., :D] /= ks
    c[..., D:] /= vs
    codes = c.to(torch.float8_e4m3fn)
    dec = codes.float()
    assert not torch.isnan(dec).any()  # no value past the format's range
    dec[..., :D] *= ks
    dec[..., D:] *= vs
    bf = dec.to(torch.bfloat16)
    assert torch.equal(bf.float(), dec)  # the decoded values are bf16 numbers
    del c, dec
    sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
    args = (dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"], a["window"])
    q = dev_bf16(a["q"])
    o8 = B.block_attn(q, codes.view(torch.uint8), *args, cache_fp8="e4m3", kv_scale=sc)
    o16 = B.block_attn(q, bf, *args)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(o8), host_bf16(o16))
