"""GPU parity of dflash_qk_norm_rope_cache and dflash_block_attn against the
oracle (DFlash2BeamAttention: q/k RMSNorm + NeoX RoPE + slot-mapped cache write,
then non-causal sliding-window attention of the query block)."""
import numpy as np
import pytest

from oracle import dflash_oracle as O
import workloads as WL
from tests.parity import ATTN_PRE_ROUND, assert_close, check_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_candidate_amd as B
    B.lib()
    return B


def _qk(B, d, with_cache=True, want_k=True, sentinel=True):
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    D = d["head_dim"]
    cs = B.rope_cos_sin(d["max_pos"], D, d["theta"], "cuda")
    cache0 = np.full_like(d["cache"], 0xFFFF) if sentinel else d["cache"]
    cache = dev_bf16(cache0) if with_cache else None
    slots = dev(d["slots"]) if with_cache else None
    q, k = B.qk_norm_rope_cache(dev_bf16(d["qkv"]), d["hq"], d["hkv"], D, dev_bf16(d["q_w"]),
                                dev_bf16(d["k_w"]), d["eps"], dev(d["positions"]), cs, slots, cache,
                                want_k=want_k)
    torch.cuda.synchronize()
    return (host_bf16(q), None if k is None else host_bf16(k),
            None if cache is None else host_bf16(cache), cache0)


def _check_qk(B, d, label):
    from tests.gpu_common import say
    q, k, cache, cache0 = _qk(B, d)
    rq, rk, rcache = O.qk_norm_rope_cache(d["qkv"], d["hq"], d["hkv"], d["head_dim"], d["q_w"], d["k_w"],
                                          d["eps"], d["positions"], d["theta"], d["slots"], cache0,
                                          d["block_size"])
    assert_close(O.bf16_to_f64(q), O.bf16_to_f64(rq), label + " q")
    assert_close(O.bf16_to_f64(k), O.bf16_to_f64(rk), label + " k")
    D = d["head_dim"]
    # exactly the slots >= 0 were written; V bits copied; K = the kernel's own k_out
    written = np.any(cache != cache0, axis=-1)
    expect = np.any(rcache != cache0, axis=-1)
    assert np.array_equal(written, expect), label + ": written cache rows differ"
    assert np.array_equal(cache[..., D:], rcache[..., D:]), label + ": V payload"
    for t, s in enumerate(d["slots"]):
        if s >= 0:
            b, o = divmod(int(s), d["block_size"])
            assert np.array_equal(cache[b, :, o, :D], k[t]), label + ": cache K != k_out"
    ulp = int(np.count_nonzero(q != rq)) + int(np.count_nonzero(k != rk))
    say(f"[qk {label}] outputs differing by rounding: {ulp} of {q.size + k.size}")


def test_qk_mid(B):
    _check_qk(B, WL.qk_inputs("mid"), "mid")


def test_qk_mid_with_padding_slots(B):
    d = WL.qk_inputs("mid", pad_fraction=0.1)
    assert (d["slots"] < 0).sum() > 0
    _check_qk(B, d, "mid+pad")


def test_qk_attention_workload(B):
    a = WL.attention_inputs("attn")
    d = dict(qkv=a["qkv"], q_w=a["q_w"], k_w=a["k_w"], positions=a["positions"], slots=a["slots"],
             cache=a["cache"], hq=a["hq"], hkv=a["hkv"], head_dim=a["head_dim"],
             block_size=a["block_size"], eps=a["eps"], theta=a["theta"], max_pos=a["max_pos"])
    _check_qk(B, d, "attn")


def test_qk_without_cache_and_without_k(B):
    d = WL.qk_inputs("mid")
    q, k, cache, _ = _qk(B, d, with_cache=False)
    rq, rk, _ = O.qk_norm_rope_cache(d["qkv"], d["hq"], d["hkv"], d["head_dim"], d["q_w"], d["k_w"],
                                     d["eps"], d["positions"], d["theta"])
    assert cache is None
    assert_close(O.bf16_to_f64(q), O.bf16_to_f64(rq), "q (no cache)")
    assert_close(O.bf16_to_f64(k), O.bf16_to_f64(rk), "k (no cache)")
    q2, k2, c2, _ = _qk(B, d, with_cache=True, want_k=False)
    assert k2 is None and np.array_equal(q2, q)


# ------------------------------------------------------------------ attention
def _attn(B, a, window=None, Lq=None):
    from tests.gpu_common import dev, dev_bf16, host_bf16
    o = B.block_attn(dev_bf16(a["q"]), dev_bf16(a["cache"]), dev(a["block_tables"]), dev(a["seq_lens"]),
                     a["query_len"] if Lq is None else Lq, a["window"] if window is None else window)
    return host_bf16(o)


def _ref_attn(a, window=None):
    D = a["head_dim"]
    return O.block_attn(a["q"], a["cache"], a["block_tables"], a["seq_lens"], a["query_len"], a["hq"],
                        a["hkv"], D, a["block_size"], a["window"] if window is None else window, D ** -0.5)


def _check_attn(got, ref, label, pre_round=ATTN_PRE_ROUND):
    from tests.gpu_common import say
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    same, one_ulp, n = check_attention(g, r, label, pre_round)
    rel = np.abs(g - r).max() / np.sqrt(np.mean(r * r))
    say(f"[attn {label}] equal {same} / within 1 ulp {one_ulp} / {n}; max|d|/rms(ref) = {rel:.3g}")


@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_attention_workload(B, q_scale):
    a = WL.attention_inputs("attn", q_scale=q_scale)
    _check_attn(_attn(B, a), _ref_attn(a), f"attn q*{q_scale}")


def _small_attn(seed, seq_lens, Lq, Hq, Hkv, window):
    rng = np.random.default_rng(seed)
    D, bs = 128, 16
    seq = np.asarray(seq_lens, np.int32)
    nb = (seq + bs - 1) // bs
    perm = rng.permutation(int(nb.sum())).astype(np.int32)
    tables = np.zeros((len(seq), int(nb.max()) + 1), np.int32)
    off = 0
    for r, n in enumerate(nb):
        tables[r, :n] = perm[off:off + n]
        off += n
    cache = WL.to_bf16_bits(rng.standard_normal((int(nb.sum()), Hkv, bs, 2 * D)).astype(np.float32))
    q = WL.to_bf16_bits((rng.standard_normal((len(seq) * Lq, Hq, D)) * 2).astype(np.float32))
    return dict(q=q, cache=cache, block_tables=tables, seq_lens=seq, query_len=Lq, hq=Hq, hkv=Hkv,
                head_dim=D, block_size=bs, window=window)


@pytest.mark.parametrize("seq_lens,Lq,Hq,Hkv,window", [
    ([16, 17, 100, 333, 64, 65], 16, 8, 2, 40),      # window cuts inside a block; ragged ends
    ([9, 30, 500], 9, 16, 4, 2048),                  # Lq = 9 (8 mask tokens), wide window
    ([40, 200], 3, 4, 4, 1),                         # group of 1; one key before each query
    ([300, 129], 16, 16, 2, 128),                    # group of 8
    ([5, 16], 8, 4, 2, 10),                          # a request shorter than the block
])
def test_attention_shapes(B, seq_lens, Lq, Hq, Hkv, window):
    a = _small_attn(sum(seq_lens) + Lq, seq_lens, Lq, Hq, Hkv, window)
    got = _attn(B, a)
    if min(seq_lens) < Lq:
        short = [r for r, L in enumerate(seq_lens) if L < Lq]
        for r in short:
            assert np.all(O.bf16_to_f64(got[r * Lq:(r + 1) * Lq]) == 0)
        keep = [r for r, L in enumerate(seq_lens) if L >= Lq]
        sub = dict(a, seq_lens=a["seq_lens"][keep], block_tables=a["block_tables"][keep],
                   q=a["q"].reshape(len(seq_lens), Lq, Hq, -1)[keep].reshape(len(keep) * Lq, Hq, -1))
        ref = _ref_attn(sub)
        got = got.reshape(len(seq_lens), Lq, Hq, -1)[keep].reshape(len(keep) * Lq, Hq, -1)
    else:
        ref = _ref_attn(a)
    _check_attn(got, ref, f"L={seq_lens} Lq={Lq} G={Hq // Hkv} W={window}")


def test_pipeline_qk_then_attention(B):
    """The draft layer's order: the fused kernel writes the block's K/V into the
    cache, then attention reads it; the oracle runs the same two steps itself."""
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16
    a = WL.attention_inputs("attn", requests=16)
    D = a["head_dim"]
    cs = B.rope_cos_sin(a["max_pos"], D, a["theta"], "cuda")
    cache = dev_bf16(a["cache"])
    q, _ = B.qk_norm_rope_cache(dev_bf16(a["qkv"]), a["hq"], a["hkv"], D, dev_bf16(a["q_w"]),
                                dev_bf16(a["k_w"]), a["eps"], dev(a["positions"]), cs, dev(a["slots"]),
                                cache, want_k=False)
    o = B.block_attn(q, cache, dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"], a["window"])
    torch.cuda.synchronize()
    rq, _, rcache = O.qk_norm_rope_cache(a["qkv"], a["hq"], a["hkv"], D, a["q_w"], a["k_w"], a["eps"],
                                         a["positions"], a["theta"], a["slots"], a["cache"], a["block_size"])
    ref = O.block_attn(rq, rcache, a["block_tables"], a["seq_lens"], a["query_len"], a["hq"], a["hkv"], D,
                       a["block_size"], a["window"], D ** -0.5)
    # the two sides' q differ by rounding in a few elements (counted by the q/k
    # tests): one ulp of a q element (2^-8 relative, |q k| <= ~16, scale 2^-3.5)
    # moves that head's scores by up to ~5e-3 and its outputs by up to ~1e-3
    _check_attn(host_bf16(o), ref, "qk -> attn", pre_round=2.0 ** -10)


def _plant_window_edges(a, value=50.0):
    """Cache copy whose V rows (every kv head) hold +-value at the keys around
    each query's window edge: its first visible key, the key just below it, and
    the request's last key.  A key wrongly in or out of one query's window then
    moves that query's output by about value / (visible keys) in every element."""
    cache = a["cache"].copy()
    D, bs, Lq, W = a["head_dim"], a["block_size"], a["query_len"], a["window"]
    plus, minus = WL.to_bf16_bits(np.float32([value, -value]))
    planted = 0
    for r in range(a["requests"]):
        L = int(a["seq_lens"][r])
        marks = {L - 1}
        for i in range(Lq):
            lo = L - Lq + i - W + 1
            marks.update(x for x in (lo - 1, lo) if x >= 0)
        for j in marks:
            b, o = divmod(j, bs)
            cache[a["block_tables"][r, b], :, o, D:] = plus if j % 2 == 0 else minus
        planted += len(marks)
    return cache, planted


def test_attention_window_edges_planted(B):
    """Large V rows at every query's window edge (R17: the window keeps the W
    keys at or before the query's position; later keys of the block are all
    visible): an off-by-one at either end, or a lost last key, fails."""
    from tests.gpu_common import say
    a = WL.attention_inputs("attn", requests=32)
    cache, planted = _plant_window_edges(a)
    a = dict(a, cache=cache)
    edged = int(np.sum(a["seq_lens"] - a["query_len"] - a["window"] + 1 > 0))
    say(f"[attn planted] {planted} planted keys; {edged} of {a['requests']} requests have a window edge")
    assert edged >= a["requests"] // 2
    _check_attn(_attn(B, a), _ref_attn(a), "window edges planted")
    # the planted rows matter: the same window one key wider changes the outputs
    wider = _ref_attn(a, window=a["window"] + 1)
    assert not np.array_equal(wider, _ref_attn(a))


def _nan_unwritten(a):
    """Cache copy whose rows at positions >= seq_len in each request's last block
    (never written) hold NaN."""
    cache = a["cache"].copy()
    bs = a["block_size"]
    nan = WL.to_bf16_bits(np.float32([np.nan]))[0]
    n = 0
    for r in range(a["requests"]):
        L = int(a["seq_lens"][r])
        if L % bs:
            cache[a["block_tables"][r, (L - 1) // bs], :, L % bs:, :] = nan
            n += bs - L % bs
    return cache, n


@pytest.mark.parametrize("fmt", [None, "e4m3", "e5m2"])
def test_attention_ignores_unwritten_slots(B, fmt):
    """The rows past each request's length in its last cache block are never
    written (a stale NaN or Inf may sit there); the attention must not read them
    into the output: equal to the oracle, which reads only written rows."""
    import torch
    from tests.gpu_common import dev, dev_bf16, host_bf16, say
    a = WL.attention_inputs("attn", requests=16)
    cache, n = _nan_unwritten(a)
    assert n > 0
    D = a["head_dim"]
    args = (dev(a["block_tables"]), dev(a["seq_lens"]), a["query_len"], a["window"])
    if fmt is None:
        o = B.block_attn(dev_bf16(a["q"]), dev_bf16(cache), *args)
        ref = O.block_attn(a["q"], cache, a["block_tables"], a["seq_lens"], a["query_len"], a["hq"], a["hkv"], D,
                           a["block_size"], a["window"], D ** -0.5)
    else:
        ks, vs = 0.0078125, 0.0625
        codes = np.empty(cache.shape, np.uint8)
        codes[..., :D] = O.bf16_to_fp8_scaled(cache[..., :D], ks, fmt)
        codes[..., D:] = O.bf16_to_fp8_scaled(cache[..., D:], vs, fmt)
        sc = torch.tensor([ks, vs], dtype=torch.float32, device="cuda")
        o = B.block_attn(dev_bf16(a["q"]), dev(codes), *args, cache_fp8=fmt, kv_scale=sc)
        ref = O.block_attn(a["q"], codes, a["block_tables"], a["seq_lens"], a["query_len"], a["hq"], a["hkv"], D,
                           a["block_size"], a["window"], D ** -0.5, cache_fp8=fmt, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    say(f"[attn unwritten NaN {fmt}] {n} NaN rows per kv head")
    _check_attn(host_bf16(o), ref, f"NaN in unwritten rows ({fmt or 'bf16'})")
