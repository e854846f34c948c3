"""CPU oracle of the DFlash2 block-draft candidate step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Plain numpy, float64 arithmetic throughout (the pages fix no accumulation
precision; float64 makes the oracle the definition up to rounding), with one
rounding at each point where the method's data type is narrower than that:

* bf16 inputs are widened exactly;
* LM-head logits are an fp32 number whose bf16 rounding is the top-k key
  (see ``lm_topk``);
* bf16 outputs (q/k after norm + RoPE, attention output) are rounded once,
  float64 -> fp32 -> bf16, each step round-to-nearest-even.

Sources (vLLM API docs of ``vllm.models.beam.nvidia.dflash2`` and of the DFlash
speculator ``vllm.v1.worker.gpu.spec_decode.dflash.speculator``):

* ``DFlash2BeamForCausalLM.compute_candidates`` and its ``LogitsProcessor``
  (``scale=output_multiplier``, ``soft_cap=final_logit_softcapping``, a cap of
  zero or less means none) -> ``lm_topk``;
* ``DFlash2BeamCandidateSelector`` (class docstring: edge score = candidate's
  own logit + <predecessor[q] * h_p, successor[c]>, predecessor of the first
  position = the anchor token; ``forward``: output ``[requests, steps, top_k,
  top_k]``; ``hidden_projection`` = bias-free ``hidden -> rank`` linear)
  -> ``candidate_edges``;
* ``DFlash2BeamAttention.forward`` (per-head q/k RMSNorm, NeoX RoPE, slot-mapped
  K/V cache write) -> ``qk_norm_rope_cache``;
* ``DFlash2BeamModel.build_context_kv_weights`` and
  ``precompute_and_store_context_kv`` (``hidden_norm`` RMSNorm of the context
  states, one bf16 linear against every layer's stacked K/V rows, then every
  layer's K-norm + RoPE and K/V cache write) -> ``rms_norm``, ``context_kv``,
  ``store_context_kv``;
* ``DFlash2BeamAttention.__init__`` / ``forward`` (bias-free ``qkv_proj`` and
  ``o_proj`` around the attention) -> ``linear``, ``draft_attention``;
* ``DFlash2BeamAttention.__init__`` (every layer non-causal sliding-window
  attention, scale ``head_dim ** -0.5``, GQA) and the speculator's query block of
  one anchor plus N mask tokens per request -> ``block_attn``.

Where the pages leave a step open, the reading taken is stated in the function.
Parity pins for every function live in ``tests/test_oracle_*.py``.  Every
function is pinned there by closed forms, invariants or brute force; the
following readings are fixed by nothing on the pages (parity unpinned by the
pages, the same reading taken by the HIP library): the order of the output
multiplier and the soft cap, the bf16 rounding of the top-k key, the cache
layout, the window boundary and the query positions of the block attention,
the angle formula with a partial rotary dim and the GPT-J pairing, and the
rounding and saturation of the fp8 cache codes.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "f64_to_f32", "lm_logit_keys", "lm_topk",
    "candidate_edges", "qk_norm_rope_cache", "block_attn", "attention_window",
    "rank_projection", "candidate_edges_from_hp", "rms_norm", "context_kv", "store_context_kv",
    "linear", "draft_attention", "rope_cos_sin", "fp8_to_f64", "f64_to_fp8", "bf16_to_fp8_scaled",
]


# --------------------------------------------------------------------------
# bf16 helpers (own implementation: bit manipulation on IEEE fp32)
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: a bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round to nearest even (numpy's IEEE cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.  NaN stays a
    quiet NaN."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 -> bf16 bits (each step round to nearest even)."""
    return f32_to_bf16(f64_to_f32(x))


# --------------------------------------------------------------------------
# fp8 (OCP E4M3 "fn" and E5M2), for fp8 K/V caches
# --------------------------------------------------------------------------
FP8_FORMATS = {
    # name: (exponent bits, mantissa bits, bias, no-infinity "fn" variant)
    "e4m3": (4, 3, 7, True),    # float8_e4m3fn: S.1111.111 is NaN, no inf, max 448
    "e5m2": (5, 2, 15, False),  # float8_e5m2: IEEE-like, S.11111.00 = inf, max 57344
}


def fp8_to_f64(codes, fmt: str) -> np.ndarray:
    """Decode fp8 codes (uint8) by the format's definition: exponent field 0 is
    subnormal (m * 2^(1 - bias - mbits)), else (1 + m / 2^mbits) * 2^(e - bias)."""
    eb, mb, bias, fn = FP8_FORMATS[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sgn = (c >> 7) & 1
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    val = np.where(e == 0, m * 2.0 ** (1 - bias - mb), (1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias))
    emax = (1 << eb) - 1
    if fn:
        val = np.where((e == emax) & (m == (1 << mb) - 1), np.nan, val)
    else:
        val = np.where(e == emax, np.where(m == 0, np.inf, np.nan), val)
    return np.where(sgn == 1, -val, val)


def _fp8_positive_table(fmt: str):
    codes = np.arange(128, dtype=np.uint8)
    vals = fp8_to_f64(codes, fmt)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]  # ascending in both


def f64_to_fp8(x, fmt: str) -> np.ndarray:
    """Round to the nearest finite fp8 value (ties to the even code), saturating
    at the largest finite magnitude; NaN -> the NaN code.  Brute force over the
    format's finite values."""
    codes, vals = _fp8_positive_table(fmt)
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (codes[i] % 2 == 0))
    c = np.where(pick_hi, codes[i], codes[i - 1])
    c = np.where(a >= vals[-1], codes[-1], c)
    c = np.where(a <= 0, 0, c)
    c = c.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), c).astype(np.uint8)


def bf16_to_fp8_scaled(bits, scale: float, fmt: str) -> np.ndarray:
    """Cache code of a bf16 value under a per-layer scale: the value divided by
    the scale in fp32 (one IEEE rounding), then ``f64_to_fp8``."""
    q = bf16_to_f64(bits).astype(np.float32) / np.float32(scale)
    return f64_to_fp8(q.astype(np.float64), fmt)


# --------------------------------------------------------------------------
# LM-head top-k
# --------------------------------------------------------------------------
def lm_logit_keys(H: np.ndarray, W: np.ndarray, multiplier: float, softcap: float,
                  rows=None, vocab_chunk: int = 16384) -> np.ndarray:
    """bf16 key of every logit: ``key[t, v]`` as bf16 bits, rows ``rows`` of H.

    logit = multiplier * <H[t], W[v]> (float64 dot product of the widened bf16
    values); then, when ``softcap > 0``, ``softcap * tanh(logit / softcap)``.
    The logit is an fp32 number and the key its bf16 rounding.

    Readings (the pages show only the processor's constructor arguments):
    scale first, cap last; cap function ``c * tanh(x / c)``; the key is the
    LM head's output dtype (bf16).
    """
    Hs = H if rows is None else H[np.asarray(rows)]
    h = bf16_to_f64(Hs)
    V = W.shape[0]
    keys = np.empty((h.shape[0], V), dtype=np.uint16)
    for v0 in range(0, V, vocab_chunk):
        w = bf16_to_f64(W[v0:v0 + vocab_chunk])
        x = multiplier * (h @ w.T)
        if softcap > 0:
            x = softcap * np.tanh(x / softcap)
        keys[:, v0:v0 + w.shape[0]] = f64_to_bf16(x)
    return keys


def topk_from_keys(keys: np.ndarray, k: int):
    """Top ``k`` of each row by (key value descending, token id ascending).

    A stable full sort of every row: the plain definition of the selection,
    with the tie rule (lower token id first) deciding membership at the k-th
    place as well as the order.  -0 and +0 compare equal (they are the same
    value).  Returns (ids int32 [T,k], values fp32 [T,k]).
    """
    vals = bf16_to_f64(keys)
    T, V = vals.shape
    ids = np.empty((T, k), dtype=np.int32)
    out = np.empty((T, k), dtype=np.float32)
    col = np.arange(V)
    for t in range(T):
        order = np.lexsort((col, -vals[t]))  # last key is primary
        ids[t] = order[:k]
        out[t] = vals[t, order[:k]].astype(np.float32)
    return ids, out


def lm_topk(H, W, k: int, multiplier: float = 1.0, softcap: float = 0.0, rows=None):
    """``compute_candidates``: the top-k token ids of each hidden state under the
    shared LM head, and their logits (bf16 keys widened to fp32)."""
    return topk_from_keys(lm_logit_keys(H, W, multiplier, softcap, rows), k)


# --------------------------------------------------------------------------
# Candidate-selector edge scores
# --------------------------------------------------------------------------
def rank_projection(H, Wp) -> np.ndarray:
    """``hidden_projection``: h_p = Wp . h, the bias-free hidden -> rank linear
    layer of the selector, in float64.  ``H`` bf16 ``[T, hidden]``, ``Wp`` bf16
    ``[rank, hidden]``; returns ``[T, rank]``."""
    return bf16_to_f64(H) @ bf16_to_f64(Wp).T


def candidate_edges_from_hp(P, S, ids, U, hp, anchor) -> np.ndarray:
    """Edge scores ``E[r, p, q, c]`` (fp32, ``[requests, steps, k, k]``) from the
    projected hidden states ``hp`` (``[Rq*steps, rank]``, row ``r*steps + p``):

    pred(r, 0, q) = anchor[r] for every q, pred(r, p, q) = ids[r, p-1, q];
    E[r,p,q,c] = U[r,p,c] + sum_i P[pred,i] * h_p[i] * S[ids[r,p,c], i].

    ``P``, ``S``: bf16 ``[vocab, rank]``; ``ids`` int ``[Rq, steps, k]``;
    ``U`` fp32 ``[Rq, steps, k]``; ``anchor`` int ``[Rq]``.
    """
    Rq, St, k = ids.shape
    R = P.shape[1]
    hp = np.asarray(hp, dtype=np.float64).reshape(Rq, St, R)
    pred = np.empty_like(ids)
    pred[:, 0, :] = np.asarray(anchor)[:, None]
    pred[:, 1:, :] = ids[:, :-1, :]
    Pf = bf16_to_f64(P)
    Sf = bf16_to_f64(S)
    a = Pf[pred] * hp[:, :, None, :]          # [Rq, St, k(q), R]
    b = Sf[ids]                               # [Rq, St, k(c), R]
    bil = np.einsum("rpqi,rpci->rpqc", a, b)
    E = np.asarray(U, dtype=np.float64)[:, :, None, :] + bil
    return E.astype(np.float32)


def candidate_edges(P, S, ids, U, H, Wp, anchor) -> np.ndarray:
    """Edge scores of the selector from the hidden states ``H`` (bf16
    ``[Rq*steps, hidden]``) and the projection ``Wp`` (bf16 ``[rank, hidden]``):
    ``candidate_edges_from_hp`` of ``rank_projection(H, Wp)``."""
    return candidate_edges_from_hp(P, S, ids, U, rank_projection(H, Wp), anchor)


# --------------------------------------------------------------------------
# q/k RMSNorm + NeoX RoPE + slot-mapped K/V cache write
# --------------------------------------------------------------------------
def rope_angles(positions: np.ndarray, D: int, theta: float) -> np.ndarray:
    """angle[t, i] = pos_t * theta ** (-2 i / D), i < D/2 (float64)."""
    i = np.arange(D // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / D)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def _rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * (mean(x^2) + eps)^-1/2 * w over the last axis (plain weight w)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope_cos_sin(positions, rotary_dim: int, theta: float, table: str = "f64"):
    """cos and sin of the RoPE angles ``[T, rotary_dim/2]`` (``rope_angles``
    with the rotary dim in the exponent).  ``table="bf16"`` rounds each value
    once to bf16, as a bf16 cos/sin cache holds them; ``"f64"`` keeps them."""
    ang = rope_angles(positions, rotary_dim, theta)
    c, s = np.cos(ang), np.sin(ang)
    if table == "bf16":
        c, s = bf16_to_f64(f64_to_bf16(c)), bf16_to_f64(f64_to_bf16(s))
    elif table != "f64":
        raise ValueError(table)
    return c, s


def _rope(y: np.ndarray, c: np.ndarray, s: np.ndarray, neox: bool) -> np.ndarray:
    """Rotate the first ``rotary_dim = 2 * c.shape[-1]`` elements of the last
    axis of ``y`` by the angles whose cos / sin are ``c`` / ``s`` (broadcast
    over the axes between): NeoX pairs ``(i, i + rotary_dim/2)``, else GPT-J
    pairs ``(2i, 2i + 1)``, both with angle index i.  The remaining elements
    pass unchanged."""
    r2 = c.shape[-1]
    out = np.array(y, dtype=np.float64, copy=True)
    if neox:
        x1, x2 = y[..., :r2], y[..., r2:2 * r2]
    else:
        x1, x2 = y[..., 0:2 * r2:2], y[..., 1:2 * r2:2]
    o1 = x1 * c - x2 * s
    o2 = x2 * c + x1 * s
    if neox:
        out[..., :r2], out[..., r2:2 * r2] = o1, o2
    else:
        out[..., 0:2 * r2:2], out[..., 1:2 * r2:2] = o1, o2
    return out


def qk_norm_rope_cache(qkv, Hq: int, Hkv: int, D: int, q_w, k_w, eps: float,
                       positions, theta: float, slots=None, cache=None,
                       block_size: int = 16, rotary_dim: int | None = None,
                       neox: bool = True, table: str = "f64",
                       cache_fp8: str | None = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Draft layer's fused q/k norm + RoPE + cache write.

    ``qkv``: bf16 ``[T, (Hq + 2 Hkv) D]``, q heads, then k heads, then v heads.
    For each token and head: RMSNorm over the head (weights ``q_w``/``k_w``,
    one eps for both), then RoPE at the token's position over the first
    ``rotary_dim`` elements (default: the head dim; NeoX pairs unless
    ``neox=False``; cos/sin as ``rope_cos_sin(..., table)``), one bf16
    rounding at the output.  With a cache, token t with ``slots[t] >= 0``
    writes K' to ``cache[slot // bs, h, slot % bs, :D]`` and its V bits
    unchanged to ``[..., D:]``; negative slots write nothing.  With
    ``cache_fp8`` the cache is uint8 and holds ``bf16_to_fp8_scaled`` of k_out
    and of V (what an attention backend stores from the layer's bf16 k and v).

    Returns ``(q_out bf16 [T,Hq,D], k_out bf16 [T,Hkv,D], cache_out or None)``.
    """
    qkv = np.asarray(qkv)
    T = qkv.shape[0]
    x = bf16_to_f64(qkv).reshape(T, Hq + 2 * Hkv, D)
    c, s = rope_cos_sin(positions, D if rotary_dim is None else rotary_dim, theta, table)
    c, s = c[:, None, :], s[:, None, :]  # [T,1,rotary_dim/2]
    q = _rope(_rms_norm(x[:, :Hq], bf16_to_f64(q_w), eps), c, s, neox)
    k = _rope(_rms_norm(x[:, Hq:Hq + Hkv], bf16_to_f64(k_w), eps), c, s, neox)
    q_out = f64_to_bf16(q)
    k_out = f64_to_bf16(k)
    cache_out = None
    if cache is not None and slots is not None:
        cache_out = np.array(cache, copy=True)
        v_bits = qkv.reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:]
        k_store = k_out
        if cache_fp8 is not None:
            k_store = bf16_to_fp8_scaled(k_out, k_scale, cache_fp8)
            v_bits = bf16_to_fp8_scaled(v_bits, v_scale, cache_fp8)
        for t in range(T):
            s = int(slots[t])
            if s < 0:
                continue
            b, o = divmod(s, block_size)
            cache_out[b, :, o, :D] = k_store[t]
            cache_out[b, :, o, D:] = v_bits[t]
    return q_out, k_out, cache_out


# --------------------------------------------------------------------------
# Context K/V precompute: hidden_norm, the stacked K/V linear, store_context_kv
# --------------------------------------------------------------------------
def rms_norm(x, w, eps: float) -> np.ndarray:
    """``ops.rms_norm``: y = x * (mean(x^2) + eps)^-1/2 * w over the last axis,
    in float64 with one bf16 rounding at the output (the reading taken for every
    norm here: the pages show only the call).  ``x`` bf16 ``[..., d]``, ``w``
    bf16 ``[d]``; returns bf16 bits."""
    return f64_to_bf16(_rms_norm(bf16_to_f64(x), bf16_to_f64(w), eps))


def context_kv(context_states, hidden_norm_w, eps: float, W_ctx, L: int, Hkv: int, D: int) -> np.ndarray:
    """``precompute_and_store_context_kv`` up to the store: the ``hidden_norm``
    RMSNorm of the context states, then ``F.linear`` with the stacked K/V rows of
    every layer's ``qkv_proj`` (``W_ctx`` bf16 ``[L * 2 * Hkv * D, hidden]``, layer
    l's K rows then its V rows), the product summed in float64 and rounded once
    to the bf16 output.  Returns bf16 bits ``[num_ctx, L, 2, Hkv, D]``."""
    normed = rms_norm(context_states, hidden_norm_w, eps)
    kv = bf16_to_f64(normed) @ bf16_to_f64(W_ctx).T
    return f64_to_bf16(kv).reshape(np.asarray(context_states).shape[0], L, 2, Hkv, D)


def store_context_kv(kv, k_norm_w, eps: float, positions, theta: float, slots, caches, block_size: int = 16,
                     rotary_dim: int | None = None, neox: bool = True, table: str = "f64",
                     cache_fp8: str | None = None, k_scale=None, v_scale=None):
    """``store_context_kv``: for every layer l at once, K = the layer's K-norm
    (weights ``k_norm_w[l]``) and NeoX RoPE at the context token's position (the
    keys the drafter's queries attend to carry both, like its own keys), one
    bf16 rounding; V unchanged.  Token t with ``slots[t] >= 0`` writes them to
    ``caches[l][slot // bs, h, slot % bs, :D]`` and ``[..., D:]``; negative slots
    write nothing.

    ``kv`` bf16 ``[num_ctx, L, 2, Hkv, D]``; ``k_norm_w`` bf16 ``[L, D]``;
    ``caches`` a list of L bf16 arrays ``[blocks, Hkv, bs, 2D]``.  The RoPE
    options are those of ``qk_norm_rope_cache``.  With ``cache_fp8`` ("e4m3" or
    "e5m2") the caches are uint8 ``[blocks, Hkv, bs, 2D]`` and layer l stores
    ``bf16_to_fp8_scaled`` of its bf16 K' and V under ``k_scale[l]`` /
    ``v_scale[l]`` (reading: the value quantised is the one the bf16 cache would
    hold).  Returns the list of updated caches.
    """
    kv = np.asarray(kv)
    n, L, _, Hkv, D = kv.shape
    c, s = rope_cos_sin(positions, D if rotary_dim is None else rotary_dim, theta, table)
    c, s = c[:, None, :], s[:, None, :]  # [n, 1, rotary_dim/2]
    out = [np.array(cc, copy=True) for cc in caches]
    for l in range(L):
        k = _rope(_rms_norm(bf16_to_f64(kv[:, l, 0]), bf16_to_f64(k_norm_w[l]), eps), c, s, neox)
        k_bits = f64_to_bf16(k)
        v_bits = kv[:, l, 1]
        if cache_fp8 is not None:
            k_bits = bf16_to_fp8_scaled(k_bits, float(k_scale[l]), cache_fp8)
            v_bits = bf16_to_fp8_scaled(v_bits, float(v_scale[l]), cache_fp8)
        for t in range(n):
            slot = int(slots[t])
            if slot < 0:
                continue
            b, o = divmod(slot, block_size)
            out[l][b, :, o, :D] = k_bits[t]
            out[l][b, :, o, D:] = v_bits[t]
    return out


# --------------------------------------------------------------------------
# Non-causal sliding-window block attention over a paged cache
# --------------------------------------------------------------------------
def attention_window(seq_len: int, Lq: int, i: int, window: int):
    """Visible key positions ``[lo, hi)`` of query ``i`` of a request.

    Reading: query i (0 = the anchor) sits at position ``seq_len - Lq + i``;
    attention is non-causal inside the block, so every key of the request up to
    ``seq_len - 1`` is visible above, and the sliding window keeps the
    ``window`` keys at or before the query's position below.
    """
    pos = seq_len - Lq + i
    return max(0, pos - window + 1), seq_len


def block_attn(q, cache, block_tables, seq_lens, Lq: int, Hq: int, Hkv: int,
               D: int, block_size: int, window: int, scale: float,
               cache_fp8: str | None = None, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """``o = softmax(q K^T * scale) V`` per (request, q head, query), float64,
    over the visible keys (``attention_window``), K/V gathered through the
    block table; kv head = q head // (Hq / Hkv).  Output bf16 ``[Rq*Lq, Hq, D]``.
    With ``cache_fp8`` the cache holds fp8 codes: K = code value * k_scale,
    V = code value * v_scale.
    """
    Rq = len(seq_lens)
    group = Hq // Hkv
    qf = bf16_to_f64(q).reshape(Rq, Lq, Hq, D)
    out = np.empty((Rq, Lq, Hq, D), dtype=np.float64)
    for r in range(Rq):
        L = int(seq_lens[r])
        lo0, _ = attention_window(L, Lq, 0, window)
        kpos = np.arange(lo0, L)
        phys = np.asarray(block_tables[r])[kpos // block_size]
        rows = cache[phys, :, kpos % block_size, :]            # [nk, Hkv, 2D]
        if cache_fp8 is None:
            Kf = bf16_to_f64(rows[:, :, :D])
            Vf = bf16_to_f64(rows[:, :, D:])
        else:
            Kf = fp8_to_f64(rows[:, :, :D], cache_fp8) * k_scale
            Vf = fp8_to_f64(rows[:, :, D:], cache_fp8) * v_scale
        visible = np.zeros((Lq, len(kpos)), dtype=bool)       # [query, key]
        for i in range(Lq):
            lo, hi = attention_window(L, Lq, i, window)
            visible[i] = (kpos >= lo) & (kpos < hi)
        for kh in range(Hkv):
            Q = qf[r, :, kh * group:(kh + 1) * group, :]       # [Lq, group, D]
            s = np.einsum("igd,jd->igj", Q, Kf[:, kh, :]) * scale
            s = np.where(visible[:, None, :], s, -np.inf)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            p /= p.sum(axis=-1, keepdims=True)
            out[r, :, kh * group:(kh + 1) * group, :] = p @ Vf[:, kh, :]
    return f64_to_bf16(out.reshape(Rq * Lq, Hq, D))


# --------------------------------------------------------------------------
# The draft layer's projections and the whole attention sublayer
# --------------------------------------------------------------------------
def linear(X, W) -> np.ndarray:
    """Bias-free ``nn.Linear`` in the model dtype: ``Y = X W^T`` summed in
    float64, rounded once to bf16.  ``X`` bf16 ``[M, K]``, ``W`` bf16 ``[N, K]``
    (out x in); returns bf16 bits ``[M, N]``."""
    return f64_to_bf16(bf16_to_f64(X) @ bf16_to_f64(W).T)


def draft_attention(hidden, W_qkv, W_o, Hq: int, Hkv: int, D: int, q_w, k_w, eps: float, positions,
                    theta: float, slots, cache, block_tables, seq_lens, Lq: int, block_size: int, window: int):
    """``DFlash2BeamAttention.forward`` on the query block: ``qkv_proj`` (its
    output row is q heads, then k heads, then v heads), the fused q/k norm +
    RoPE + cache write, the non-causal window attention of the block over the
    cache (scale ``D ** -0.5``), ``o_proj``.  Returns ``(out bf16 [T, hidden],
    updated cache)``."""
    qkv = linear(hidden, W_qkv)
    q, _, cache2 = qk_norm_rope_cache(qkv, Hq, Hkv, D, q_w, k_w, eps, positions, theta, slots, cache, block_size)
    o = block_attn(q, cache2, block_tables, seq_lens, Lq, Hq, Hkv, D, block_size, window, D ** -0.5)
    return linear(np.asarray(o).reshape(len(o), Hq * D), W_o), cache2
