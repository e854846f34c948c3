"""Seeded synthetic inputs for the DFlash2 block-draft candidate step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  The CPU oracle (``oracle/``) and the HIP library's tests
and benchmark both take their inputs from here, so the two sides see the same
bits.

Shapes follow the workloads of the DFlash2 drafter (vLLM API docs,
``vllm.models.beam.nvidia.dflash2``): hidden states ``[requests*steps,
hidden]`` through the shared LM head ``[vocab, hidden]`` (``DFlash2BeamForCausalLM``),
codebooks ``[vocab, rank]`` and a ``hidden -> rank`` projection
(``DFlash2BeamCandidateSelector.__init__``), a fused ``qkv`` row per query token
(``DFlash2BeamAttention.forward``) and a paged K/V cache.

Every bf16 tensor is returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# --------------------------------------------------------------------------
# Workload table.  Sizes are the five synthetic workloads of the candidate
# step; values the workloads leave open are marked "chosen".
# --------------------------------------------------------------------------
CONFIGS = {
    "tiny": dict(
        requests=2, steps=4, top_k=4, vocab=1024, hidden=256, rank=16,
        softcap=0.0, multiplier=1.0, seed=101,
    ),
    "mid": dict(
        requests=32, steps=8, top_k=8, vocab=32768, hidden=2048, rank=64,
        softcap=30.0, multiplier=1.0, seed=102,
        # draft-layer q/k-norm + RoPE + cache write at this size
        qk=dict(hq=16, hkv=4, head_dim=128, query_len=9, cache_slots=4096,
                block_size=16,          # chosen (same as the attention workload)
                eps=1e-6, theta=1e6,    # chosen (same as the attention workload)
                ctx_lo=512, ctx_hi=4096),  # chosen: context length per request
    ),
    "full": dict(
        requests=256, steps=16, top_k=16, vocab=151936, hidden=4096, rank=128,
        softcap=30.0, multiplier=0.5, seed=103,
    ),
    "attn": dict(
        requests=128, query_len=16, hq=32, hkv=8, head_dim=128, window=2048,
        ctx_lo=512, ctx_hi=8192, block_size=16, eps=1e-6, theta=1e6, seed=104,
    ),
    "large": dict(
        requests=512, steps=16, top_k=32, vocab=262144, hidden=5120, rank=256,
        softcap=30.0, multiplier=1.0,  # multiplier chosen: the workload names none
        seed=105, lm_mantissa_bits=4,
    ),
}

# Context K/V precompute (every draft layer's K/V of the context tokens from one
# stacked linear): the attention workload's shapes (128 requests, 16 new
# context tokens each, 8 kv heads of 128, eps 1e-6, theta 1e6, 16-token
# blocks) with the drafter's hidden size of the full candidate head.
CONTEXT_CONFIGS = {
    # sized for the CPU oracle: two row tiles (one ragged), four column tiles,
    # hidden 328 (not a multiple of 64: the K-tail path)
    "ctx_small": dict(requests=20, tokens=15, hidden=328, layers=2, hkv=2, head_dim=128,
                      ctx_lo=0, ctx_hi=3000, block_size=16, eps=1e-6, theta=1e6, seed=106),
    # many tiles over a short K (hidden 136, a K tail): 16 row tiles x 8192
    # columns, where 256-column tiles need no more rounds than 128-column ones
    "ctx_wide": dict(requests=256, tokens=16, hidden=136, layers=4, hkv=8, head_dim=128,
                     ctx_lo=0, ctx_hi=9000, block_size=16, eps=1e-6, theta=1e6, seed=108),
    "ctx": dict(requests=128, tokens=16, hidden=4096,
                layers=5,  # chosen: the pages do not give the drafter's layer count
                hkv=8, head_dim=128, ctx_lo=512, ctx_hi=8192, block_size=16, eps=1e-6, theta=1e6,
                seed=107),
}

SIGMA_W = 0.02  # N(0, 0.02) init of the LM head, codebooks and projection

_CHUNK = 1 << 22  # elements per independent random stream (fixed: results do not
                  # depend on the number of threads)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_chunks(seed: int, stream: int, n: int, sigma: float, out: np.ndarray,
                 convert=None) -> None:
    """Fill ``out`` (length ``n``) with N(0, sigma^2) draws.

    Chunk ``i`` of ``_CHUNK`` elements comes from its own PCG64 stream,
    ``SeedSequence([seed, stream, i])``, so the values are fixed by
    (seed, stream) whatever the number of threads.  ``convert`` maps a float32
    chunk to ``out``'s dtype.
    """
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, i])))
        buf = g.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            buf *= np.float32(sigma)
        out[lo:hi] = buf if convert is None else convert(buf)

    if nchunks <= 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))


def normal_f32(seed: int, stream: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """``n`` float32 draws of N(0, sigma^2) (see ``_fill_chunks``)."""
    out = np.empty(n, dtype=np.float32)
    _fill_chunks(seed, stream, n, sigma, out)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (round to nearest even), via torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_normal(seed: int, stream: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) draws rounded to bf16 (bit patterns); the float32 draws are
    the same as ``normal_f32(seed, stream, ...)``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _fill_chunks(seed, stream, n, sigma, out, convert=to_bf16_bits)
    return out.reshape(shape)


def keep_mantissa_bits(bits: np.ndarray, m: int) -> np.ndarray:
    """Round bf16 values (bit patterns) to ``m`` explicit mantissa bits, ties to
    even.  Used to make LM-head logits tie-heavy in the large-vocab workload."""
    drop = 7 - m
    if drop <= 0:
        return bits
    flat = np.ascontiguousarray(bits).reshape(-1)
    out = np.empty_like(flat)
    half = np.uint32(1 << (drop - 1))

    def part(lo: int) -> None:
        # in chunks: full-size uint32 temporaries of a 1.3 G-element weight
        # take minutes to page in
        u = flat[lo:lo + _CHUNK].astype(np.uint32)
        lsb = (u >> np.uint32(drop)) & np.uint32(1)
        r = ((u + half - np.uint32(1) + lsb) >> np.uint32(drop)) << np.uint32(drop)
        keep_special = (u & np.uint32(0x7F80)) == np.uint32(0x7F80)  # inf / nan untouched
        r = np.where(keep_special, u, r)
        out[lo:lo + _CHUNK] = (r & np.uint32(0xFFFF)).astype(np.uint16)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(part, range(0, flat.size, _CHUNK)))
    return out.reshape(np.shape(bits))


# --------------------------------------------------------------------------
# Candidate head (LM-head top-k and edge scores)
# --------------------------------------------------------------------------
def candidate_inputs(name: str, requests: int | None = None) -> dict:
    """Inputs of the LM-head top-k and the candidate edges for workload ``name``.

    Draw order (streams): 0 hidden states, 1 LM head, 2 predecessor codebook,
    3 successor codebook, 4 projection, 5 anchors, 6 candidate ids, 7 unary
    logits.  ``requests`` may shrink the batch (the first rows of the full draw
    are kept, so a smaller batch is a prefix of the full one).
    """
    c = CONFIGS[name]
    seed = c["seed"]
    R_full, S, k, V, Hd, R = (c["requests"], c["steps"], c["top_k"], c["vocab"],
                              c["hidden"], c["rank"])
    Rq = R_full if requests is None else int(requests)
    T_full = R_full * S
    H = bf16_normal(seed, 0, (T_full, Hd))[: Rq * S].copy()
    W = bf16_normal(seed, 1, (V, Hd), SIGMA_W)
    if c.get("lm_mantissa_bits"):
        W = keep_mantissa_bits(W, c["lm_mantissa_bits"])
    P = bf16_normal(seed, 2, (V, R), SIGMA_W)
    Sc = bf16_normal(seed, 3, (V, R), SIGMA_W)
    Wp = bf16_normal(seed, 4, (R, Hd), SIGMA_W)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5])))
    anchor = g.integers(0, V, size=R_full, dtype=np.int64).astype(np.int32)[:Rq].copy()
    # Candidate ids for the edge stage on its own: k distinct ids per position.
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
    ids = np.empty((R_full, S, k), dtype=np.int32)
    for t in range(R_full * S):
        ids.reshape(-1, k)[t] = g.choice(V, size=k, replace=False)
    ids = ids[:Rq].copy()
    # Unary logits: the scale of real LM-head logits (std ~ 0.02*sqrt(hidden)).
    U = normal_f32(seed, 7, R_full * S * k, SIGMA_W * math.sqrt(Hd)).reshape(R_full, S, k)[:Rq].copy()
    return dict(H=H, W=W, P=P, S=Sc, Wp=Wp, anchor=anchor, ids=ids, U=U,
                requests=Rq, steps=S, top_k=k, vocab=V, hidden=Hd, rank=R,
                softcap=c["softcap"], multiplier=c["multiplier"])


# --------------------------------------------------------------------------
# Draft-layer q/k-norm + RoPE + cache write, and block attention
# --------------------------------------------------------------------------
def _paged_layout(g: np.random.Generator, seq_lens: np.ndarray, block_size: int):
    nblk_per = (seq_lens + block_size - 1) // block_size
    total = int(nblk_per.sum())
    perm = g.permutation(total).astype(np.int32)
    max_blocks = int(nblk_per.max())
    tables = np.zeros((len(seq_lens), max_blocks), dtype=np.int32)
    off = 0
    for r, n in enumerate(nblk_per):
        tables[r, :n] = perm[off:off + n]
        off += n
    return tables, total


def attention_inputs(name: str = "attn", requests: int | None = None,
                     q_scale: float = 1.0) -> dict:
    """Paged-cache attention inputs (and the qkv rows of the query block).

    Context lengths ``ctx_r`` are uniform integers in ``[ctx_lo, ctx_hi]``; the
    query block of request r holds tokens ``ctx_r .. ctx_r+Lq-1`` and
    ``seq_lens[r] = ctx_r + Lq``.  Physical cache blocks are a random
    permutation, scattered into the block tables.  Cache K and V, the queries and
    the qkv rows are N(0,1) bf16; ``q_scale`` multiplies the queries before
    rounding (a peaked-softmax variant).
    """
    c = CONFIGS[name]
    seed = c["seed"]
    Rq_full, Lq, Hq, Hkv, D, bs = (c["requests"], c["query_len"], c["hq"], c["hkv"],
                                   c["head_dim"], c["block_size"])
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    ctx = g.integers(c["ctx_lo"], c["ctx_hi"] + 1, size=Rq_full, dtype=np.int64)
    Rq = Rq_full if requests is None else int(requests)
    ctx = ctx[:Rq].copy()
    seq = (ctx + Lq).astype(np.int32)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    tables, nblk = _paged_layout(g, seq.astype(np.int64), bs)
    cache = bf16_normal(seed, 2, (nblk, Hkv, bs, 2 * D))
    qf = normal_f32(seed, 3, Rq * Lq * Hq * D)
    if q_scale != 1.0:
        qf *= np.float32(q_scale)
    q = to_bf16_bits(qf).reshape(Rq * Lq, Hq, D)
    qkv = bf16_normal(seed, 4, (Rq * Lq, (Hq + 2 * Hkv) * D))
    gw = normal_f32(seed, 5, 2 * D, 0.1) + np.float32(1.0)
    q_w = to_bf16_bits(gw[:D])
    k_w = to_bf16_bits(gw[D:])
    positions = (ctx[:, None] + np.arange(Lq)[None, :]).reshape(-1).astype(np.int64)
    blk = tables[np.repeat(np.arange(Rq), Lq), positions // bs].astype(np.int64)
    slots = blk * bs + positions % bs
    return dict(q=q, cache=cache, block_tables=tables, seq_lens=seq, ctx=ctx,
                qkv=qkv, q_w=q_w, k_w=k_w, positions=positions, slots=slots,
                requests=Rq, query_len=Lq, hq=Hq, hkv=Hkv, head_dim=D,
                block_size=bs, window=c["window"], eps=c["eps"], theta=c["theta"],
                num_blocks=nblk, max_pos=int(positions.max()) + 1)


def qk_inputs(name: str = "mid", pad_fraction: float = 0.0) -> dict:
    """Inputs of the fused q/k-norm + RoPE + cache write for workload ``name``
    (``mid``: slots are the first ``T_q`` entries of a random permutation of the
    cache's slots; ``pad_fraction`` of them are set to -1, the skip value)."""
    c = CONFIGS[name]
    qc = c["qk"]
    seed = c["seed"] + 1000
    Rq, Lq, Hq, Hkv, D = c["requests"], qc["query_len"], qc["hq"], qc["hkv"], qc["head_dim"]
    bs = qc["block_size"]
    Tq = Rq * Lq
    qkv = bf16_normal(seed, 0, (Tq, (Hq + 2 * Hkv) * D))
    gw = normal_f32(seed, 1, 2 * D, 0.1) + np.float32(1.0)
    q_w = to_bf16_bits(gw[:D])
    k_w = to_bf16_bits(gw[D:])
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    ctx = g.integers(qc["ctx_lo"], qc["ctx_hi"], size=Rq, dtype=np.int64)
    positions = (ctx[:, None] + np.arange(Lq)[None, :]).reshape(-1).astype(np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    slots = g.permutation(qc["cache_slots"])[:Tq].astype(np.int64)
    if pad_fraction > 0:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
        pad = g.random(Tq) < pad_fraction
        slots[pad] = -1
    nblk = qc["cache_slots"] // bs
    cache = bf16_normal(seed, 5, (nblk, Hkv, bs, 2 * D))
    return dict(qkv=qkv, q_w=q_w, k_w=k_w, positions=positions, slots=slots,
                cache=cache, tokens=Tq, hq=Hq, hkv=Hkv, head_dim=D, block_size=bs,
                num_blocks=nblk, eps=qc["eps"], theta=qc["theta"],
                max_pos=int(positions.max()) + 1)


def context_kv_inputs(name: str = "ctx", pad_fraction: float = 0.0) -> dict:
    """Inputs of the context K/V precompute for workload ``name``.

    Request r has ``ctx_r`` tokens cached (uniform in ``[ctx_lo, ctx_hi]``) and
    adds ``tokens`` context tokens at positions ``ctx_r .. ctx_r + tokens - 1``;
    each token's slot comes from the request's block table (physical blocks a
    random permutation).  Context states N(0,1), W_kv N(0, 0.02), the
    hidden_norm and K-norm weights 1 + 0.1 N(0,1), all bf16.  The layer caches
    are not drawn here (a caller fills them).  ``pad_fraction`` of the slots
    are set to -1, the skip value.
    """
    c = CONTEXT_CONFIGS[name]
    seed = c["seed"]
    Rq, Lt, Hd, L, Hkv, D, bs = (c["requests"], c["tokens"], c["hidden"], c["layers"], c["hkv"],
                                 c["head_dim"], c["block_size"])
    n = Rq * Lt
    ctx_states = bf16_normal(seed, 0, (n, Hd))
    hn_w = to_bf16_bits(normal_f32(seed, 1, Hd, 0.1) + np.float32(1.0))
    W_kv = bf16_normal(seed, 2, (L * 2 * Hkv * D, Hd), SIGMA_W)
    k_norm_w = to_bf16_bits(normal_f32(seed, 3, L * D, 0.1) + np.float32(1.0)).reshape(L, D)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
    ctx = g.integers(c["ctx_lo"], c["ctx_hi"] + 1, size=Rq, dtype=np.int64)
    positions = (ctx[:, None] + np.arange(Lt)[None, :]).reshape(-1).astype(np.int64)
    # blocks holding the new tokens only: the rest of each request's table is
    # irrelevant to this step
    first = ctx // bs
    last = (ctx + Lt - 1) // bs
    nblk = int((last - first + 1).sum())
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5])))
    perm = g.permutation(nblk).astype(np.int64)
    slots = np.empty(n, dtype=np.int64)
    off = 0
    for r in range(Rq):
        nb = int(last[r] - first[r] + 1)
        p = positions[r * Lt:(r + 1) * Lt]
        slots[r * Lt:(r + 1) * Lt] = perm[off + (p // bs - first[r])] * bs + p % bs
        off += nb
    if pad_fraction > 0:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
        slots[g.random(n) < pad_fraction] = -1
    return dict(ctx_states=ctx_states, hidden_norm_w=hn_w, W_kv=W_kv, k_norm_w=k_norm_w,
                positions=positions, slots=slots, num_ctx=n, hidden=Hd, layers=L, hkv=Hkv,
                head_dim=D, block_size=bs, num_blocks=nblk, eps=c["eps"], theta=c["theta"],
                max_pos=int(positions.max()) + 1)


def draft_layer_inputs(requests: int | None = None, attn: dict | None = None) -> dict:
    """One draft attention sublayer on the attention workload's query block:
    ``attention_inputs("attn", requests)`` (or ``attn``, already drawn) plus the
    block's hidden states ``[Rq*16, 4096]`` ~ N(0, 1) and the bias-free
    projections ``W_qkv [(32 + 2*8)*128, 4096]`` and ``W_o [4096, 32*128]`` ~
    N(0, 0.02), bf16."""
    a = attention_inputs("attn", requests=requests) if attn is None else attn
    seed = CONFIGS["attn"]["seed"]
    hidden = 4096  # the drafter's hidden size (= the candidate head's)
    Hq, Hkv, D = a["hq"], a["hkv"], a["head_dim"]
    T = a["requests"] * a["query_len"]
    a = dict(a)
    a["hidden_states"] = bf16_normal(seed, 10, (T, hidden))
    a["W_qkv"] = bf16_normal(seed, 11, ((Hq + 2 * Hkv) * D, hidden), SIGMA_W)
    a["W_o"] = bf16_normal(seed, 12, (hidden, Hq * D), SIGMA_W)
    a["hidden"] = hidden
    return a
