"""Python binding of libdflash.so, the DFlash2 block-draft candidate step on
MI355X (gfx950).

Argument marshalling only: every computation runs in the HIP kernels behind the
C ABI of ``include/dflash.h``.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os

import torch

__all__ = [
    "DFlashError", "lib", "lm_topk", "lm_topk_workspace_size", "lm_topk_noalloc", "lm_topk_proj", "candidate_edges",
    "candidate_edges_workspace_size", "candidate_edges_hp", "rope_cos_sin", "qk_norm_rope_cache", "block_attn",
    "context_kv", "context_kv_workspace_size", "linear", "draft_attention", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

_c_i32, _c_i64, _c_f32, _c_f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
_c_p, _c_sz = ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "dflash_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dflash_version": (ctypes.c_int, []),
    "dflash_lm_topk_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "dflash_lm_topk": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_f32, _c_f32,
                                      _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dflash_lm_topk_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_f32, _c_f32,
                                              _c_p, _c_p, _c_p]),
    "dflash_lm_topk_proj": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32, _c_f32, _c_f32,
                                           _c_p, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dflash_candidate_edges_workspace_size": (_c_sz, [_c_i64, _c_i32, _c_i64]),
    "dflash_candidate_edges_hp": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32,
                                                 _c_i64, _c_i32, _c_p, _c_p]),
    "dflash_candidate_edges": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32,
                                              _c_i32, _c_i64, _c_i32, _c_i64, _c_p, _c_p, _c_sz, _c_p]),
    "dflash_rope_cos_sin": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_f64, _c_p]),
    "dflash_rope_cos_sin_bf16": (ctypes.c_int, [_c_p, _c_i64, _c_i32, _c_f64, _c_p]),
    "dflash_qk_norm_rope_cache_ex": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                                                    _c_f32, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                                                    _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]),
    "dflash_context_kv_ex": (ctypes.c_int, [_c_p, _c_p, _c_f32, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                            _c_p, _c_f32, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                                            _c_i64, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "dflash_qk_norm_rope_cache": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                                                 _c_f32, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_i32,
                                                 _c_p, _c_p, _c_p]),
    "dflash_block_attn_workspace_size": (_c_sz, [_c_i64, _c_i32, _c_i32, _c_i32]),
    "dflash_context_kv_workspace_size": (_c_sz, [_c_i64, _c_i64]),
    "dflash_linear": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p]),
    "dflash_context_kv": (ctypes.c_int, [_c_p, _c_p, _c_f32, _c_p, _c_i64, _c_i64, _c_i32, _c_i32, _c_i32,
                                         _c_p, _c_f32, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_i32,
                                         _c_p, _c_p, _c_sz, _c_p]),
    "dflash_block_attn": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i64, _c_i32, _c_i32,
                                         _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_sz, _c_p]),
    "dflash_block_attn_ex": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_i64, _c_i32, _c_i32,
                                            _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _c_p, _c_p, _c_p,
                                            _c_sz, _c_p]),
}

_LIB = None


class DFlashError(RuntimeError):
    """A libdflash call returned a non-OK status."""


def lib() -> ctypes.CDLL:
    """The loaded libdflash.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise DFlashError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_draft_candidate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().dflash_status_string(status).decode()
        raise DFlashError(f"{what}: status {status} ({msg})")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _on_stream(fn):
    """Run a binding call with ``stream`` (when given) as torch's current stream,
    so that the outputs and the workspace it allocates belong to the stream the
    kernels run on: the caching allocator then reuses a freed workspace only
    after the kernels queued on that stream."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kwargs):
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return call


def _workspace(nbytes: int, device, ws):
    if ws is None:
        return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    return ws


# ---------------------------------------------------------------- LM-head top-k
def lm_topk_workspace_size(T: int, V: int, Hd: int, k: int) -> int:
    return int(lib().dflash_lm_topk_workspace_size(T, V, Hd, k))


@_on_stream
def lm_topk(H: torch.Tensor, W: torch.Tensor, k: int, output_multiplier: float = 1.0,
            softcap: float = 0.0, ids: torch.Tensor | None = None,
            logits: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            stream=None):
    """Top-k token ids and logits of ``H [T, Hd]`` (bf16) under the LM head
    ``W [V, Hd]`` (bf16).  Returns ``(ids int32 [T, k], logits fp32 [T, k])``."""
    T, Hd = H.shape
    V = W.shape[0]
    if W.shape[1] != Hd:
        raise ValueError("H and W disagree on the hidden size")
    dev = H.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    logits = torch.empty((T, k), dtype=torch.float32, device=dev) if logits is None else logits
    ws = _workspace(lm_topk_workspace_size(T, V, Hd, k), dev, workspace)
    st = lib().dflash_lm_topk(_dev(H, torch.bfloat16, "H"), _dev(W, torch.bfloat16, "W"), T, V, Hd, k,
                              float(output_multiplier), float(softcap),
                              _dev(ids, torch.int32, "ids"), _dev(logits, torch.float32, "logits"),
                              ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dflash_lm_topk")
    return ids, logits


@_on_stream
def lm_topk_noalloc(H: torch.Tensor, W: torch.Tensor, k: int, output_multiplier: float = 1.0,
                    softcap: float = 0.0, ids: torch.Tensor | None = None,
                    logits: torch.Tensor | None = None, stream=None):
    """``lm_topk`` whose scratch is the library's own device array (the C call
    allocates nothing; pass ``ids`` and ``logits`` to allocate nothing here
    either).  Calls that overlap on one GPU race on that array."""
    T, Hd = H.shape
    V = W.shape[0]
    if W.shape[1] != Hd:
        raise ValueError("H and W disagree on the hidden size")
    dev = H.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    logits = torch.empty((T, k), dtype=torch.float32, device=dev) if logits is None else logits
    st = lib().dflash_lm_topk_noalloc(_dev(H, torch.bfloat16, "H"), _dev(W, torch.bfloat16, "W"), T, V, Hd, k,
                                      float(output_multiplier), float(softcap),
                                      _dev(ids, torch.int32, "ids"), _dev(logits, torch.float32, "logits"),
                                      _stream(stream))
    _check(st, "dflash_lm_topk_noalloc")
    return ids, logits


@_on_stream
def lm_topk_proj(H: torch.Tensor, W: torch.Tensor, k: int, output_multiplier: float, softcap: float,
                 W_proj: torch.Tensor, ids: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                 hp: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """``lm_topk`` plus the rank projection ``hp = H . W_proj^T`` (fp32 [T, R])
    from the same pass over H.  Returns ``(ids, logits, hp)``."""
    T, Hd = H.shape
    V = W.shape[0]
    R = W_proj.shape[0]
    if W.shape[1] != Hd or W_proj.shape[1] != Hd:
        raise ValueError("H, W and W_proj disagree on the hidden size")
    dev = H.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    logits = torch.empty((T, k), dtype=torch.float32, device=dev) if logits is None else logits
    hp = torch.empty((T, R), dtype=torch.float32, device=dev) if hp is None else hp
    ws = _workspace(lm_topk_workspace_size(T, V, Hd, k), dev, workspace)
    st = lib().dflash_lm_topk_proj(_dev(H, torch.bfloat16, "H"), _dev(W, torch.bfloat16, "W"), T, V, Hd, k,
                                   float(output_multiplier), float(softcap),
                                   _dev(W_proj, torch.bfloat16, "W_proj"), R,
                                   _dev(ids, torch.int32, "ids"), _dev(logits, torch.float32, "logits"),
                                   _dev(hp, torch.float32, "hp"),
                                   ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dflash_lm_topk_proj")
    return ids, logits, hp


# ---------------------------------------------------------------- edge scores
def candidate_edges_workspace_size(T: int, R: int, Hd: int) -> int:
    return int(lib().dflash_candidate_edges_workspace_size(T, R, Hd))


@_on_stream
def candidate_edges(pred_cb, succ_cb, cand_ids, unary, H, W_proj, anchor,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Edge scores ``[Rq, S, k, k]`` (fp32) of the candidate selector."""
    Rq, S, k = cand_ids.shape
    V, R = pred_cb.shape
    Hd = H.shape[1]
    if succ_cb.shape != (V, R) or W_proj.shape != (R, Hd) or H.shape[0] != Rq * S:
        raise ValueError("shape mismatch between codebooks, projection and hidden states")
    if unary.shape != (Rq, S, k) or anchor.shape != (Rq,):
        raise ValueError("unary must be [Rq, S, k] and anchor [Rq]")
    dev = H.device
    out = torch.empty((Rq, S, k, k), dtype=torch.float32, device=dev) if out is None else out
    ws = _workspace(candidate_edges_workspace_size(Rq * S, R, Hd), dev, workspace)
    st = lib().dflash_candidate_edges(
        _dev(pred_cb, torch.bfloat16, "pred_cb"), _dev(succ_cb, torch.bfloat16, "succ_cb"),
        _dev(cand_ids, torch.int32, "cand_ids"), _dev(unary, torch.float32, "unary"),
        _dev(H, torch.bfloat16, "H"), _dev(W_proj, torch.bfloat16, "W_proj"),
        _dev(anchor, torch.int32, "anchor"), Rq, S, k, V, R, Hd,
        _dev(out, torch.float32, "out"), ws.data_ptr(), ws.numel() * ws.element_size(),
        _stream(stream))
    _check(st, "dflash_candidate_edges")
    return out


@_on_stream
def candidate_edges_hp(pred_cb, succ_cb, cand_ids, unary, hp, anchor, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Edge scores ``[Rq, S, k, k]`` (fp32) from a given projection ``hp``
    (fp32 [Rq*S, R], e.g. from ``lm_topk_proj``)."""
    Rq, S, k = cand_ids.shape
    V, R = pred_cb.shape
    if succ_cb.shape != (V, R) or hp.shape != (Rq * S, R):
        raise ValueError("shape mismatch between codebooks and projection")
    if unary.shape != (Rq, S, k) or anchor.shape != (Rq,):
        raise ValueError("unary must be [Rq, S, k] and anchor [Rq]")
    out = torch.empty((Rq, S, k, k), dtype=torch.float32, device=hp.device) if out is None else out
    st = lib().dflash_candidate_edges_hp(
        _dev(pred_cb, torch.bfloat16, "pred_cb"), _dev(succ_cb, torch.bfloat16, "succ_cb"),
        _dev(cand_ids, torch.int32, "cand_ids"), _dev(unary, torch.float32, "unary"),
        _dev(hp, torch.float32, "hp"), _dev(anchor, torch.int32, "anchor"), Rq, S, k, V, R,
        _dev(out, torch.float32, "out"), _stream(stream))
    _check(st, "dflash_candidate_edges_hp")
    return out


# ---------------------------------------------------------------- q/k norm, RoPE, cache
@_on_stream
def rope_cos_sin(max_pos: int, D: int, theta: float, device, out=None, stream=None,
                 dtype=torch.float32) -> torch.Tensor:
    """``[max_pos, D]`` table (``D`` = the rotary dim): cos in ``[:, :D/2]``,
    sin in ``[:, D/2:]``; fp32, or bf16 with ``dtype=torch.bfloat16``."""
    out = torch.empty((max_pos, D), dtype=dtype, device=device) if out is None else out
    if dtype == torch.bfloat16:
        _check(lib().dflash_rope_cos_sin_bf16(_dev(out, torch.bfloat16, "cos_sin"), max_pos, D, float(theta),
                                              _stream(stream)), "dflash_rope_cos_sin_bf16")
    else:
        _check(lib().dflash_rope_cos_sin(_dev(out, torch.float32, "cos_sin"), max_pos, D, float(theta),
                                         _stream(stream)), "dflash_rope_cos_sin")
    return out


FP8_CODES = {None: 0, "e4m3": 1, "e5m2": 2}


def _cache_args(cache_fp8, scales, n_scales):
    """(format code, scales pointer) of the fp8 cache options; fp8 caches are
    torch.uint8 tensors and the scales a device fp32 tensor of n_scales."""
    if cache_fp8 not in FP8_CODES:
        raise ValueError("cache_fp8 must be None, 'e4m3' or 'e5m2'")
    if cache_fp8 is None:
        return 0, None
    if scales is None or scales.numel() != n_scales:
        raise ValueError(f"an fp8 cache needs {n_scales} scales")
    return FP8_CODES[cache_fp8], _dev(scales, torch.float32, "kv_scale")


def _rope_args(cos_sin, D, rotary_dim, is_neox):
    """(pointer, rotary_dim, is_neox, table_bf16) of a RoPE table argument."""
    rot = D if rotary_dim is None else int(rotary_dim)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != rot:
        raise ValueError("cos_sin must be [max_pos, rotary_dim]")
    bf = cos_sin.dtype == torch.bfloat16
    return _dev(cos_sin, torch.bfloat16 if bf else torch.float32, "cos_sin"), rot, int(bool(is_neox)), int(bf)


@_on_stream
def qk_norm_rope_cache(qkv, Hq: int, Hkv: int, D: int, q_w, k_w, eps: float, positions, cos_sin,
                       slots=None, kv_cache=None, q_out=None, k_out=None, want_k: bool = True,
                       stream=None, rotary_dim: int | None = None, is_neox: bool = True,
                       cache_fp8: str | None = None, kv_scale=None):
    """Fused per-head RMSNorm + NeoX RoPE of the q and k heads of ``qkv``
    ``[T, >= (Hq + 2 Hkv) D]`` (bf16), writing K/V into ``kv_cache`` at
    ``slots`` when both are given.  Returns ``(q_out, k_out or None)``."""
    T = qkv.shape[0]
    if qkv.dim() != 2 or qkv.stride(1) != 1:
        raise ValueError("qkv must be 2-D with unit column stride")
    dev = qkv.device
    q_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev) if q_out is None else q_out
    if want_k and k_out is None:
        k_out = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device=dev)
    if (slots is None) != (kv_cache is None):
        raise ValueError("slots and kv_cache go together")
    nblk, bs = (kv_cache.shape[0], kv_cache.shape[2]) if kv_cache is not None else (0, 0)
    if kv_cache is not None and (kv_cache.dim() != 4 or kv_cache.shape[1] != Hkv or kv_cache.shape[3] != 2 * D):
        raise ValueError("kv_cache must be [num_blocks, Hkv, block_size, 2D]")
    if qkv.dtype != torch.bfloat16 or not qkv.is_cuda:
        raise TypeError("qkv must be a bf16 device tensor")
    cs_ptr, rot, neox, tbf = _rope_args(cos_sin, D, rotary_dim, is_neox)
    f8, sc = _cache_args(cache_fp8, kv_scale, 2)
    cache_dtype = torch.uint8 if f8 else torch.bfloat16
    st = lib().dflash_qk_norm_rope_cache_ex(
        qkv.data_ptr(), qkv.stride(0), T, Hq, Hkv, D, _dev(q_w, torch.bfloat16, "q_w"),
        _dev(k_w, torch.bfloat16, "k_w"), float(eps), _dev(positions, torch.int64, "positions"),
        cs_ptr, cos_sin.shape[0], rot, neox, tbf,
        None if slots is None else _dev(slots, torch.int64, "slots"),
        None if kv_cache is None else _dev(kv_cache, cache_dtype, "kv_cache"), nblk, bs, f8, sc,
        _dev(q_out, torch.bfloat16, "q_out"), None if k_out is None else _dev(k_out, torch.bfloat16, "k_out"),
        _stream(stream))
    _check(st, "dflash_qk_norm_rope_cache_ex")
    return q_out, k_out


# ---------------------------------------------------------------- block attention
@_on_stream
def block_attn(q, kv_cache, block_tables, seq_lens, Lq: int, window: int, scale: float | None = None,
               out=None, workspace=None, stream=None, cache_fp8: str | None = None,
               kv_scale=None) -> torch.Tensor:
    """Non-causal sliding-window attention of each request's ``Lq`` queries
    ``q [Rq*Lq, Hq, D]`` over the paged cache ``[num_blocks, Hkv, bs, 2D]``
    (bf16, or uint8 fp8 codes with ``cache_fp8`` and the device ``kv_scale``
    [k_scale, v_scale])."""
    TQ, Hq, D = q.shape
    nblk, Hkv, bs, D2 = kv_cache.shape
    if D2 != 2 * D:
        raise ValueError("kv_cache last dim must be 2 * head_dim")
    Rq = seq_lens.shape[0]
    if TQ != Rq * Lq:
        raise ValueError("q must hold Lq queries per request")
    scale = D ** -0.5 if scale is None else scale
    out = torch.empty_like(q) if out is None else out
    ws = _workspace(int(lib().dflash_block_attn_workspace_size(Rq, Lq, Hq, D)), q.device, workspace)
    f8, sc = _cache_args(cache_fp8, kv_scale, 2)
    st = lib().dflash_block_attn_ex(
        _dev(q, torch.bfloat16, "q"), _dev(kv_cache, torch.uint8 if f8 else torch.bfloat16, "kv_cache"), nblk,
        _dev(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, torch.int32, "seq_lens"), Rq, Lq, Hq, Hkv, D, bs, int(window), float(scale), f8, sc,
        _dev(out, torch.bfloat16, "out"), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dflash_block_attn_ex")
    return out


# ---------------------------------------------------------------- context K/V precompute
def context_kv_workspace_size(num_ctx: int, Hd: int) -> int:
    return int(lib().dflash_context_kv_workspace_size(num_ctx, Hd))


@_on_stream
def context_kv(ctx_states, hidden_norm_w, hidden_eps: float, W_kv, L: int, Hkv: int, D: int, k_norm_w,
               k_eps: float, positions, cos_sin, slots=None, caches=None, kv_out=None, want_kv: bool = False,
               workspace=None, stream=None, rotary_dim: int | None = None, is_neox: bool = True,
               cache_fp8: str | None = None, kv_scales=None):
    """Context K/V of every draft layer: ``hidden_norm`` of ``ctx_states
    [num_ctx, Hd]`` (bf16), the stacked K/V linear ``W_kv [L*2*Hkv*D, Hd]``,
    then each layer's K-norm (``k_norm_w [L, D]``) + NeoX RoPE and the write of
    K and V into ``caches[l]`` (``[num_blocks, Hkv, bs, 2D]`` bf16) at ``slots``.
    Returns ``kv_out`` (``[num_ctx, L, 2, Hkv, D]``, the linear's output before
    the K norm) when ``want_kv`` or ``kv_out`` is given, else None."""
    n, Hd = ctx_states.shape
    if W_kv.shape != (L * 2 * Hkv * D, Hd) or k_norm_w.shape != (L, D) or hidden_norm_w.shape != (Hd,):
        raise ValueError("shape mismatch between context states, hidden_norm, W_kv and k_norm_w")
    if (slots is None) != (caches is None):
        raise ValueError("slots and caches go together")
    dev = ctx_states.device
    if want_kv and kv_out is None:
        kv_out = torch.empty((n, L, 2, Hkv, D), dtype=torch.bfloat16, device=dev)
    ptrs, nblk, bs = None, 0, 0
    if caches is not None:
        if len(caches) != L:
            raise ValueError("one cache per layer")
        c0 = caches[0]
        nblk, bs = c0.shape[0], c0.shape[2]
        for c in caches:
            if c.shape != (nblk, Hkv, bs, 2 * D):
                raise ValueError("every cache must be [num_blocks, Hkv, block_size, 2D]")
        ptrs = (ctypes.c_void_p * L)(*[_dev(c, torch.uint8 if cache_fp8 else torch.bfloat16, "cache")
                                       for c in caches])
    ws = _workspace(context_kv_workspace_size(n, Hd), dev, workspace)
    cs_ptr, rot, neox, tbf = _rope_args(cos_sin, D, rotary_dim, is_neox)
    f8, sc = _cache_args(cache_fp8, kv_scales, 2 * L)
    st = lib().dflash_context_kv_ex(
        _dev(ctx_states, torch.bfloat16, "ctx_states"), _dev(hidden_norm_w, torch.bfloat16, "hidden_norm_w"),
        float(hidden_eps), _dev(W_kv, torch.bfloat16, "W_kv"), n, Hd, L, Hkv, D,
        _dev(k_norm_w, torch.bfloat16, "k_norm_w"), float(k_eps), _dev(positions, torch.int64, "positions"),
        cs_ptr, cos_sin.shape[0], rot, neox, tbf,
        None if slots is None else _dev(slots, torch.int64, "slots"),
        None if ptrs is None else ctypes.cast(ptrs, ctypes.c_void_p), nblk, bs, f8, sc,
        None if kv_out is None else _dev(kv_out, torch.bfloat16, "kv_out"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "dflash_context_kv_ex")
    return kv_out


# ---------------------------------------------------------------- draft-layer projections
@_on_stream
def linear(X, W, out=None, stream=None) -> torch.Tensor:
    """``bf16(X [M, K] . W [N, K]^T)`` (bias-free nn.Linear, fp32 accumulate)."""
    if X.dim() != 2 or W.dim() != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("X must be [M, K] and W [N, K]")
    M, K = X.shape
    N = W.shape[0]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device) if out is None else out
    if out.dim() != 2 or out.shape[0] != M or out.shape[1] < N or out.stride(1) != 1 or out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 [M, >= N] with unit column stride")
    st = lib().dflash_linear(_dev(X, torch.bfloat16, "X"), _dev(W, torch.bfloat16, "W"), M, N, K, out.data_ptr(),
                             out.stride(0), _stream(stream))
    _check(st, "dflash_linear")
    return out


@_on_stream
def draft_attention(hidden, W_qkv, W_o, Hq: int, Hkv: int, D: int, q_w, k_w, eps: float, positions, cos_sin,
                    slots, kv_cache, block_tables, seq_lens, Lq: int, window: int, stream=None) -> torch.Tensor:
    """One draft attention sublayer (DFlash2BeamAttention.forward) on the
    query block: ``qkv_proj``, the fused q/k norm + RoPE + cache write, the
    non-causal window attention over the cache, ``o_proj``.  Four calls into the
    library; returns ``[T, hidden]`` bf16."""
    T = hidden.shape[0]
    qkv = linear(hidden, W_qkv, stream=stream)
    q, _ = qk_norm_rope_cache(qkv, Hq, Hkv, D, q_w, k_w, eps, positions, cos_sin, slots, kv_cache,
                              want_k=False, stream=stream)
    o = block_attn(q, kv_cache, block_tables, seq_lens, Lq, window, stream=stream)
    return linear(o.view(T, Hq * D), W_o, stream=stream)
