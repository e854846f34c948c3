/*
 * dflash.h -- C ABI of libdflash.so: the DFlash2 block-draft candidate step on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the DFlash2 drafter as the vLLM API docs of
 * `vllm.models.beam.nvidia.dflash2` describe it:
 *   - dflash_lm_topk            DFlash2BeamForCausalLM.compute_candidates and its
 *                               logits processor (scale = output_multiplier,
 *                               soft cap = final_logit_softcapping);
 *   - dflash_candidate_edges    DFlash2BeamCandidateSelector (class docstring and
 *                               forward: edge scores [requests, steps, top_k, top_k]);
 *   - dflash_lm_topk_proj       dflash_lm_topk plus the selector's hidden_projection
 *                               in the same pass over the hidden states, and
 *     dflash_candidate_edges_hp the edge scores from that projection;
 *   - dflash_qk_norm_rope_cache DFlash2BeamAttention.forward, the fused per-head
 *                               q/k RMSNorm + NeoX RoPE + slot-mapped cache write;
 *   - dflash_block_attn         DFlash2BeamAttention: non-causal sliding-window
 *                               attention of the query block over the cache
 *                               (scale head_dim ** -0.5, grouped K/V heads);
 *   - dflash_context_kv         DFlash2BeamModel.precompute_and_store_context_kv:
 *                               hidden_norm, the stacked K/V linear of every
 *                               draft layer, K-norm + RoPE and the cache writes;
 *   - dflash_linear             the draft layer's bias-free qkv_proj / o_proj.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller; bf16 tensors
 *     are passed as uint16_t bit patterns.  Tensors are dense row-major unless a
 *     stride argument says otherwise.  Every pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work on that stream: they never synchronise and never allocate.  Scratch
 *     memory comes from the caller (`ws`, sized by the *_workspace_size query),
 *     except for dflash_lm_topk_noalloc, whose scratch is a fixed device array
 *     of the library (see there).
 *   - The library keeps no state between calls; calls on different streams
 *     may run concurrently if their output buffers and workspaces differ.
 *   - Return value: a dflash_status.  On any non-OK status nothing was enqueued,
 *     except DFLASH_ERR_HIP, which reports a launch failure.
 *   - Device-side index data (token ids, slots, positions, block tables) is not
 *     validated by the host: out-of-range values are clamped or skipped on the
 *     device as each function states, so that no access leaves its buffer; the
 *     results for such entries are unspecified.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFLASH_OK = 0,
    DFLASH_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, k > vocab ... */
    DFLASH_ERR_UNSUPPORTED = 2, /* a size the library does not handle (see each call) */
    DFLASH_ERR_WORKSPACE = 3,   /* ws smaller than the *_workspace_size query */
    DFLASH_ERR_HIP = 4,         /* a HIP launch failed */
    DFLASH_ERR_SCRATCH = 5      /* a no-alloc call needs more than the library's static scratch */
} dflash_status;

/* Human-readable text of a status code (static storage). */
const char* dflash_status_string(int status);

/* Version of this library: major * 10000 + minor * 100 + patch. */
int dflash_version(void);

/* ------------------------------------------------------------------------
 * LM-head top-k (compute_candidates).
 *
 *   logit[t, v] = output_multiplier * sum_j H[t, j] * W[v, j]      (fp32 accumulate)
 *   if softcap > 0: logit = softcap * tanh(logit / softcap)         (scale, then cap)
 *   key[t, v]   = bf16(logit)   (round to nearest even)
 *   ids[t, :]   = the k token ids of largest key, sorted by key descending;
 *                 equal keys: lower token id first (this rule also decides which
 *                 ids enter at the k-th place)
 *   logits[t,:] = the keys of those ids, widened to fp32.
 *
 *   H       bf16 [T, Hd]      hidden states, row t = request * steps + step
 *   W       bf16 [V, Hd]      LM-head weight (the target's, shared)
 *   ids     int32 [T, k]      output
 *   logits  fp32  [T, k]      output
 *   ws      workspace of dflash_lm_topk_workspace_size(T, V, Hd, k) bytes
 *
 * Requirements: T, V, Hd >= 1; Hd % 8 == 0, Hd < 2^22; 1 <= k <= min(V, 64);
 * output_multiplier finite and > 0; softcap <= 0 (off) or finite.
 * The result does not depend on the stream, workspace contents or timing
 * (deterministic).
 * ---------------------------------------------------------------------- */
size_t dflash_lm_topk_workspace_size(int64_t T, int64_t V, int64_t Hd, int32_t k);
int dflash_lm_topk(const uint16_t* H, const uint16_t* W,
                   int64_t T, int64_t V, int64_t Hd, int32_t k,
                   float output_multiplier, float softcap,
                   int32_t* ids, float* logits,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dflash_lm_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and requirements
 * as dflash_lm_topk (bit-identical outputs: the same kernels), minus ws.
 *
 * The partial lists go to a device array of the library,
 * DFLASH_LM_TOPK_SCRATCH_BYTES (16 MiB) per GPU, held until the process ends.
 * The call allocates nothing.  Its first call on a device looks up that
 * device's address of the array (hipGetSymbolAddress), so call it with the
 * device of H, W, ids, logits and the stream current.  All calls on one GPU
 * share the array: calls that overlap on one GPU (different streams, or
 * threads without ordering) race and give undefined results; serialise them,
 * e.g. on one stream.  Nothing in the array needs clearing between calls.
 *
 * Returns DFLASH_ERR_SCRATCH, before anything is enqueued, when
 * dflash_lm_topk_workspace_size(T, V, Hd, k) exceeds the array (e.g. T = 8192
 * rows at k = 32 fit exactly; more do not).
 * ---------------------------------------------------------------------- */
#define DFLASH_LM_TOPK_SCRATCH_BYTES ((size_t)16 << 20)
int dflash_lm_topk_noalloc(const uint16_t* H, const uint16_t* W,
                           int64_t T, int64_t V, int64_t Hd, int32_t k,
                           float output_multiplier, float softcap,
                           int32_t* ids, float* logits, void* stream);

/* ------------------------------------------------------------------------
 * Candidate-selector edge scores (DFlash2BeamCandidateSelector).
 *
 *   hp[t, i]       = sum_j W_proj[i, j] * H[t, j]                   (fp32, not rounded)
 *   pred(r, 0, q)  = anchor[r];  pred(r, p, q) = cand_ids[r, p-1, q]  (p >= 1)
 *   edges[r,p,q,c] = unary[r,p,c]
 *                    + sum_i pred_cb[pred(r,p,q), i] * hp[r*S+p, i] * succ_cb[cand_ids[r,p,c], i]
 *
 *   pred_cb, succ_cb  bf16 [V, R]         predecessor / successor codebooks
 *   cand_ids          int32 [Rq, S, k]    candidate ids (e.g. from dflash_lm_topk)
 *   unary             fp32  [Rq, S, k]    the candidates' own logits
 *   H                 bf16  [Rq*S, Hd]    hidden states, row r*S + p
 *   W_proj            bf16  [R, Hd]       hidden -> rank projection (no bias)
 *   anchor            int32 [Rq]          token before the block (predecessor at p = 0)
 *   edges             fp32  [Rq, S, k, k] output, index order (r, p, q = predecessor, c)
 *   ws                dflash_candidate_edges_workspace_size(Rq*S, R, Hd) bytes
 *
 * Requirements: Rq, S, V >= 1; 1 <= k <= min(V, 64); R % 16 == 0, 16 <= R <= 256;
 * Hd % 8 == 0, Hd < 2^22.  Ids and anchors outside [0, V) are clamped into range.
 * Deterministic; edges[r, 0, q, :] is bit-identical for every q.
 * ---------------------------------------------------------------------- */
size_t dflash_candidate_edges_workspace_size(int64_t T, int32_t R, int64_t Hd);
int dflash_candidate_edges(const uint16_t* pred_cb, const uint16_t* succ_cb,
                           const int32_t* cand_ids, const float* unary,
                           const uint16_t* H, const uint16_t* W_proj,
                           const int32_t* anchor,
                           int64_t Rq, int32_t S, int32_t k, int64_t V, int32_t R, int64_t Hd,
                           float* edges, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The LM-head top-k of dflash_lm_topk with the selector's rank projection
 * computed in the same pass over H (the projection is the separate
 * hidden_projection linear layer of DFlash2BeamCandidateSelector; here
 * W_proj's rows are appended to the LM head's column tiles, so H is read once
 * for both):
 *
 *   ids, logits       exactly as dflash_lm_topk returns them (bit-identical)
 *   hp[t, i]          = sum_j W_proj[i, j] * H[t, j]   fp32 [T, R], not rounded
 *                       (MFMA accumulation order; no scale, cap or selection)
 *
 *   W_proj            bf16 [R, Hd]
 *   ws                dflash_lm_topk_workspace_size(T, V, Hd, k) bytes
 *
 * Requirements: those of dflash_lm_topk; 1 <= R <= 4096; W_proj and hp 16-byte
 * aligned.  Deterministic.
 * ---------------------------------------------------------------------- */
int dflash_lm_topk_proj(const uint16_t* H, const uint16_t* W,
                        int64_t T, int64_t V, int64_t Hd, int32_t k,
                        float output_multiplier, float softcap,
                        const uint16_t* W_proj, int32_t R,
                        int32_t* ids, float* logits, float* hp,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Candidate-selector edge scores from a given projection hp (fp32 [Rq*S, R],
 * e.g. from dflash_lm_topk_proj): the formula of dflash_candidate_edges with
 * hp[r*S + p, i] in place of the projection.  No workspace.
 *
 * Requirements: Rq, S, V >= 1; 1 <= k <= min(V, 64); R % 16 == 0, 16 <= R <= 256.
 * Ids and anchors outside [0, V) are clamped into range.  Deterministic;
 * edges[r, 0, q, :] is bit-identical for every q.
 * ---------------------------------------------------------------------- */
int dflash_candidate_edges_hp(const uint16_t* pred_cb, const uint16_t* succ_cb,
                              const int32_t* cand_ids, const float* unary, const float* hp,
                              const int32_t* anchor,
                              int64_t Rq, int32_t S, int32_t k, int64_t V, int32_t R,
                              float* edges, void* stream);

/* ------------------------------------------------------------------------
 * RoPE table for dflash_qk_norm_rope_cache (get_rope with NeoX pairing,
 * rotary dim = head dim):
 *   cos_sin[p, i]       = cos(p * theta^(-2i/D)),  i < D/2
 *   cos_sin[p, D/2 + i] = sin(p * theta^(-2i/D))
 * computed in fp64 on the device and rounded to fp32.
 *   cos_sin  fp32 [max_pos, D]  output
 * Requirements: max_pos >= 1, D even and >= 2, theta > 0.
 * ---------------------------------------------------------------------- */
int dflash_rope_cos_sin(float* cos_sin, int64_t max_pos, int32_t D, double theta, void* stream);

/* The same table in bf16 (the dtype of the cos/sin cache the pages' fused ops
 * assert), [max_pos, rotary_dim]: each entry computed in fp64 and rounded to
 * fp32, then to bf16 (round to nearest even each time).  For the *_ex calls
 * with table_bf16 = 1.  Requirements as dflash_rope_cos_sin. */
int dflash_rope_cos_sin_bf16(uint16_t* cos_sin, int64_t max_pos, int32_t rotary_dim, double theta,
                             void* stream);

/* ------------------------------------------------------------------------
 * Fused per-head q/k RMSNorm + NeoX RoPE + K/V cache write
 * (DFlash2BeamAttention.forward: beam_qk_norm_rope).
 *
 * For token t and head h, x = the head's D values of row t of qkv:
 *   y = x * (mean(x^2) + eps)^-1/2 * w          (w = q_w for q heads, k_w for k heads)
 *   NeoX rotation of pairs (i, i + D/2) by the angle of position positions[t]:
 *     y'[i]       = y[i] * cos - y[i+D/2] * sin
 *     y'[i + D/2] = y[i+D/2] * cos + y[i] * sin
 *   q_out[t, h, :] = bf16(y'),  k_out[t, h, :] = bf16(y')   (one rounding, fp32 inside)
 * With a cache (slots and kv_cache both non-NULL) and slots[t] >= 0:
 *   kv_cache[slot / block_size, h, slot % block_size, 0:D]  = k_out[t, h, :]
 *   kv_cache[slot / block_size, h, slot % block_size, D:2D] = v[t, h, :] (bits copied)
 * Negative slots (padding) and slots >= num_blocks * block_size write nothing.
 *
 *   qkv       bf16 [T_q, row_stride]: q heads (Hq*D), then k heads (Hkv*D),
 *             then v heads (Hkv*D) at the start of each row; row_stride >= (Hq+2Hkv)*D
 *   q_w, k_w  bf16 [D]
 *   positions int64 [T_q]  (clamped into [0, max_pos))
 *   cos_sin   fp32 [max_pos, D]  (dflash_rope_cos_sin)
 *   slots     int64 [T_q] or NULL;  kv_cache bf16 [num_blocks, Hkv, block_size, 2D] or NULL
 *             (both NULL: no cache write; exactly one NULL is INVALID_ARG)
 *   q_out     bf16 [T_q, Hq, D];  k_out bf16 [T_q, Hkv, D] or NULL
 *             (k_out may be NULL only when the cache is written)
 * Requirements: D == 128; row_stride % 8 == 0; T_q >= 1; Hq, Hkv >= 1.
 * ---------------------------------------------------------------------- */
int dflash_qk_norm_rope_cache(const uint16_t* qkv, int64_t row_stride,
                              int64_t T_q, int32_t Hq, int32_t Hkv, int32_t D,
                              const uint16_t* q_w, const uint16_t* k_w, float eps,
                              const int64_t* positions, const float* cos_sin, int64_t max_pos,
                              const int64_t* slots, uint16_t* kv_cache,
                              int64_t num_blocks, int32_t block_size,
                              uint16_t* q_out, uint16_t* k_out, void* stream);

/* ------------------------------------------------------------------------
 * Context K/V precompute for every draft layer at once
 * (DFlash2BeamModel.build_context_kv_weights, precompute_and_store_context_kv
 * and the store_context_kv op it calls):
 *   normed = bf16(x * (mean(x^2) + hidden_eps)^-1/2 * hidden_norm_w)   per row of ctx_states
 *   kv     = bf16(normed @ W_kv^T)  viewed as [num_ctx, L, 2, Hkv, D]  (fp32 accumulate)
 * then for layer l, kv head h and token t with a cache row:
 *   K = kv[t, l, 0, h, :] through the layer's K RMSNorm (weight k_norm_w[l], k_eps)
 *       and the NeoX rotation of dflash_qk_norm_rope_cache at positions[t]
 *       (fp32 inside, one bf16 rounding);
 *   caches[l][slot / block_size, h, slot % block_size, 0:D]  = K
 *   caches[l][slot / block_size, h, slot % block_size, D:2D] = kv[t, l, 1, h, :]
 * Negative slots (padding) and slots >= num_blocks * block_size write nothing.
 *
 *   ctx_states     bf16 [num_ctx, Hd]
 *   hidden_norm_w  bf16 [Hd]
 *   W_kv           bf16 [L * 2 * Hkv * D, Hd]: layer l's K rows (Hkv * D), then
 *                  its V rows, for l = 0 .. L-1 (each layer's qkv_proj rows past q)
 *   k_norm_w       bf16 [L, D]
 *   positions      int64 [num_ctx]  (clamped into [0, max_pos))
 *   cos_sin        fp32 [max_pos, D]  (dflash_rope_cos_sin)
 *   slots          int64 [num_ctx] or NULL
 *   caches         HOST array of L DEVICE pointers, each bf16
 *                  [num_blocks, Hkv, block_size, 2D] (one layer's cache), or NULL.
 *                  slots and caches are both NULL (no cache write: the linear
 *                  alone, as for a profiling run) or both non-NULL; the array
 *                  itself is read during the call only.
 *   kv_out         bf16 [num_ctx, L, 2, Hkv, D] or NULL: kv before the K norm
 *   ws             dflash_context_kv_workspace_size(num_ctx, Hd) bytes
 *                  (the normed states)
 * Requirements: D == 128; Hd % 8 == 0; 1 <= L <= 64; num_ctx, Hkv >= 1.
 * ---------------------------------------------------------------------- */
size_t dflash_context_kv_workspace_size(int64_t num_ctx, int64_t Hd);
int dflash_context_kv(const uint16_t* ctx_states, const uint16_t* hidden_norm_w, float hidden_eps,
                      const uint16_t* W_kv, int64_t num_ctx, int64_t Hd,
                      int32_t L, int32_t Hkv, int32_t D,
                      const uint16_t* k_norm_w, float k_eps,
                      const int64_t* positions, const float* cos_sin, int64_t max_pos,
                      const int64_t* slots, uint16_t* const* caches,
                      int64_t num_blocks, int32_t block_size,
                      uint16_t* kv_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Bias-free linear with a bf16 output, for the draft layer's projections
 * around its attention (DFlash2BeamAttention: qkv_proj, whose output row is
 * the q|k|v row of dflash_qk_norm_rope_cache, and o_proj on the attention
 * output):
 *   Y[m, n] = bf16( sum_k X[m, k] * W[n, k] )     (fp32 accumulate, one rounding)
 *
 *   X  bf16 [M, K]
 *   W  bf16 [N, K]   (nn.Linear's weight: out x in)
 *   Y  bf16 [M, ldy], columns 0 .. N-1 written, the rest untouched
 * Requirements: M, N, K >= 1; ldy >= N; N, K, ldy multiples of 8.
 * No workspace.
 * ---------------------------------------------------------------------- */
int dflash_linear(const uint16_t* X, const uint16_t* W, int64_t M, int64_t N, int64_t K,
                  uint16_t* Y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * RoPE options of the fused q/k op and of store_context_kv (both take the
 * head dim, the rotary dim and is_neox_style; the table the pages pass is a
 * bf16 cos/sin cache):
 *
 * dflash_qk_norm_rope_cache_ex and dflash_context_kv_ex are
 * dflash_qk_norm_rope_cache and dflash_context_kv with the rotation
 * generalised; the plain calls are the _ex calls with rotary_dim = D,
 * is_neox = 1, table_bf16 = 0.
 *   rotary_dim  the first rotary_dim elements of each head are rotated, the
 *               rest pass through after the norm; angle index i (i < rotary_dim/2)
 *               turns by pos * theta^(-2i/rotary_dim)
 *   is_neox     1: pairs (i, i + rotary_dim/2); 0: pairs (2i, 2i + 1) (GPT-J)
 *   cos_sin     [max_pos, rotary_dim]: cos of angle index i at column i, sin at
 *               rotary_dim/2 + i; fp32 (table_bf16 = 0, dflash_rope_cos_sin) or
 *               bf16 (table_bf16 = 1, dflash_rope_cos_sin_bf16)
 *   cache_fp8   the cache's dtype: 0 bf16 (as the plain calls), 1 fp8 E4M3
 *               ("fn": bias 7, max 448, no infinities), 2 fp8 E5M2 (bias 15,
 *               max 57344).  With fp8 the cache holds one byte per element
 *               ([num_blocks, Hkv, block_size, 2D] bytes) and a stored value is
 *               the bf16 value the bf16 cache would hold (K after its norm and
 *               RoPE, rounded; V as given or as the linear's bf16 output),
 *               divided by the layer's scale in fp32, rounded to the nearest
 *               fp8 value (ties to the even code) and saturated at the largest
 *               finite one; NaN -> 0x7F.
 *   kv_scale(s) DEVICE fp32: dflash_qk_norm_rope_cache_ex [2] = {k_scale,
 *               v_scale}; dflash_context_kv_ex [L, 2], layer l's pair at 2l.
 *               NULL when cache_fp8 = 0.
 * Requirements: 2 <= rotary_dim <= D, even (else INVALID_ARG); rotary_dim a
 * multiple of 16 with is_neox = 1 and of 8 with is_neox = 0 (else UNSUPPORTED);
 * is_neox, table_bf16 in {0, 1}; cache_fp8 in {0, 1, 2}, and with fp8 a cache
 * and the scales (else INVALID_ARG).  Everything else as in the plain calls.
 * ---------------------------------------------------------------------- */
int dflash_qk_norm_rope_cache_ex(const uint16_t* qkv, int64_t row_stride,
                                 int64_t T_q, int32_t Hq, int32_t Hkv, int32_t D,
                                 const uint16_t* q_w, const uint16_t* k_w, float eps,
                                 const int64_t* positions, const void* cos_sin, int64_t max_pos,
                                 int32_t rotary_dim, int32_t is_neox, int32_t table_bf16,
                                 const int64_t* slots, uint16_t* kv_cache,
                                 int64_t num_blocks, int32_t block_size,
                                 int32_t cache_fp8, const float* kv_scale,
                                 uint16_t* q_out, uint16_t* k_out, void* stream);
int dflash_context_kv_ex(const uint16_t* ctx_states, const uint16_t* hidden_norm_w, float hidden_eps,
                         const uint16_t* W_kv, int64_t num_ctx, int64_t Hd,
                         int32_t L, int32_t Hkv, int32_t D,
                         const uint16_t* k_norm_w, float k_eps,
                         const int64_t* positions, const void* cos_sin, int64_t max_pos,
                         int32_t rotary_dim, int32_t is_neox, int32_t table_bf16,
                         const int64_t* slots, uint16_t* const* caches,
                         int64_t num_blocks, int32_t block_size,
                         int32_t cache_fp8, const float* kv_scales,
                         uint16_t* kv_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Non-causal sliding-window block attention over a paged cache
 * (DFlash2BeamAttention.attn with the context K/V already in the cache).
 *
 * Request r has seq_lens[r] tokens in the cache, the last Lq of which are its
 * query block; query i (0 = the anchor) sits at position pos = seq_lens[r]-Lq+i.
 * Key j of request r is visible to query i iff  pos - window + 1 <= j < seq_lens[r]
 * (non-causal inside the block; the window keeps `window` keys at or before
 * the query).  With kv head g = h / (Hq / Hkv):
 *   out[r*Lq+i, h, :] = softmax_j(scale * q[r*Lq+i, h, :] . K[j, g, :]) @ V[j, g, :]
 * in fp32, rounded once to bf16.  K[j, g] = kv_cache[b, g, j % bs, 0:D] and
 * V[j, g] = kv_cache[b, g, j % bs, D:2D] with b = block_tables[r, j / bs].
 *
 *   q             bf16 [Rq*Lq, Hq, D]
 *   kv_cache      bf16 [num_blocks, Hkv, block_size, 2D]
 *   block_tables  int32 [Rq, max_blocks]  (entries clamped into [0, num_blocks))
 *   seq_lens      int32 [Rq]  (clamped into [0, max_blocks * block_size])
 *   out           bf16 [Rq*Lq, Hq, D]
 *   ws            dflash_block_attn_workspace_size(...) bytes (currently 0)
 * Requirements: D == 128; 1 <= Lq <= 16; Hq % Hkv == 0 with Hq / Hkv in
 * {1, 2, 4, 8}; block_size == 16; window >= 1.  A query with no visible key
 * (seq_lens[r] < Lq) gets zeros.
 * ---------------------------------------------------------------------- */
size_t dflash_block_attn_workspace_size(int64_t Rq, int32_t Lq, int32_t Hq, int32_t D);
int dflash_block_attn(const uint16_t* q, const uint16_t* kv_cache, int64_t num_blocks,
                      const int32_t* block_tables, int32_t max_blocks,
                      const int32_t* seq_lens,
                      int64_t Rq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t block_size, int32_t window, float scale,
                      uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dflash_block_attn over an fp8 cache: the same attention with
 * cache_fp8 = 1 (E4M3fn) or 2 (E5M2), kv_cache then one byte per element
 * [num_blocks, Hkv, block_size, 2D], and K[j, g] = code value * kv_scale[0],
 * V[j, g] = code value * kv_scale[1] (kv_scale a DEVICE fp32 [2]).  The codes
 * are decoded exactly (every finite fp8 value is a bf16 value); the scales are
 * applied to the scores and to the output.  cache_fp8 = 0 is dflash_block_attn
 * (kv_scale unused).  cache_fp8 outside {0, 1, 2}, or fp8 without scales, is
 * INVALID_ARG.
 * ---------------------------------------------------------------------- */
int dflash_block_attn_ex(const uint16_t* q, const void* kv_cache, int64_t num_blocks,
                         const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* seq_lens,
                         int64_t Rq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                         int32_t window, float scale, int32_t cache_fp8, const float* kv_scale,
                         uint16_t* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
