/*
 * attn_sdpa.h -- C ABI of the MI355X (gfx950) attention library.
 *
 * Operations (definitions as in "Attention Is All You Need"):
 *   attn_sdpa_fwd  scaled dot-product attention, section 3.2.1, Eq. 1:
 *                  O = softmax(Q K^T * scale) V per (batch, head), scale
 *                  defaulting to 1/sqrt(d_k) (footnote 4 of the paper; the
 *                  variance argument is restated in the rockcohen.cc deep read,
 *                  section 5.1).
 *   attn_mha_fwd   multi-head attention, section 3.2.2:
 *                  Y = Concat(head_1..head_h) W^O,
 *                  head_i = Attention(X_q W_i^Q, X_kv W_i^K, X_kv W_i^V)
 *                  (restated on the vlmlib.cn summary and rockcohen.cc 5.2).
 *                  Self-attention passes x_kv == x_q; encoder-decoder
 *                  attention passes the encoder output as x_kv (section 3.2.3;
 *                  rockcohen.cc 5.3).
 *   attn_sdpa_window_fwd  restricted self-attention: each query attends only
 *                  to the keys of its neighbourhood of radius r, |i - j| <= r
 *                  (the paper's proposal for very long inputs, cost O(r n d):
 *                  section 4 and Table 1; the csdn blog, section 4.3).
 *   attn_decode_fwd one decoding step over a key/value cache: the newest
 *                  queries of each sequence attend to the cached keys up to
 *                  their own position (autoregressive generation, section
 *                  3.2.3; attention-paper-guide sections 05 and 07+; the csdn
 *                  blog, section 3.6).
 *   attn_linear_fwd one projection of that block on its own, Y = X.W (the
 *                  products X W_i^Q, X W_i^K, X W_i^V and Concat(...) W^O of
 *                  section 3.2.2; rockcohen.cc 5.2).
 *   attn_mha_block_fwd  the attention sublayer around the block, post-LN:
 *                  y = LayerNorm(h + MultiHead(h, kv, kv)), h = x (+ the
 *                  sinusoidal positional encoding), with the residual add and
 *                  LayerNorm fused into the output projection (paper sections
 *                  3.1 and 3.5 on the vlmlib.cn summary; rockcohen.cc sections
 *                  5.4 and 5.5; the LN formula on the ai-master transformer_lab
 *                  page).
 *   attn_sdpa_bwd  gradients of Eq. 1 with respect to Q, K and V for a given
 *                  gradient of O (the model is trained end to end: the
 *                  vlmlib.cn summary's training-objective paragraph;
 *                  attention-paper-guide section 05), from the chain rule
 *                  through the softmax, recomputing the weights from the
 *                  forward's lse.
 *
 * Masking.  Key j is legal for query i iff j < L_kv[b] (when key lengths are
 * given) and, with ATTN_MASK_CAUSAL, j <= i (the decoder's illegal
 * connections, set to -inf before the softmax: rockcohen.cc 5.3 and 6.3;
 * the diagonal stays legal).  Causal masking is aligned at the top-left
 * (query i, key i) for any n_q, n_kv.  Illegal keys get weight exactly 0 and
 * their K/V memory is never used in the arithmetic (it may hold NaN).  A query
 * row with no legal key, and every row i >= L_q[b] when query lengths are
 * given, is written as zeros (and its lse as -inf).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; it only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a negative attn_status is returned.
 *     Nothing is printed.  Asynchronous device faults surface at the caller's
 *     next synchronisation.
 *   - Lengths arrays are device int32 [batch]; values are clamped to [0, n].
 *   - Thread safety: calls may be made from several host threads.  The
 *     library's only host state is the per-thread value behind
 *     attn_last_hip_error and, for attn_sdpa_bwd_noalloc, the per-device
 *     address of its scratch array, looked up once under a lock.
 */
#ifndef ATTN_SDPA_H
#define ATTN_SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 8

typedef void* attn_stream_t; /* hipStream_t */

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum { ATTN_MASK_NONE = 0, ATTN_MASK_CAUSAL = 1 } attn_mask;

typedef enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* null pointer, negative size, bad enum, scale not finite/positive */
  ATTN_E_UNSUPPORTED = -2, /* valid but not implemented (head size, dtype, ...) */
  ATTN_E_ALIGN = -3,       /* pointer or stride misaligned for the vector loads */
  ATTN_E_WORKSPACE = -4,   /* workspace missing or too small */
  ATTN_E_HIP = -5          /* the HIP runtime rejected a launch */
} attn_status;

/* Element strides of a [batch, heads, n, d] tensor; the d stride is always 1.
 * Passing NULL for a strides pointer means contiguous [batch, heads, n, d]. */
typedef struct {
  int64_t b, h, n;
} attn_strides;

/*
 * attn_sdpa_fwd -- scaled dot-product attention, forward.
 *
 *   q  [batch, heads, n_q,  d_k]   o   [batch, heads, n_q, d_v]
 *   k  [batch, heads, n_kv, d_k]   lse [batch, heads, n_q] fp32, contiguous
 *   v  [batch, heads, n_kv, d_v]       (natural log of the softmax denominator,
 *                                       lse = max_j s_j + ln sum_j e^{s_j - max})
 *   dt          ATTN_BF16: q/k/v/o are bf16; products accumulate in fp32, the
 *               weights are rounded to bf16 for the P.V product, and O is
 *               rounded to bf16 once (round to nearest even).
 *               ATTN_F32: q/k/v/o are fp32, all arithmetic fp32.
 *   batch, heads >= 1; n_q, n_kv >= 0
 *   d_k, d_v    bf16: d_k = d_v = 64.  f32: 1 <= d_k, d_v <= 64.
 *   sq, sk, sv, so  element strides (NULL = contiguous); bf16 needs every
 *               stride and base pointer 16-byte aligned, row (n) strides of
 *               Q, K, V >= 64 elements (when that n > 1), and each (batch,
 *               head) slice of Q, K, V below 2 GiB; f32 needs 4-byte alignment.
 *   scale       0 means 1/sqrt(d_k); otherwise must be finite and > 0.
 *   mask        ATTN_MASK_NONE or ATTN_MASK_CAUSAL.
 *   seqlens_q   device int32 [batch] or NULL.
 *   seqlens_kv  device int32 [batch] or NULL.
 *   lse         device fp32 [batch*heads*n_q] or NULL.
 * q and o may be NULL when n_q = 0; k and v may be NULL when n_kv = 0.
 * Returns ATTN_OK or a negative attn_status.  o must not alias q, k or v.
 */
int attn_sdpa_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                  const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                  const void* v, const attn_strides* sv, void* o, const attn_strides* so,
                  float scale, attn_mask mask, const int32_t* seqlens_q,
                  const int32_t* seqlens_kv, float* lse, attn_stream_t stream);

/*
 * attn_sdpa_window_fwd -- attn_sdpa_fwd restricted to a band: key j is legal
 * for query i only if also |i - j| <= window (window >= 0; a neighbourhood of
 * 2*window + 1 positions centred on i, cut at the sequence ends; with
 * ATTN_MASK_CAUSAL the keys i - window .. i).  Every other argument and rule
 * is as for attn_sdpa_fwd; key tiles outside every query's band are never
 * read.  window < 0 gives ATTN_E_INVALID.
 */
int attn_sdpa_window_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                         const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                         const void* v, const attn_strides* sv, void* o, const attn_strides* so,
                         float scale, attn_mask mask, int window, const int32_t* seqlens_q,
                         const int32_t* seqlens_kv, float* lse, attn_stream_t stream);

/*
 * attn_mha_workspace_bytes -- workspace that attn_mha_fwd needs for these
 * sizes (projections and the head concatenation, bf16), or 0 if the sizes
 * are invalid or unsupported.
 */
size_t attn_mha_workspace_bytes(attn_dtype dt, int batch, int n_q, int n_kv, int d_model,
                                int heads, int d_k, int d_v);

/*
 * attn_mha_fwd -- multi-head attention block, forward (no bias, as in the
 * formula of section 3.2.2).
 *
 *   x_q   [batch, n_q,  d_model] bf16 (queries; the decoder side)
 *   x_kv  [batch, n_kv, d_model] bf16 (keys/values; may equal x_q; may be
 *         NULL when n_kv = 0, which gives zero attention output)
 *   w_q, w_k  [d_model, heads*d_k] row-major, Y = X.W (head h owns columns
 *             [h*d_k, (h+1)*d_k))
 *   w_v       [d_model, heads*d_v]
 *   w_o       [heads*d_v, d_model]  (row h*d_v + c of the concatenation is
 *             head h's output column c)
 *   y         [batch, n_q, d_model] bf16, written in full
 *   dt        ATTN_BF16 only; d_k = d_v = 64; d_model a multiple of 64.
 *   heads     d_model / d_k: the heads split d_model (d_k = d_v = d_model/h,
 *             section 3.2.2); heads*d_k != d_model or heads*d_v != d_model
 *             is ATTN_E_INVALID.
 *   scale, mask, seqlens_q, seqlens_kv: as in attn_sdpa_fwd (padded query
 *             rows give zero rows of y).
 *   workspace device memory of at least attn_mha_workspace_bytes(...) bytes,
 *             256-byte aligned; contents on entry are ignored.
 * All inputs must be contiguous and 16-byte aligned.  y must not alias any
 * input or the workspace.
 */
int attn_mha_fwd(attn_dtype dt, int batch, int n_q, int n_kv, int d_model, int heads, int d_k,
                 int d_v, const void* x_q, const void* x_kv, const void* w_q, const void* w_k,
                 const void* w_v, const void* w_o, void* y, float scale, attn_mask mask,
                 const int32_t* seqlens_q, const int32_t* seqlens_kv, void* workspace,
                 size_t workspace_bytes, attn_stream_t stream);

/* Human-readable name of an attn_status value (static storage). */
const char* attn_status_str(int status);

/*
 * attn_last_hip_error -- the hipError_t value behind the most recent
 * ATTN_E_HIP returned on the calling host thread (0 if none so far); it is
 * kept until the next ATTN_E_HIP on that thread.  attn_hip_error_str names
 * such a value (HIP's own description, static storage).
 */
int attn_last_hip_error(void);
const char* attn_hip_error_str(int hip_error);

/*
 * attn_decode_workspace_bytes -- workspace that attn_decode_fwd needs for
 * these sizes (fp32 partial results of the key chunks), or 0 if the sizes
 * are invalid or unsupported.
 */
size_t attn_decode_workspace_bytes(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k,
                                   int d_v);

/*
 * attn_decode_fwd -- one decoding step over a key/value cache.
 *
 * The n_q queries of sequence b are its newest positions: query i sits at
 * position P = L_kv[b] - n_q + i, where L_kv[b] = seqlens_kv[b] (clamped to
 * [0, n_kv]) or n_kv, and attends to the cached keys j <= P (the decoder's
 * causal mask, aligned at the end of the cache).  Cache rows j >= L_kv[b] are
 * never used and may hold anything.  A query with P < 0 has no legal key:
 * its row of o is zeros and its lse -inf.  n_q = 1 is plain attention of the
 * new token over the first L_kv[b] keys.
 *
 *   q  [batch, heads, n_q, 64]     o   [batch, heads, n_q, 64]
 *   k  [batch, heads, n_kv, 64]    lse [batch, heads, n_q] fp32 or NULL
 *   v  [batch, heads, n_kv, 64]        (natural log of the softmax denominator)
 *   dt          ATTN_BF16 only (ATTN_F32 gives ATTN_E_UNSUPPORTED); d_k = d_v = 64.
 *   1 <= n_q <= 32 (n_q = 0 does nothing), n_kv >= 0 (the cache capacity).
 *   sq, sk, sv, so, scale: as in attn_sdpa_fwd (strides NULL = contiguous,
 *               16-byte alignment, row strides >= 64 elements).
 *   seqlens_kv  device int32 [batch] (cache lengths including the n_q new
 *               positions) or NULL.
 *   workspace   device memory of at least attn_decode_workspace_bytes(...)
 *               bytes, 256-byte aligned; contents on entry are ignored.
 * The keys are processed in chunks of whole 64-key tiles, one wave per chunk.
 * With at most four chunks per (b, h) the chunks of a (b, h) run in one
 * workgroup and merge in LDS (the workspace is then not written); otherwise
 * they run as independent workgroups and a second kernel merges them through
 * the workspace.  o must not alias q, k, v or the workspace.  Returns ATTN_OK
 * or a negative attn_status.
 */
int attn_decode_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                    const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                    const void* v, const attn_strides* sv, void* o, const attn_strides* so, float scale,
                    const int32_t* seqlens_kv, float* lse, void* workspace, size_t workspace_bytes,
                    attn_stream_t stream);

/*
 * attn_linear_fwd -- y = x . w, no bias (one projection of the multi-head
 * block, section 3.2.2).
 *
 *   x   [m, k] bf16, row stride ldx elements (ldx >= k)
 *   w   [k, n] bf16, row-major and contiguous (row stride n): Y = X.W as in
 *       the projections of attn_mha_fwd
 *   y   [m, n] bf16, row stride ldy elements (ldy >= n); the m x n block is
 *       written in full, the rest of each row is not touched
 *   dt  ATTN_BF16 only (ATTN_F32 gives ATTN_E_UNSUPPORTED): fp32 accumulation,
 *       y rounded to bf16 once (round to nearest even).
 *   m >= 0; k >= 1 and a multiple of 64; n >= 8 and a multiple of 8
 *       (otherwise ATTN_E_UNSUPPORTED); k * n * 2 bytes below 2 GiB.
 *   x, w, y 16-byte aligned and ldx, ldy multiples of 8 (ATTN_E_ALIGN).
 *   x, w, y may be NULL when m = 0 (nothing is enqueued).
 * y must not overlap x or w.  Returns ATTN_OK or a negative attn_status.
 */
int attn_linear_fwd(attn_dtype dt, int m, int k, int n, const void* x, int64_t ldx, const void* w,
                    void* y, int64_t ldy, attn_stream_t stream);

/*
 * attn_mha_block_workspace_bytes -- workspace attn_mha_block_fwd needs: that
 * of attn_mha_fwd plus, with add_pe, h [batch, n_q, d_model] bf16; 0 when the
 * sizes are invalid or unsupported.
 */
size_t attn_mha_block_workspace_bytes(attn_dtype dt, int batch, int n_q, int n_kv, int d_model,
                                      int heads, int d_k, int d_v, int add_pe);

/*
 * attn_mha_block_fwd -- the attention sublayer of the encoder and decoder:
 *
 *   h = x_q + PE       if add_pe (PE[i][2j] = sin(i / 10000^(2j/d_model)),
 *                      PE[i][2j+1] = cos(...), position i from 0; h is rounded
 *                      to bf16 once); else h = x_q
 *   z = h + MultiHead(h, kv, kv)     kv = h when x_kv == x_q (self-attention),
 *                                    else x_kv (cross-attention)
 *   y = ln_gamma * (z - mean(z)) / sqrt(var(z) + ln_eps) + ln_beta
 *                      per position, mean and population variance over the
 *                      d_model features, z kept in fp32 (never stored)
 *
 *   x_q [batch, n_q, d_model], x_kv [batch, n_kv, d_model] (may be NULL when
 *   n_kv = 0), y [batch, n_q, d_model]; w_* as for attn_mha_fwd; ln_gamma,
 *   ln_beta [d_model]; all bf16, contiguous, 16-byte aligned.  dt = ATTN_BF16, d_k = d_v = 64,
 *   d_model in {256, 512, 768, 1024} (otherwise ATTN_E_UNSUPPORTED), heads*d_k =
 *   heads*d_v = d_model (otherwise ATTN_E_INVALID).
 *   add_pe is 0 or 1 and needs x_kv == x_q (and then n_kv == n_q); ln_eps
 *   finite and > 0; scale, mask and the lengths as for attn_mha_fwd (rows
 *   i >= L_q get the attention output 0, so their y is LayerNorm(h)).
 *   workspace: attn_mha_block_workspace_bytes(...) bytes, 256-byte aligned.
 * y must not overlap any input or the workspace.  Returns ATTN_OK or a
 * negative attn_status; nothing is enqueued on error.
 */
int attn_mha_block_fwd(attn_dtype dt, int batch, int n_q, int n_kv, int d_model, int heads, int d_k,
                       int d_v, const void* x_q, const void* x_kv, int add_pe, const void* w_q,
                       const void* w_k, const void* w_v, const void* w_o, const void* ln_gamma,
                       const void* ln_beta, float ln_eps, void* y, float scale, attn_mask mask,
                       const int32_t* seqlens_q, const int32_t* seqlens_kv, void* workspace,
                       size_t workspace_bytes, attn_stream_t stream);

/*
 * attn_sdpa_bwd_workspace_bytes -- workspace attn_sdpa_bwd needs for these
 * sizes (batch*heads*n_q*8 bytes rounded up to 256), or 0 when they are
 * invalid or unsupported.
 */
size_t attn_sdpa_bwd_workspace_bytes(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k,
                                     int d_v);

/*
 * attn_sdpa_bwd -- gradients of scaled dot-product attention.
 *
 * For a loss with gradient dO at the output of attn_sdpa_fwd (same q, k, v,
 * scale, mask and lengths), writes, per (batch, head), with P the forward's
 * weights and D_i = sum_c dO_ic O_ic:
 *   dV = P^T dO,   dS = P * (dO V^T - D),   dQ = scale dS K,   dK = scale dS^T Q.
 * P is recomputed as exp(scale q_i.k_j - lse_i), so o and lse must be the
 * outputs of that forward call.  Gradients of padded query rows (i >= L_q),
 * of rows with no legal key and of keys no query may use (j >= L_kv) are
 * written as zeros.
 *
 *   q, k, v, o, dout, dq, dk, dv   bf16 [batch, heads, n, 64], strides as for
 *               attn_sdpa_fwd (NULL = contiguous): sq for q, sk for k, sv
 *               for v, so for o, sdo for dout, sdq for dq, sdk for dk, sdv
 *               for dv.  Same alignment and size rules as attn_sdpa_fwd.
 *   lse         device fp32 [batch*heads*n_q], the forward's lse (required).
 *   dt          ATTN_BF16 only (ATTN_F32 gives ATTN_E_UNSUPPORTED): products
 *               accumulate in fp32, P and dS are rounded to bf16 for the
 *               products that consume them, dQ, dK, dV once to bf16.
 *   workspace   device memory of attn_sdpa_bwd_workspace_bytes(...) bytes,
 *               256-byte aligned; contents on entry are ignored.
 * dq, dk, dv are overwritten (not accumulated into) and must not overlap each
 * other, the inputs or the workspace.  Returns ATTN_OK or a negative
 * attn_status; nothing is enqueued on error.
 */
int attn_sdpa_bwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                  const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                  const void* v, const attn_strides* sv, const void* o, const attn_strides* so,
                  const void* dout, const attn_strides* sdo, const float* lse, void* dq,
                  const attn_strides* sdq, void* dk, const attn_strides* sdk, void* dv,
                  const attn_strides* sdv, float scale, attn_mask mask, const int32_t* seqlens_q,
                  const int32_t* seqlens_kv, void* workspace, size_t workspace_bytes,
                  attn_stream_t stream);

/*
 * attn_sdpa_bwd_noalloc -- attn_sdpa_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving or training loops, harnesses that forbid allocation).
 *
 * Same arguments, results and errors as attn_sdpa_bwd, minus workspace and
 * workspace_bytes.  The per-row terms it needs live in a fixed 16 MiB device
 * array of the library instead, one per device, held until the process ends:
 * batch * heads * n_q may be at most 2,097,152 (8 bytes per query row);
 * larger calls return ATTN_E_WORKSPACE before anything is enqueued.  The
 * array's address on the current device is looked up at the first call on
 * that device (the current device must be the one `stream` belongs to; a
 * failed lookup returns ATTN_E_HIP).  No call allocates or frees memory.
 * Every call on one device uses the same array and overwrites what an earlier
 * call left there before reading it: calls on one device whose kernels may
 * run concurrently (different streams without ordering between them) race
 * and must not be made; calls ordered on one stream are fine.
 */
int attn_sdpa_bwd_noalloc(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                          const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                          const void* v, const attn_strides* sv, const void* o, const attn_strides* so,
                          const void* dout, const attn_strides* sdo, const float* lse, void* dq,
                          const attn_strides* sdq, void* dk, const attn_strides* sdk, void* dv,
                          const attn_strides* sdv, float scale, attn_mask mask, const int32_t* seqlens_q,
                          const int32_t* seqlens_kv, attn_stream_t stream);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SDPA_H */
