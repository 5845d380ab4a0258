// C ABI of the attention library: host-side validation, layout bookkeeping
// and launches.  Every argument is checked before anything is enqueued, so an
// error never leaves a partial launch behind.  No allocation, no
// synchronisation, no printing.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/attn_sdpa.h"
#include "internal.h"

namespace {

using attn::GemmBf16Params;
using attn::SdpaBwdParams;
using attn::SdpaDecodeParams;
using attn::SdpaBf16Params;
using attn::SdpaF32Params;

constexpr int kMaxGrid = 0x7fffffff;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Contiguous [batch, heads, n, d] strides when s is null.
attn_strides resolve(const attn_strides* s, int heads, int n, int d) {
  if (s) return *s;
  attn_strides c;
  c.n = d;
  c.h = (int64_t)n * d;
  c.b = (int64_t)heads * n * d;
  return c;
}

bool strides_ok(const attn_strides& s) { return s.b >= 0 && s.h >= 0 && s.n >= 0; }

bool strides_aligned(const attn_strides& s, int64_t elems) {
  return s.b % elems == 0 && s.h % elems == 0 && s.n % elems == 0;
}

// The HIP error behind the last ATTN_E_HIP of this host thread.
thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip_error = (int)e;
  return ATTN_E_HIP;
}

// Shared checks of the SDPA arguments; fills the resolved strides and scale.
int check_sdpa(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
               const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
               const void* v, const attn_strides* sv, void* o, const attn_strides* so,
               float* scale, attn_mask mask, const float* lse, attn_strides out[4]) {
  if (dt != ATTN_F32 && dt != ATTN_BF16) return ATTN_E_INVALID;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL) return ATTN_E_INVALID;
  if (batch < 1 || heads < 1 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1) return ATTN_E_INVALID;
  // a tensor with no rows may be a null pointer
  if ((n_q > 0 && (!q || !o)) || (n_kv > 0 && (!k || !v))) return ATTN_E_INVALID;
  if (*scale == 0.f) *scale = 1.f / sqrtf((float)d_k);
  if (!(isfinite(*scale) && *scale > 0.f)) return ATTN_E_INVALID;
  out[0] = resolve(sq, heads, n_q, d_k);
  out[1] = resolve(sk, heads, n_kv, d_k);
  out[2] = resolve(sv, heads, n_kv, d_v);
  out[3] = resolve(so, heads, n_q, d_v);
  for (int t = 0; t < 4; ++t)
    if (!strides_ok(out[t])) return ATTN_E_INVALID;
  if (dt == ATTN_BF16) {
    if (d_k != 64 || d_v != 64) return ATTN_E_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_E_ALIGN;
    for (int t = 0; t < 4; ++t)
      if (!strides_aligned(out[t], 8)) return ATTN_E_ALIGN;
    const int64_t qblocks = ((int64_t)n_q + 127) / 128;
    if (qblocks * batch * heads > kMaxGrid) return ATTN_E_UNSUPPORTED;
    // Q/K/V rows are fetched through 32-bit buffer offsets from each (b, h)
    // slice, and rows past the lengths must fall outside the buffer range:
    // rows may not overlap and a slice (rounded up to 64 rows) must stay
    // below 2 GiB.
    if (n_kv > 1 && (out[1].n < 64 || out[2].n < 64)) return ATTN_E_UNSUPPORTED;
    if (n_q > 1 && out[0].n < 64) return ATTN_E_UNSUPPORTED;
    const int64_t rows = ((int64_t)n_kv + 63) / 64 * 64;
    const int64_t qrows = ((int64_t)n_q + 127) / 128 * 128;
    if (rows * out[1].n * 2 + 128 > 0x7fffffffLL || rows * out[2].n * 2 + 128 > 0x7fffffffLL ||
        qrows * out[0].n * 2 + 128 > 0x7fffffffLL)
      return ATTN_E_UNSUPPORTED;
  } else {
    if (d_k > 64 || d_v > 64) return ATTN_E_UNSUPPORTED;
    if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(o, 4)) return ATTN_E_ALIGN;
    if (heads > 65535 || batch > 65535) return ATTN_E_UNSUPPORTED;
  }
  if (lse && !aligned(lse, 4)) return ATTN_E_ALIGN;
  return ATTN_OK;
}

int launch_sdpa(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                const void* q, const void* k, const void* v, void* o, const attn_strides st[4],
                float scale, attn_mask mask, int window, const int32_t* lq, const int32_t* lkv,
                float* lse, hipStream_t stream) {
  if (dt == ATTN_BF16) {
    SdpaBf16Params p = {};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.seqlens_q = lq;
    p.seqlens_kv = lkv;
    p.qs_b = st[0].b; p.qs_h = st[0].h; p.qs_n = st[0].n;
    p.ks_b = st[1].b; p.ks_h = st[1].h; p.ks_n = st[1].n;
    p.vs_b = st[2].b; p.vs_h = st[2].h; p.vs_n = st[2].n;
    p.os_b = st[3].b; p.os_h = st[3].h; p.os_n = st[3].n;
    p.batch = batch; p.heads = heads; p.n_q = n_q; p.n_kv = n_kv;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.causal = mask == ATTN_MASK_CAUSAL;
    p.window = window;
    return hip_status(attn::launch_sdpa_bf16(p, stream));
  }
  SdpaF32Params p = {};
  p.q = static_cast<const float*>(q);
  p.k = static_cast<const float*>(k);
  p.v = static_cast<const float*>(v);
  p.o = static_cast<float*>(o);
  p.lse = lse;
  p.seqlens_q = lq;
  p.seqlens_kv = lkv;
  p.qs_b = st[0].b; p.qs_h = st[0].h; p.qs_n = st[0].n;
  p.ks_b = st[1].b; p.ks_h = st[1].h; p.ks_n = st[1].n;
  p.vs_b = st[2].b; p.vs_h = st[2].h; p.vs_n = st[2].n;
  p.os_b = st[3].b; p.os_h = st[3].h; p.os_n = st[3].n;
  p.batch = batch; p.heads = heads; p.n_q = n_q; p.n_kv = n_kv; p.d_k = d_k; p.d_v = d_v;
  p.scale = scale;
  p.causal = mask == ATTN_MASK_CAUSAL;
  p.window = window;
  return hip_status(attn::launch_sdpa_f32(p, stream));
}

// Workspace of the decoding step: fp32 partial O [B*H][chunks][n_q][64], then
// (m, l) pairs [B*H][chunks][n_q][2], each region 256-byte aligned.
struct DecodeLayout {
  int chunk_tiles, n_chunks;
  size_t ml_off, total_bytes;
};

size_t round256(size_t x);

DecodeLayout decode_layout(int batch, int heads, int n_q, int n_kv) {
  DecodeLayout L;
  attn::sdpa_decode_plan(batch, heads, n_kv, &L.chunk_tiles, &L.n_chunks);
  const size_t rows = (size_t)batch * heads * L.n_chunks * n_q;
  L.ml_off = round256(rows * 64 * sizeof(float));
  L.total_bytes = L.ml_off + round256(rows * 2 * sizeof(float));
  return L;
}

// Decoding-step sizes: bf16, head size 64, 1 <= n_q <= 32, grids in range.
bool decode_sizes_ok(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v, int* err) {
  if (dt != ATTN_F32 && dt != ATTN_BF16) { *err = ATTN_E_INVALID; return false; }
  if (batch < 1 || heads < 1 || n_q < 1 || n_kv < 0 || d_k < 1 || d_v < 1) {
    *err = ATTN_E_INVALID;
    return false;
  }
  if (dt != ATTN_BF16 || d_k != 64 || d_v != 64 || n_q > 32) { *err = ATTN_E_UNSUPPORTED; return false; }
  int ct, nc;
  attn::sdpa_decode_plan(batch, heads, n_kv, &ct, &nc);
  if ((int64_t)batch * heads * nc > kMaxGrid || (int64_t)batch * heads * n_q > kMaxGrid) {
    *err = ATTN_E_UNSUPPORTED;
    return false;
  }
  return true;
}

// Workspace regions of the MHA block (bf16 elements), each 256-byte aligned.
struct MhaLayout {
  size_t q_off, kv_off, o_off, total_bytes;  // byte offsets
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes of the multi-head block.  The heads split the model width:
// d_k = d_v = d_model / h ("Attention Is All You Need" section 3.2.2; the
// rockcohen.cc deep read, section 5.2), so h*d_k != d_model or h*d_v !=
// d_model is an invalid call, not an unsupported one.
bool mha_sizes_ok(attn_dtype dt, int batch, int n_q, int n_kv, int d_model, int heads, int d_k,
                  int d_v, int* err) {
  if (dt != ATTN_F32 && dt != ATTN_BF16) { *err = ATTN_E_INVALID; return false; }
  if (batch < 1 || n_q < 0 || n_kv < 0 || d_model < 1 || heads < 1 || d_k < 1 || d_v < 1 ||
      (int64_t)heads * d_k != d_model || (int64_t)heads * d_v != d_model) {
    *err = ATTN_E_INVALID;
    return false;
  }
  if (dt != ATTN_BF16 || d_k != 64 || d_v != 64) {
    *err = ATTN_E_UNSUPPORTED;
    return false;
  }
  // GEMM row counts and workspace offsets must fit the kernels' index types
  if ((int64_t)batch * n_q > kMaxGrid || (int64_t)batch * n_kv > kMaxGrid ||
      (int64_t)heads * 64 * 3 > kMaxGrid) {
    *err = ATTN_E_UNSUPPORTED;
    return false;
  }
  // The attention step reads the projections through 32-bit buffer offsets
  // within each (b, h) slice, as attn_sdpa_fwd does: the rows a launch may
  // touch (queries rounded up to 128, keys to 64) times the row stride of
  // the workspace layout (3*h*64 elements for self-attention's fused
  // [Q | K | V]; h*64 and 2*h*64 for cross-attention, bounded by the
  // former) must stay below 2 GiB, and the grid must fit.
  const int64_t row_bytes = 3LL * heads * 64 * 2;
  const int64_t qrows = ((int64_t)n_q + 127) / 128 * 128, krows = ((int64_t)n_kv + 63) / 64 * 64;
  if (qrows * row_bytes + 128 > 0x7fffffffLL || krows * row_bytes + 128 > 0x7fffffffLL ||
      ((int64_t)n_q + 127) / 128 * batch * heads > kMaxGrid) {
    *err = ATTN_E_UNSUPPORTED;
    return false;
  }
  return true;
}

MhaLayout mha_layout(int batch, int n_q, int n_kv, int heads) {
  const size_t hd = (size_t)heads * 64;
  MhaLayout L;
  L.q_off = 0;                                                   // Q  [B*n_q, H*64]
  L.kv_off = round256(L.q_off + (size_t)batch * n_q * hd * 2);   // KV [B*n_kv, 2*H*64]
  L.o_off = round256(L.kv_off + (size_t)batch * n_kv * 2 * hd * 2);  // Ocat [B*n_q, H*64]
  L.total_bytes = round256(L.o_off + (size_t)batch * n_q * hd * 2);
  return L;
}

// Backward sizes: bf16, head size 64, grids and the workspace offsets in range.
bool bwd_sizes_ok(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v, int* err) {
  if (dt != ATTN_F32 && dt != ATTN_BF16) { *err = ATTN_E_INVALID; return false; }
  if (batch < 1 || heads < 1 || n_q < 0 || n_kv < 0 || d_k < 1 || d_v < 1) {
    *err = ATTN_E_INVALID;
    return false;
  }
  if (dt != ATTN_BF16 || d_k != 64 || d_v != 64) { *err = ATTN_E_UNSUPPORTED; return false; }
  const int64_t bh = (int64_t)batch * heads;
  if (bh > kMaxGrid || ((int64_t)n_q + 127) / 128 * bh > kMaxGrid ||
      ((int64_t)n_kv + 127) / 128 * bh > kMaxGrid || (bh * n_q + 31) / 32 > kMaxGrid ||
      (int64_t)n_q * 8 > 0x7fffffffLL) {
    *err = ATTN_E_UNSUPPORTED;
    return false;
  }
  return true;
}

size_t bwd_workspace(int batch, int heads, int n_q) {
  return round256((size_t)batch * heads * n_q * 2 * sizeof(float));
}

// Steps 1-2 of the multi-head block: the Q/K/V projections of x_q and x_kv
// (one GEMM over three weight panels for self-attention) and the attention of
// every head, written as the concatenation [B*n_q, H*64] at the workspace's
// o_off.  Shapes and pointers are validated by the caller.
int mha_project_attend(int batch, int n_q, int n_kv, int d_model, int heads, const uint16_t* xq,
                       const uint16_t* xkv, bool self_attn, const void* w_q, const void* w_k,
                       const void* w_v, float scale, attn_mask mask, const int32_t* seqlens_q,
                       const int32_t* seqlens_kv, char* ws, const MhaLayout& L, hipStream_t stream) {
  uint16_t* qbuf = reinterpret_cast<uint16_t*>(ws + L.q_off);
  uint16_t* kvbuf = reinterpret_cast<uint16_t*>(ws + L.kv_off);
  uint16_t* obuf = reinterpret_cast<uint16_t*>(ws + L.o_off);
  const int hd = heads * 64;
  attn_strides st[4];
  const uint16_t *qp, *kp, *vp;
  int rc;
  if (self_attn) {
    // self-attention: one GEMM over the three weight panels,
    // [Q | K | V] = X [W^Q | W^K | W^V] -> [B*n, 3*H*64] at the start of the
    // workspace (it fits before the concatenation region)
    GemmBf16Params g = {};
    g.a = xq;
    g.b[0] = static_cast<const uint16_t*>(w_q);
    g.b[1] = static_cast<const uint16_t*>(w_k);
    g.b[2] = static_cast<const uint16_t*>(w_v);
    g.c = qbuf;
    g.lda = d_model; g.ldc = 3 * hd; g.M = batch * n_q; g.N = 3 * hd; g.K = d_model; g.n_panel = hd;
    rc = hip_status(attn::launch_gemm_bf16(g, stream));
    st[0] = attn_strides{(int64_t)n_q * 3 * hd, 64, 3 * hd};
    st[1] = st[2] = st[0];
    qp = qbuf;
    kp = qbuf + hd;
    vp = qbuf + 2 * hd;
  } else {
    // cross-attention: Q = X_q W^Q -> [B*n_q, H*64];
    // [K | V] = X_kv [W^K | W^V] -> [B*n_kv, 2*H*64]
    GemmBf16Params gq = {};
    gq.a = xq;
    gq.b[0] = static_cast<const uint16_t*>(w_q);
    gq.c = qbuf;
    gq.lda = d_model; gq.ldc = hd; gq.M = batch * n_q; gq.N = hd; gq.K = d_model; gq.n_panel = hd;
    GemmBf16Params gkv = {};
    gkv.a = xkv;
    gkv.b[0] = static_cast<const uint16_t*>(w_k);
    gkv.b[1] = static_cast<const uint16_t*>(w_v);
    gkv.c = kvbuf;
    gkv.lda = d_model; gkv.ldc = 2 * hd; gkv.M = batch * n_kv; gkv.N = 2 * hd; gkv.K = d_model;
    gkv.n_panel = hd;
    rc = hip_status(attn::launch_gemm_bf16(gq, stream));
    if (rc == ATTN_OK) rc = hip_status(attn::launch_gemm_bf16(gkv, stream));
    st[0] = attn_strides{(int64_t)n_q * hd, 64, hd};
    st[1] = attn_strides{(int64_t)n_kv * 2 * hd, 64, 2 * hd};
    st[2] = st[1];
    qp = qbuf;
    kp = kvbuf;
    vp = kvbuf + hd;
  }
  if (rc != ATTN_OK) return rc;
  // attention per head, reading the projections through strides and writing
  // the concatenation [B, n_q, H, 64] directly
  st[3] = attn_strides{(int64_t)n_q * hd, 64, hd};
  return launch_sdpa(ATTN_BF16, batch, heads, n_q, n_kv, 64, 64, qp, kp, vp, obuf, st, scale, mask, -1,
                     seqlens_q, seqlens_kv, nullptr, stream);
}

// The sublayer's extra workspace: h = x + PE [B*n_q, d_model] after the MHA
// regions (only when the encoding is added).
size_t block_h_off(const MhaLayout& L) { return L.total_bytes; }
size_t block_total(const MhaLayout& L, int batch, int n_q, int d_model, bool add_pe) {
  return L.total_bytes + (add_pe ? round256((size_t)batch * n_q * d_model * 2) : 0);
}
bool block_dmodel_ok(int d_model) {
  return d_model == 256 || d_model == 512 || d_model == 768 || d_model == 1024;
}

// The backward's checks and launches; `workspace` is the caller's buffer or
// the fixed scratch (scratch_call: already looked up and sized).
int sdpa_bwd_impl(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                  const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                  const void* v, const attn_strides* sv, const void* o, const attn_strides* so,
                  const void* dout, const attn_strides* sdo, const float* lse, void* dq,
                  const attn_strides* sdq, void* dk, const attn_strides* sdk, void* dv,
                  const attn_strides* sdv, float scale, attn_mask mask, const int32_t* seqlens_q,
                  const int32_t* seqlens_kv, bool scratch_call, void* workspace, size_t workspace_bytes,
                  attn_stream_t stream) {
  int err = ATTN_OK;
  if (!bwd_sizes_ok(dt, batch, heads, n_q, n_kv, d_k, d_v, &err)) return err;
  attn_strides st[4];
  const int rc = check_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv,
                            const_cast<void*>(o), so, &scale, mask, lse, st);
  if (rc != ATTN_OK) return rc;
  // the gradients have the shapes of q, k and v; dO that of o
  if ((n_q > 0 && (!dout || !dq || !lse)) || (n_kv > 0 && (!dk || !dv))) return ATTN_E_INVALID;
  const attn_strides s_do = resolve(sdo, heads, n_q, 64), s_dq = resolve(sdq, heads, n_q, 64);
  const attn_strides s_dk = resolve(sdk, heads, n_kv, 64), s_dv = resolve(sdv, heads, n_kv, 64);
  const attn_strides* extra[4] = {&s_do, &s_dq, &s_dk, &s_dv};
  for (const attn_strides* e : extra) {
    if (!strides_ok(*e)) return ATTN_E_INVALID;
    if (!strides_aligned(*e, 8)) return ATTN_E_ALIGN;
  }
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return ATTN_E_ALIGN;
  // dO rows stream through the same 32-bit buffer offsets as Q rows
  if (n_q > 1 && s_do.n < 64) return ATTN_E_UNSUPPORTED;
  if ((((int64_t)n_q + 127) / 128 * 128) * s_do.n * 2 + 128 > 0x7fffffffLL) return ATTN_E_UNSUPPORTED;
  if (n_q > 0) {
    if (scratch_call) {
      // the fixed scratch: sizes beyond it are rejected before any HIP call
      if (bwd_workspace(batch, heads, n_q) > attn::kBwdScratchBytes) return ATTN_E_WORKSPACE;
      if (hip_status(attn::bwd_scratch(&workspace)) != ATTN_OK) return ATTN_E_HIP;
      workspace_bytes = attn::kBwdScratchBytes;
    }
    if (!workspace || workspace_bytes < bwd_workspace(batch, heads, n_q)) return ATTN_E_WORKSPACE;
    if (!aligned(workspace, 256)) return ATTN_E_ALIGN;
  }
  if (n_q == 0 && n_kv == 0) return ATTN_OK;   // nothing to do: no launch
  SdpaBwdParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.ld = static_cast<float*>(workspace);
  p.seqlens_q = seqlens_q;
  p.seqlens_kv = seqlens_kv;
  p.qs_b = st[0].b; p.qs_h = st[0].h; p.qs_n = st[0].n;
  p.ks_b = st[1].b; p.ks_h = st[1].h; p.ks_n = st[1].n;
  p.vs_b = st[2].b; p.vs_h = st[2].h; p.vs_n = st[2].n;
  p.os_b = st[3].b; p.os_h = st[3].h; p.os_n = st[3].n;
  p.dos_b = s_do.b; p.dos_h = s_do.h; p.dos_n = s_do.n;
  p.dqs_b = s_dq.b; p.dqs_h = s_dq.h; p.dqs_n = s_dq.n;
  p.dks_b = s_dk.b; p.dks_h = s_dk.h; p.dks_n = s_dk.n;
  p.dvs_b = s_dv.b; p.dvs_h = s_dv.h; p.dvs_n = s_dv.n;
  p.batch = batch; p.heads = heads; p.n_q = n_q; p.n_kv = n_kv;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = mask == ATTN_MASK_CAUSAL;
  return hip_status(attn::launch_sdpa_bwd_bf16(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {


int attn_abi_version(void) { return ATTN_ABI_VERSION; }

int attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_hip_error_str(int hip_error) { return hipGetErrorString((hipError_t)hip_error); }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported configuration";
    case ATTN_E_ALIGN: return "misaligned pointer or stride";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int attn_sdpa_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                  const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                  const void* v, const attn_strides* sv, void* o, const attn_strides* so,
                  float scale, attn_mask mask, const int32_t* seqlens_q,
                  const int32_t* seqlens_kv, float* lse, attn_stream_t stream) {
  attn_strides st[4];
  const int rc = check_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv, o, so,
                            &scale, mask, lse, st);
  if (rc != ATTN_OK) return rc;
  return launch_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, k, v, o, st, scale, mask, -1,
                     seqlens_q, seqlens_kv, lse, static_cast<hipStream_t>(stream));
}

int attn_sdpa_window_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                         const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                         const void* v, const attn_strides* sv, void* o, const attn_strides* so,
                         float scale, attn_mask mask, int window, const int32_t* seqlens_q,
                         const int32_t* seqlens_kv, float* lse, attn_stream_t stream) {
  if (window < 0) return ATTN_E_INVALID;
  attn_strides st[4];
  const int rc = check_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv, o, so,
                            &scale, mask, lse, st);
  if (rc != ATTN_OK) return rc;
  // |i - j| <= max(n_q, n_kv) holds for every pair, so a wider radius is the
  // same call; clamping keeps the kernels' bound arithmetic (q0 + rows +
  // window) in int range
  if (window > n_q && window > n_kv) window = n_q > n_kv ? n_q : n_kv;
  return launch_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, k, v, o, st, scale, mask, window,
                     seqlens_q, seqlens_kv, lse, static_cast<hipStream_t>(stream));
}

size_t attn_mha_workspace_bytes(attn_dtype dt, int batch, int n_q, int n_kv, int d_model,
                                int heads, int d_k, int d_v) {
  int err;
  if (!mha_sizes_ok(dt, batch, n_q, n_kv, d_model, heads, d_k, d_v, &err)) return 0;
  return mha_layout(batch, n_q, n_kv, heads).total_bytes;
}

int attn_mha_fwd(attn_dtype dt, int batch, int n_q, int n_kv, int d_model, int heads, int d_k,
                 int d_v, const void* x_q, const void* x_kv, const void* w_q, const void* w_k,
                 const void* w_v, const void* w_o, void* y, float scale, attn_mask mask,
                 const int32_t* seqlens_q, const int32_t* seqlens_kv, void* workspace,
                 size_t workspace_bytes, attn_stream_t stream_) {
  int err = ATTN_OK;
  if (!mha_sizes_ok(dt, batch, n_q, n_kv, d_model, heads, d_k, d_v, &err)) return err;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL) return ATTN_E_INVALID;
  if (!x_q || (!x_kv && n_kv > 0) || !w_q || !w_k || !w_v || !w_o || !y) return ATTN_E_INVALID;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d_k);
  if (!(isfinite(scale) && scale > 0.f)) return ATTN_E_INVALID;
  const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, w_o, y};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return ATTN_E_ALIGN;
  const MhaLayout L = mha_layout(batch, n_q, n_kv, heads);
  if (!workspace || workspace_bytes < L.total_bytes) return ATTN_E_WORKSPACE;
  if (!aligned(workspace, 256)) return ATTN_E_ALIGN;

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const bool self_attn = x_kv == x_q && n_kv == n_q;
  int rc = mha_project_attend(batch, n_q, n_kv, d_model, heads, static_cast<const uint16_t*>(x_q),
                              static_cast<const uint16_t*>(x_kv), self_attn, w_q, w_k, w_v, scale, mask,
                              seqlens_q, seqlens_kv, ws, L, stream);
  if (rc != ATTN_OK) return rc;

  // 3. output projection: Y = Ocat W^O -> [B*n_q, d_model]
  const int hd = heads * 64;
  GemmBf16Params go = {};
  go.a = reinterpret_cast<const uint16_t*>(ws + L.o_off);
  go.b[0] = static_cast<const uint16_t*>(w_o);
  go.c = static_cast<uint16_t*>(y);
  go.lda = hd; go.ldc = d_model; go.M = batch * n_q; go.N = d_model; go.K = hd; go.n_panel = d_model;
  return hip_status(attn::launch_gemm_bf16(go, stream));
}

size_t attn_mha_block_workspace_bytes(attn_dtype dt, int batch, int n_q, int n_kv, int d_model,
                                      int heads, int d_k, int d_v, int add_pe) {
  int err;
  if (!mha_sizes_ok(dt, batch, n_q, n_kv, d_model, heads, d_k, d_v, &err) || !block_dmodel_ok(d_model))
    return 0;
  return block_total(mha_layout(batch, n_q, n_kv, heads), batch, n_q, d_model, add_pe != 0);
}

int attn_mha_block_fwd(attn_dtype dt, int batch, int n_q, int n_kv, int d_model, int heads, int d_k,
                       int d_v, const void* x_q, const void* x_kv, int add_pe, const void* w_q,
                       const void* w_k, const void* w_v, const void* w_o, const void* ln_gamma,
                       const void* ln_beta, float ln_eps, void* y, float scale, attn_mask mask,
                       const int32_t* seqlens_q, const int32_t* seqlens_kv, void* workspace,
                       size_t workspace_bytes, attn_stream_t stream_) {
  int err = ATTN_OK;
  if (!mha_sizes_ok(dt, batch, n_q, n_kv, d_model, heads, d_k, d_v, &err)) return err;
  if (!block_dmodel_ok(d_model)) return ATTN_E_UNSUPPORTED;
  if (mask != ATTN_MASK_NONE && mask != ATTN_MASK_CAUSAL) return ATTN_E_INVALID;
  if (!x_q || (!x_kv && n_kv > 0) || !w_q || !w_k || !w_v || !w_o || !ln_gamma || !ln_beta || !y)
    return ATTN_E_INVALID;
  const bool self_attn = x_kv == x_q;
  if (self_attn && n_kv != n_q) return ATTN_E_INVALID;
  if (add_pe != 0 && add_pe != 1) return ATTN_E_INVALID;
  if (add_pe && !self_attn) return ATTN_E_INVALID;     // the encoding belongs to the sublayer's own input
  if (!(isfinite(ln_eps) && ln_eps > 0.f)) return ATTN_E_INVALID;
  if (scale == 0.f) scale = 1.f / sqrtf((float)d_k);
  if (!(isfinite(scale) && scale > 0.f)) return ATTN_E_INVALID;
  const void* ptrs[] = {x_q, x_kv, w_q, w_k, w_v, w_o, ln_gamma, ln_beta, y};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return ATTN_E_ALIGN;
  const MhaLayout L = mha_layout(batch, n_q, n_kv, heads);
  if (!workspace || workspace_bytes < block_total(L, batch, n_q, d_model, add_pe != 0))
    return ATTN_E_WORKSPACE;
  if (!aligned(workspace, 256)) return ATTN_E_ALIGN;
  if (n_q == 0) return ATTN_OK;   // no output rows: nothing to do

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const uint16_t* h = static_cast<const uint16_t*>(x_q);
  int rc = ATTN_OK;
  if (add_pe) {
    // 0. h = x + PE, the sublayer's input and its residual
    uint16_t* hb = reinterpret_cast<uint16_t*>(ws + block_h_off(L));
    attn::PeAddParams pp = {};
    pp.x = static_cast<const uint16_t*>(x_q);
    pp.h = hb;
    pp.ldx = d_model; pp.ldh = d_model;
    pp.batch = batch; pp.n = n_q; pp.d_model = d_model;
    rc = hip_status(attn::launch_pe_add_bf16(pp, stream));
    h = hb;
  }
  if (rc != ATTN_OK) return rc;
  rc = mha_project_attend(batch, n_q, n_kv, d_model, heads, h, self_attn ? h : static_cast<const uint16_t*>(x_kv),
                          self_attn, w_q, w_k, w_v, scale, mask, seqlens_q, seqlens_kv, ws, L, stream);
  if (rc != ATTN_OK) return rc;
  // 3. y = LayerNorm(h + Ocat W^O) in the output projection's epilogue
  attn::GemmLnParams gl = {};
  gl.a = reinterpret_cast<const uint16_t*>(ws + L.o_off);
  gl.w = static_cast<const uint16_t*>(w_o);
  gl.res = h;
  gl.gamma = static_cast<const uint16_t*>(ln_gamma);
  gl.beta = static_cast<const uint16_t*>(ln_beta);
  gl.y = static_cast<uint16_t*>(y);
  gl.lda = heads * 64; gl.ldr = d_model; gl.ldy = d_model;
  gl.M = batch * n_q; gl.N = d_model; gl.K = heads * 64;
  gl.eps = ln_eps;
  return hip_status(attn::launch_gemm_bf16_ln(gl, stream));
}

int attn_linear_fwd(attn_dtype dt, int m, int k, int n, const void* x, int64_t ldx, const void* w,
                    void* y, int64_t ldy, attn_stream_t stream_) {
  if (dt != ATTN_F32 && dt != ATTN_BF16) return ATTN_E_INVALID;
  if (m < 0 || k < 1 || n < 1 || ldx < k || ldy < n) return ATTN_E_INVALID;
  if (dt != ATTN_BF16 || k % 64 != 0 || n % 8 != 0 || (int64_t)k * n * 2 >= 0x7fffffffLL)
    return ATTN_E_UNSUPPORTED;
  if (m == 0) return ATTN_OK;
  if (!x || !w || !y) return ATTN_E_INVALID;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || ldx % 8 != 0 || ldy % 8 != 0)
    return ATTN_E_ALIGN;
  if (((int64_t)m + 127) / 128 * (((int64_t)n + 127) / 128) > kMaxGrid) return ATTN_E_UNSUPPORTED;
  GemmBf16Params g = {};
  g.a = static_cast<const uint16_t*>(x);
  g.b[0] = static_cast<const uint16_t*>(w);
  g.c = static_cast<uint16_t*>(y);
  g.lda = ldx; g.ldc = ldy; g.M = m; g.N = n; g.K = k; g.n_panel = n;
  return hip_status(attn::launch_gemm_bf16(g, static_cast<hipStream_t>(stream_)));
}

size_t attn_decode_workspace_bytes(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k,
                                   int d_v) {
  int err;
  if (!decode_sizes_ok(dt, batch, heads, n_q, n_kv, d_k, d_v, &err)) return 0;
  return decode_layout(batch, heads, n_q, n_kv).total_bytes;
}

int attn_decode_fwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                    const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                    const void* v, const attn_strides* sv, void* o, const attn_strides* so, float scale,
                    const int32_t* seqlens_kv, float* lse, void* workspace, size_t workspace_bytes,
                    attn_stream_t stream) {
  if (n_q == 0 && dt == ATTN_BF16 && batch >= 1 && heads >= 1 && n_kv >= 0) return ATTN_OK;
  int err = ATTN_OK;
  if (!decode_sizes_ok(dt, batch, heads, n_q, n_kv, d_k, d_v, &err)) return err;
  attn_strides st[4];
  const int rc = check_sdpa(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv, o, so, &scale,
                            ATTN_MASK_NONE, lse, st);
  if (rc != ATTN_OK) return rc;
  const DecodeLayout L = decode_layout(batch, heads, n_q, n_kv);
  if (!workspace || workspace_bytes < L.total_bytes) return ATTN_E_WORKSPACE;
  if (!aligned(workspace, 256)) return ATTN_E_ALIGN;
  SdpaDecodeParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.seqlens_kv = seqlens_kv;
  p.qs_b = st[0].b; p.qs_h = st[0].h; p.qs_n = st[0].n;
  p.ks_b = st[1].b; p.ks_h = st[1].h; p.ks_n = st[1].n;
  p.vs_b = st[2].b; p.vs_h = st[2].h; p.vs_n = st[2].n;
  p.os_b = st[3].b; p.os_h = st[3].h; p.os_n = st[3].n;
  p.batch = batch; p.heads = heads; p.n_q = n_q; p.n_kv = n_kv;
  p.chunk_tiles = L.chunk_tiles; p.n_chunks = L.n_chunks;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.part_o = static_cast<float*>(workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ml_off);
  return hip_status(attn::launch_sdpa_decode_bf16(p, static_cast<hipStream_t>(stream)));
}

size_t attn_sdpa_bwd_workspace_bytes(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k,
                                     int d_v) {
  int err;
  if (!bwd_sizes_ok(dt, batch, heads, n_q, n_kv, d_k, d_v, &err)) return 0;
  return bwd_workspace(batch, heads, n_q);
}

int attn_sdpa_bwd(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                  const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                  const void* v, const attn_strides* sv, const void* o, const attn_strides* so,
                  const void* dout, const attn_strides* sdo, const float* lse, void* dq,
                  const attn_strides* sdq, void* dk, const attn_strides* sdk, void* dv,
                  const attn_strides* sdv, float scale, attn_mask mask, const int32_t* seqlens_q,
                  const int32_t* seqlens_kv, void* workspace, size_t workspace_bytes,
                  attn_stream_t stream) {
  return sdpa_bwd_impl(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv, o, so, dout, sdo, lse,
                       dq, sdq, dk, sdk, dv, sdv, scale, mask, seqlens_q, seqlens_kv, false, workspace,
                       workspace_bytes, stream);
}

int attn_sdpa_bwd_noalloc(attn_dtype dt, int batch, int heads, int n_q, int n_kv, int d_k, int d_v,
                          const void* q, const attn_strides* sq, const void* k, const attn_strides* sk,
                          const void* v, const attn_strides* sv, const void* o, const attn_strides* so,
                          const void* dout, const attn_strides* sdo, const float* lse, void* dq,
                          const attn_strides* sdq, void* dk, const attn_strides* sdk, void* dv,
                          const attn_strides* sdv, float scale, attn_mask mask, const int32_t* seqlens_q,
                          const int32_t* seqlens_kv, attn_stream_t stream) {
  return sdpa_bwd_impl(dt, batch, heads, n_q, n_kv, d_k, d_v, q, sq, k, sk, v, sv, o, so, dout, sdo, lse,
                       dq, sdq, dk, sdk, dv, sdv, scale, mask, seqlens_q, seqlens_kv, true, nullptr, 0,
                       stream);
}

}  // extern "C"
