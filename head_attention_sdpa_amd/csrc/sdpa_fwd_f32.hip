// Scaled dot-product attention forward in fp32 (storage and arithmetic),
// head sizes 1..64, gfx950.
//
// O = softmax(Q K^T * scale) V per (batch, head) ("Attention Is All You Need"
// section 3.2.1, Eq. 1), causal mask and key padding as -inf at the softmax
// input (section 3.2.3; rockcohen.cc sections 5.3 and 6.3), online softmax
// with a running max (shift invariance, rockcohen.cc section 3.2).
//
// This is the full-precision path for small problems: one thread per query
// row, the query and output rows in registers, K and V rows read through the
// cache (all 64 lanes of a wave read the same key row, so each load is a
// broadcast).  Scores use fp32 FMA; exponentials use the accurate expf.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace attn {
namespace {

constexpr int DMAX = 64;

__global__ __launch_bounds__(64) void sdpa_fwd_f32_kernel(const SdpaF32Params p) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= p.n_q) return;

  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  float* orow = p.o + b * p.os_b + h * p.os_h + (int64_t)i * p.os_n;
  float* lse = p.lse ? p.lse + ((int64_t)b * p.heads + h) * p.n_q + i : nullptr;

  int jbeg = 0, jend = (i < Lq) ? Lkv : 0;
  if (p.causal) jend = min(jend, i + 1);
  if (p.window >= 0) {   // restricted attention: keys |i - j| <= window
    jbeg = max(0, i - p.window);
    jend = min(jend, i + p.window + 1);
  }

  float q[DMAX], o[DMAX];
  const float* qrow = p.q + b * p.qs_b + h * p.qs_h + (int64_t)i * p.qs_n;
#pragma unroll
  for (int c = 0; c < DMAX; ++c) {
    q[c] = (c < p.d_k && jend > jbeg) ? qrow[c] : 0.f;
    o[c] = 0.f;
  }

  const float* Kb = p.k + b * p.ks_b + h * p.ks_h;
  const float* Vb = p.v + b * p.vs_b + h * p.vs_h;
  float m = -INFINITY, l = 0.f;
  for (int j = jbeg; j < jend; ++j) {
    const float* krow = Kb + (int64_t)j * p.ks_n;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < DMAX; ++c)
      if (c < p.d_k) dot = fmaf(q[c], krow[c], dot);
    const float s = dot * p.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);   // m = -inf on the first key: alpha = 0
    const float e = expf(s - m_new);
    l = fmaf(l, alpha, e);
    const float* vrow = Vb + (int64_t)j * p.vs_n;
#pragma unroll
    for (int c = 0; c < DMAX; ++c)
      if (c < p.d_v) o[c] = fmaf(o[c], alpha, e * vrow[c]);
    m = m_new;
  }

  const bool valid = l > 0.f;
  const float inv = valid ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < DMAX; ++c)
    if (c < p.d_v) orow[c] = o[c] * inv;
  if (lse) *lse = valid ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_sdpa_f32(const SdpaF32Params& p, hipStream_t stream) {
  if (p.n_q == 0 || p.batch == 0 || p.heads == 0) return hipSuccess;
  const dim3 grid((p.n_q + 63) / 64, p.heads, p.batch);
  return launch_kernel(sdpa_fwd_f32_kernel, grid, dim3(64), stream, p);
}

}  // namespace attn
