// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Scaled dot-product attention, bf16 storage, head size 64.
struct SdpaBf16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                   // [batch*heads*n_q] or null
  const int32_t* seqlens_q;     // [batch] or null
  const int32_t* seqlens_kv;    // [batch] or null
  int64_t qs_b, qs_h, qs_n;     // element strides (d stride 1)
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int batch, heads, n_q, n_kv;
  int n_qblocks;                // ceil(n_q / queries per workgroup)
  float scale_log2;             // scale * log2(e): scores go straight to exp2
  int causal;
  int window;                   // >= 0: only keys with |i - j| <= window (restricted attention)
};

// One decoding step over a key/value cache, bf16, head size 64: the n_q
// (<= 32) queries are the newest positions L_kv - n_q + i of each sequence.
// Keys are split into chunks of chunk_tiles * 64; each chunk leaves its
// unnormalised partial result in the workspace, and a second kernel merges
// the chunks.
struct SdpaDecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                   // [batch*heads*n_q] or null
  const int32_t* seqlens_kv;    // [batch] or null (= n_kv)
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int batch, heads, n_q, n_kv;
  int chunk_tiles, n_chunks;    // key tiles per chunk; chunks per (b, h)
  float scale_log2;
  float* part_o;                // [batch*heads][n_chunks][n_q][64]: sum_j 2^(s_j - m) V_j
  float* part_ml;               // [batch*heads][n_chunks][n_q][2]: shift m (log2 units), sum l
};

// Chunking of the decoding step for these sizes (the workspace depends on it).
void sdpa_decode_plan(int batch, int heads, int n_kv, int* chunk_tiles, int* n_chunks);

// Gradients of scaled dot-product attention, bf16 storage, head size 64.
struct SdpaBwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;            // forward output
  const uint16_t* dout;         // gradient of the loss with respect to o
  const float* lse;             // forward log-sum-exp [batch*heads*n_q] (natural log)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* ld;                    // workspace: lse*log2(e) [batch*heads*n_q] (+inf: no weight), then -D = -dO.O [batch*heads*n_q];
                                // written by the dQ kernel, read by the dK/dV kernel
  const int32_t* seqlens_q;
  const int32_t* seqlens_kv;
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int64_t dos_b, dos_h, dos_n;
  int64_t dqs_b, dqs_h, dqs_n;
  int64_t dks_b, dks_h, dks_n;
  int64_t dvs_b, dvs_h, dvs_n;
  int batch, heads, n_q, n_kv;
  float scale, scale_log2;
  int causal;
};

// Scaled dot-product attention, fp32 storage and arithmetic, head sizes <= 64.
struct SdpaF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* seqlens_q;
  const int32_t* seqlens_kv;
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int batch, heads, n_q, n_kv, d_k, d_v;
  float scale;
  int causal;
  int window;                   // >= 0: only keys with |i - j| <= window
};

// C[M, N] = A[M, K] . B[K, N], bf16 in, fp32 accumulate, bf16 out (RNE).
// A row-major with row stride lda; B given as up to three row-major column
// panels (B = [B0 | B1 | B2], each [K, n_panel]); C row-major with stride ldc.
struct GemmBf16Params {
  const uint16_t* a;
  const uint16_t* b[3];
  uint16_t* c;
  int64_t lda, ldc;
  int M, N, K;
  int n_panel;                  // columns per B panel (N = panels * n_panel)
};

// h = RNE(x + PE) for x [batch, n, d_model] bf16 (row strides ldx, ldh
// elements), PE the sinusoidal positional encoding of position i.
struct PeAddParams {
  const uint16_t* x;
  uint16_t* h;
  int64_t ldx, ldh;
  int batch, n, d_model;        // d_model a multiple of 8
};

// y = LayerNorm(res + a . w) over the N = d_model columns of each row: a
// [M, K] (row stride lda), w [K, N] row-major contiguous, res and y [M, N]
// (row strides ldr, ldy), gamma and beta [N]; all bf16, fp32 arithmetic.
struct GemmLnParams {
  const uint16_t* a;
  const uint16_t* w;
  const uint16_t* res;
  const uint16_t* gamma;
  const uint16_t* beta;
  uint16_t* y;
  int64_t lda, ldr, ldy;
  int M, N, K;                  // N in {256, 512, 768, 1024}, K a multiple of 16
  float eps;
};

// Enqueues kernel<<<grid, block, 0, stream>>>(p) and returns the status of
// this launch alone.  (hipGetLastError after a launch would also return an
// error left behind by any earlier call on the same host thread, made by
// another library, and blame it on this launch.)
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream, const P& p) {
  void* args[] = {const_cast<P*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

// Launchers: return hipSuccess or the launch error.  Shapes are validated by
// the caller (abi.cpp) before these are reached.
hipError_t launch_sdpa_bf16(const SdpaBf16Params& p, hipStream_t stream);
hipError_t launch_sdpa_f32(const SdpaF32Params& p, hipStream_t stream);
hipError_t launch_sdpa_decode_bf16(const SdpaDecodeParams& p, hipStream_t stream);
hipError_t launch_sdpa_bwd_bf16(const SdpaBwdParams& p, hipStream_t stream);
// The backward's fixed per-device scratch (for callers that cannot allocate):
// its size, and its device address on the current device (looked up once
// per device).
constexpr size_t kBwdScratchBytes = (size_t)16 << 20;
hipError_t bwd_scratch(void** ptr);
hipError_t launch_gemm_bf16(const GemmBf16Params& p, hipStream_t stream);
hipError_t launch_pe_add_bf16(const PeAddParams& p, hipStream_t stream);
hipError_t launch_gemm_bf16_ln(const GemmLnParams& p, hipStream_t stream);
bool gemm_bf16_main_supported(const GemmBf16Params& p);   // shapes the fast kernel takes

// Queries per workgroup of the streaming bf16 SDPA kernel.
int sdpa_bf16_block_m(int batch, int heads, int n_q);
// True when the bf16 SDPA runs one workgroup per (batch, head) with all keys
// resident in LDS (short sequences, no band).
bool sdpa_bf16_resident(int n_q, int n_kv, int window);

}  // namespace attn
