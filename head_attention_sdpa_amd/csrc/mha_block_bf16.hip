// The attention sublayer around the multi-head block, gfx950:
//   h = x + PE                    (sinusoidal positional encoding, paper
//                                  section 3.5 on the vlmlib.cn summary and
//                                  rockcohen.cc section 5.4)
//   y = LayerNorm(h + Concat(heads) W^O)
//                                 (post-LN sublayer, paper section 3.1 on the
//                                  vlmlib.cn summary; LN as on the ai-master
//                                  transformer_lab page: gamma (z - mean) /
//                                  sqrt(var + eps) + beta over the d_model
//                                  features of one position)
//
// pe_add_bf16: one thread per (position, 8 columns) computes the 8 encoding
//   values once (angle pos * 10000^(-2i/d) in fp64, reduced to [-pi, pi],
//   then fp32 sine/cosine) and adds them to that position of every sequence,
//   one RNE rounding to bf16.
// gemm_bf16_ln_kernel: the W^O product with the residual add and LayerNorm in
//   its epilogue.  A workgroup owns 64 whole output rows (all d_model <= 1024
//   columns), so the row statistics never leave the chip: 8 waves, wave w the
//   columns [w*d/8, (w+1)*d/8) of all 64 rows (d/8 = 32*NB).  K advances 32 at
//   a time; the Ocat slice [64][32] and the W^O slice [32][d] of a step are
//   copied global -> LDS by buffer_load ... lds into a 2-stage ring.  The
//   product runs transposed (D = W^T . Ocat^T on MFMA 32x32x16 bf16), W read
//   with ds_read_b64_tr_b16, so each accumulator lane holds one output row and
//   4 consecutive columns per register group.  Epilogue: the residual tile
//   arrives in the idle ring by LDS DMA, z = acc + h in fp32, the row mean and
//   then the mean squared deviation (two passes, each a lane sum, a
//   partner-lane sum and an 8-wave sum through LDS), y = gamma (z - mean) /
//   sqrt(var + eps) + beta rounded once to bf16 and written as whole rows.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pe_add_bf16(const PeAddParams p) {
  const int d8 = p.d_model / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)p.n * d8) return;
  const int pos = (int)(t / d8), c0 = (int)(t - (int64_t)pos * d8) * 8;
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  constexpr double kLog2_10000 = 13.287712379549449391481277717958;
  float pe[8];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int i2 = c0 + j;   // even column 2i; column i2 + 1 is its cosine
    const double w = exp2(-(double)i2 * (kLog2_10000 / (double)p.d_model));
    const double a = (double)pos * w;
    const double r = a - kTwoPi * rint(a * (1.0 / kTwoPi));
    float s, c;
    sincosf((float)r, &s, &c);
    pe[j] = s;
    pe[j + 1] = c;
  }
  const __bf16* x = reinterpret_cast<const __bf16*>(p.x);
  __bf16* h = reinterpret_cast<__bf16*>(p.h);
  for (int b = 0; b < p.batch; ++b) {
    const int64_t row = (int64_t)b * p.n + pos;
    const bf16x8 xv = *reinterpret_cast<const bf16x8*>(x + row * p.ldx + c0);
    bf16x8 hv;
#pragma unroll
    for (int j = 0; j < 8; ++j) hv[j] = (__bf16)((float)xv[j] + pe[j]);
    *reinterpret_cast<bf16x8*>(h + row * p.ldh + c0) = hv;
  }
}

// ---------------------------------------------------------------------------
constexpr int LBM = 64;        // output rows per workgroup
constexpr int LWAVES = 8;

// Ocat slice [64][16*KS]: chunk c of row r at c ^ swz_xr<KS>(r), so that 16
// consecutive rows read one chunk each on distinct banks (32-byte rows for
// KS = 1, 64-byte rows for KS = 2).
template <int KS>
__device__ __forceinline__ int swz_xr(int r) { return KS == 1 ? (r >> 3) & 1 : (r >> 2) & 3; }
// W^O slice [16*KS][d]: chunk c of row r at c ^ 4*(r & 3) (the transposed
// reads touch 4 consecutive rows x 64 bytes).
__device__ __forceinline__ int swz_wr(int r) { return 4 * (r & 3); }

// LDS address of a DMA destination, wave-uniform by construction; said so to
// the compiler so that it stays in a scalar register.
__device__ __forceinline__ uint32_t uniform_lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(p));
}

// NB: 256-column groups of d_model (wave w owns columns [32*NB*w, 32*NB*(w+1)));
// KS: 16-deep k steps per ring stage; NS: ring stages.
template <int NB, int KS, int NS>
__global__ __launch_bounds__(64 * LWAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_ln_kernel(const GemmLnParams p) {
  constexpr int N = 256 * NB;                 // d_model
  constexpr int LK = 16 * KS;                 // k per stage
  constexpr int X_E = LBM * LK;               // bf16 elements of the Ocat slice
  constexpr int W_E = LK * N;                 // bf16 elements of the W slice
  constexpr int STAGE_E = X_E + W_E;
  constexpr int WCH = N / 8;                  // 16-byte chunks per W row
  constexpr int XCH = LK / 8;                 // 16-byte chunks per Ocat row
  constexpr int WIPW = KS * NB;               // W-slice DMA instructions per wave
  static_assert(NS * STAGE_E >= LBM * N, "the output tile must fit the ring");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NS * STAGE_E];
  __shared__ float red[LWAVES][LBM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int m0 = blockIdx.x * LBM;
  const int c0 = wave * 32 * NB;              // this wave's first output column

  const __bf16* A = reinterpret_cast<const __bf16*>(p.a) + (int64_t)m0 * p.lda;
  const __bf16* W = reinterpret_cast<const __bf16*>(p.w);
  const int rows_here = min(LBM, p.M - m0);
  const uint32_t a_bytes = (uint32_t)((int64_t)(rows_here - 1) * p.lda * 2 + (int64_t)p.K * 2);
  const uint32_t w_bytes = (uint32_t)((int64_t)p.K * N * 2);
  const i32x4 rw = make_rsrc(W, w_bytes);

  // DMA plan per stage: the W slice is 8*KS*NB instructions of 1 KiB (KS*NB
  // per wave), instruction u covering flattened chunks 64u..64u+63 of the
  // [LK][N/8] chunk grid; the Ocat slice is 2*KS more (one each for waves
  // 0 .. 2*KS-1).
  uint32_t w_off[WIPW];
#pragma unroll
  for (int i = 0; i < WIPW; ++i) {
    const int f = (wave * WIPW + i) * 64 + lane;
    const int r = f / WCH, pos = f - r * WCH;
    w_off[i] = (uint32_t)(((int64_t)r * N + (pos ^ swz_wr(r)) * 8) * 2);
  }
  const bool x_wave = wave < 2 * KS;
  uint32_t x_off = 0;
  if (x_wave) {
    const int f = wave * 64 + lane;           // chunks of the [64][XCH] grid
    const int r = f / XCH, pos = f - r * XCH;
    x_off = (uint32_t)(((int64_t)r * p.lda + (pos ^ swz_xr<KS>(r)) * 8) * 2);
  }
  // k-step order: workgroup i starts at step 2*(i/8) mod nk and wraps around.
  // Every workgroup streams all of W^O; the 32 workgroups on one XCD are
  // i = x, x+8, x+16, ... (dealt round-robin), and in a common order they
  // would ask their L2 for the same W^O slice at the same moment, queueing on
  // the same channels.  Starting points two steps apart spread them over the
  // matrix (measured on the sublayer shape: 60.5 -> 54.2 us; one step apart
  // 54.7, four 54.4, eight 55.5, sixteen 56.6).  The sum over k is exact up
  // to the fp32 rounding order.
  const int nk_all = p.K / LK;
  const int k_rot = nk_all > 0 ? (int)(((unsigned)(blockIdx.x >> 3) * 2u) % (unsigned)nk_all) : 0;
  auto issue_stage = [&](int s) {
    const int k0 = (s + k_rot < nk_all ? s + k_rot : s + k_rot - nk_all) * LK;
    __bf16* st = smem + (s % NS) * STAGE_E;
#pragma unroll
    for (int i = 0; i < WIPW; ++i)
      dma16(w_off[i] + (uint32_t)k0 * N * 2, rw, uniform_lds_addr(st + X_E + (wave * WIPW + i) * 512));
    if (x_wave) {
      const i32x4 ra = make_rsrc(A + k0, a_bytes >= (uint32_t)k0 * 2 ? a_bytes - (uint32_t)k0 * 2 : 0u);
      dma16(x_off, ra, uniform_lds_addr(st + wave * 512));
    }
  };
  auto wait_ring = [&](int n_after) {   // at most n_after later stages in flight
    if (x_wave) wait_vmcnt_le<WIPW + 1>(n_after * (WIPW + 1));
    else wait_vmcnt_le<WIPW>(n_after * WIPW);
  };

  const int nk = p.K / LK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue_stage(s);

  f32x16 acc[2][NB];   // [m block][n block]
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

  // the residual tile [64][N] for the epilogue: copy i of this wave lands at
  // LDS elements [512 I, 512 I + 512), I = 4*NB*wave + i, as whole-row pieces
  // (16-byte chunk c of row r at c ^ (r & 15))
  const __bf16* R = reinterpret_cast<const __bf16*>(p.res) + (int64_t)m0 * p.ldr;
  const i32x4 rr = make_rsrc(R, (uint32_t)((int64_t)(rows_here - 1) * p.ldr * 2 + N * 2));
  auto res_copy = [&](int i) {
    const int I = wave * 4 * NB + i;
    const int f = I * 64 + lane;
    const int r = f / WCH, pos = f - r * WCH;
    dma16((uint32_t)(((int64_t)r * p.ldr + (pos ^ (r & 15)) * 8) * 2), rr, uniform_lds_addr(smem + I * 512));
  };
  auto res_in_stage = [&](int i, int u) {   // copy i overlaps ring stage u
    const int I = wave * 4 * NB + i;
    return I * 512 < (u + 1) * STAGE_E && (I + 1) * 512 > u * STAGE_E;
  };

  const int k16 = lane & 15, chalf = (lane >> 4) & 1;
  const int tr_row = g * 8 + (k16 >> 2);              // k row of this pointer lane (+4 for the upper half)
  const int tr_col = chalf * 16 + 4 * (k16 & 3);      // column offset in the 32-column block

  for (int s = 0; s < nk; ++s) {
    wait_ring(min(NS - 2, nk - 1 - s));
    barrier_lds();
    if (s + NS - 1 < nk) issue_stage(s + NS - 1);
    if (s == nk - 1) {
      // every other stage is idle now: the residual pieces that land there
      // are copied during the last step instead of after it (measured on the
      // sublayer shape: 52.4-52.6 -> 52.0 us)
#pragma unroll
      for (int i = 0; i < 4 * NB; ++i)
        if (!res_in_stage(i, s % NS)) res_copy(i);
    }
    const __bf16* Xs = smem + (s % NS) * STAGE_E;
    const __bf16* Ws = Xs + X_E;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // B operand (Ocat^T): lane = output row 32*mb + l32, k = 16*ks + 8g + 0..7
      bf16x8 xf[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + l32;
        xf[mb] = *reinterpret_cast<const bf16x8*>(Xs + r * LK + 8 * ((2 * ks + g) ^ swz_xr<KS>(r)));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // A operand (W^T): lane = output column c0 + 32*nb + l32, k = 16*ks + 8g + 0..7
        const int col = c0 + 32 * nb + tr_col;            // a multiple of 4: inside one chunk
        const int r0 = 16 * ks + tr_row, r1 = r0 + 4;
        const bf16x4 lo = tr_read(Ws + r0 * N + 8 * ((col >> 3) ^ swz_wr(r0)) + (col & 7));
        const bf16x4 hi = tr_read(Ws + r1 * N + 8 * ((col >> 3) ^ swz_wr(r1)) + (col & 7));
        const bf16x8 wf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma32(wf, xf[mb], acc[mb][nb]);
      }
    }
  }

  // ---- epilogue: register r of acc[mb][nb] is column c0 + 32*nb + 8*(r/4) +
  // 4*g + r%4 of row m0 + 32*mb + l32.  The residual tile [64][N] comes into
  // the (now idle) ring by LDS DMA in whole rows, and y leaves through it the
  // same way; in LDS, 16-byte chunk c of row r sits at c ^ (r & 15), so the
  // reads and writes in the accumulator layout (32 rows x one chunk) touch
  // distinct banks.
  __syncthreads();   // every wave is done with the ring
  {
#pragma unroll
    for (int i = 0; i < 4 * NB; ++i)
      if (nk == 0 || res_in_stage(i, (nk - 1) % NS)) res_copy(i);
    wait_vmcnt<0>();
  }
  __syncthreads();
  auto tile_at = [&](int r, int n) { return smem + r * N + 8 * ((n >> 3) ^ (r & 15)) + (n & 7); };
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = 32 * mb + l32;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = c0 + 32 * nb + 8 * rg + 4 * g;
        const bf16x4 hv = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(tile_at(r, n)));
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mb][nb][4 * rg + t] += (float)hv[t];   // rows past M: 0 + 0
      }
  }
  const float inv_n = 1.0f / (float)N;
  float mean[2], rstd[2];
  // mean
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float s = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[mb][nb][r];
    s = sum_with_partner(s);
    if (g == 0) red[wave][32 * mb + l32] = s;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < LWAVES; ++w) s += red[w][32 * mb + l32];
    mean[mb] = s * inv_n;
  }
  __syncthreads();   // every wave has read the sums before they are overwritten
  // variance (mean squared deviation)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float s = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dv = acc[mb][nb][r] - mean[mb];
        s = fmaf(dv, dv, s);
      }
    s = sum_with_partner(s);
    if (g == 0) red[wave][32 * mb + l32] = s;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < LWAVES; ++w) s += red[w][32 * mb + l32];
    rstd[mb] = 1.0f / sqrtf(s * inv_n + p.eps);
  }
  // y = gamma (z - mean) rstd + beta, into the tile (each lane overwrites the
  // residual values it read), then whole rows out
  const __bf16* G = reinterpret_cast<const __bf16*>(p.gamma);
  const __bf16* Bt = reinterpret_cast<const __bf16*>(p.beta);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int n = c0 + 32 * nb + 8 * rg + 4 * g;
      const bf16x4 gv = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(G + n));
      const bf16x4 bv = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(Bt + n));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        bf16x4 o;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          o[t] = (__bf16)fmaf((float)gv[t], (acc[mb][nb][4 * rg + t] - mean[mb]) * rstd[mb], (float)bv[t]);
        *reinterpret_cast<u32x2*>(tile_at(32 * mb + l32, n)) = __builtin_bit_cast(u32x2, o);
      }
    }
  __syncthreads();
  __bf16* Y = reinterpret_cast<__bf16*>(p.y) + (int64_t)m0 * p.ldy;
  for (int f = tid; f < rows_here * WCH; f += 64 * LWAVES) {
    const int r = f / WCH, pos = f - r * WCH;
    *reinterpret_cast<u32x4*>(Y + (int64_t)r * p.ldy + (pos ^ (r & 15)) * 8) =
        *reinterpret_cast<const u32x4*>(smem + r * N + pos * 8);
  }
}

}  // namespace

hipError_t launch_pe_add_bf16(const PeAddParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.n * (p.d_model / 8);
  if (threads == 0 || p.batch == 0) return hipSuccess;
  return launch_kernel(pe_add_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), stream, p);
}

// 32-deep k stages in a 2-stage ring (136 KiB): one barrier per 16 MFMAs
// per wave; 16-deep stages in a 4-stage ring were 6% slower.
constexpr int LN_KS = 2, LN_NS = 2;

hipError_t launch_gemm_bf16_ln(const GemmLnParams& p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.M + LBM - 1) / LBM)), block(64 * LWAVES);
  switch (p.N) {
    case 256: return launch_kernel(gemm_bf16_ln_kernel<1, LN_KS, LN_NS>, grid, block, stream, p);
    case 512: return launch_kernel(gemm_bf16_ln_kernel<2, LN_KS, LN_NS>, grid, block, stream, p);
    case 768: return launch_kernel(gemm_bf16_ln_kernel<3, LN_KS, LN_NS>, grid, block, stream, p);
    case 1024: return launch_kernel(gemm_bf16_ln_kernel<4, LN_KS, LN_NS>, grid, block, stream, p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
