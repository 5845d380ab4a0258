// Gradients of scaled dot-product attention, bf16 storage, head size 64, gfx950.
//
// The model of "Attention Is All You Need" is trained end to end (the vlmlib.cn
// summary's training-objective paragraph; attention-paper-guide section 05), so
// the attention layer needs dQ, dK and dV for a given dO.  With P the forward
// weights and D_i = sum_c dO_ic O_ic (the softmax Jacobian applied to dO):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ = scale dS K,
//   dK = scale dS^T Q.
// P is recomputed from the scores and the forward's log-sum-exp, exp(s - lse),
// so nothing of size n_q x n_kv is stored.  Two kernels, in this order:
//
//   sdpa_bwd_dq        workgroup = (b, h, 128 queries), the forward's
//                      decomposition: S^T = K Q^T and dP^T = V dO^T with one
//                      query per lane column, dQ^T += K^T dS^T.  It first
//                      forms each row's D (fp32) and lse in log2 units (+inf
//                      for padded rows and rows without keys, so their weights
//                      are exactly 0) and leaves them in the workspace.
//   sdpa_bwd_dkdv      workgroup = (b, h, 128 keys), wave w owns 32 keys and
//                      keeps their K and V fragments in registers; query tiles
//                      of 64 (Q, dO and the per-row terms) stream through an
//                      LDS-DMA ring.  Per tile and 32-query block the wave
//                      computes S = Q K^T and dP = dO V^T with one key per lane
//                      column, then dV^T += dO^T P and dK^T += Q^T dS with the
//                      score accumulators as the B operands (their rows are
//                      the queries in the order the C layout gives them; the
//                      dO^T and Q^T operands are read transposed in the same
//                      order).
//
// Every product is v_mfma_f32_32x32x16_bf16 (fp32 accumulation); P and dS are
// rounded to bf16 for the products, and dQ, dK, dV once to bf16 at the store.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int D = 64;          // head size (d_k = d_v)
constexpr int BT = 64;         // rows per streamed tile (queries or keys)
constexpr int TILE_E = BT * D; // bf16 elements of one [64][64] tile (8 KiB)
constexpr float LOG2E = 1.4426950408889634f;

// Tiles here are read both ways: as rows (one 16-byte chunk of 32 consecutive
// rows per half-wave) and transposed (8 rows x 64 bytes per ds_read_b64_tr_b16).
// The 16-byte chunk c of row r sits at chunk position c ^ swz_qt(r); bits 0-1
// of the swizzle spread 8 consecutive rows' chunk over distinct bank groups
// for the row reads, bit 2 moves rows 4m+2, 4m+3 to the other half of the
// banks, which the transposed reads need.
__device__ __forceinline__ int swz_qt(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// A [32 x 16] operand (rows r0 + lane%32, columns 16*dstep + 8*g + 0..7) read
// from a row-major [64][64] tile.
__device__ __forceinline__ bf16x8 rows_frag(const __bf16* tile, int r, int dstep, int g) {
  const int c = 2 * dstep + g;
  return *reinterpret_cast<const bf16x8*>(tile + r * D + 8 * (c ^ swz_qt(r)));
}

// The transposed operand of block (cb, jb, s): element t of lane l is
// tile[row(t)][32*cb + l%32] with row(t) = 32*jb + 16*s + 8*(t/4) + 4*g + t%4,
// the row order of the score accumulator's C layout, read with two
// ds_read_b64_tr_b16.
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* tile, int cb, int jb, int s, int lane) {
  const int k16 = lane & 15, g = lane >> 5;
  const int chalf = (lane >> 4) & 1;
  const int tr_row = g * 4 + (k16 >> 2);
  const int tr_chunk = 2 * chalf + ((k16 & 3) >> 1);
  const int tr_half = 4 * (k16 & 1);
  bf16x4 part[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int row = 32 * jb + 16 * s + 8 * hh + tr_row;
    part[hh] = tr_read(tile + row * D + tr_half + 8 * ((4 * cb + tr_chunk) ^ swz_qt(row)));
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Registers 8s..8s+7 of an accumulator, rounded to bf16, as an MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; t += 2) {
    const bf16x2 h = __builtin_convertvector(f32x2{x[t], x[t + 1]}, bf16x2);
    r[t] = h[0];
    r[t + 1] = h[1];
  }
  return r;
}

// ---------------------------------------------------------------------------
template <int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void sdpa_bwd_dkdv(const SdpaBwdParams p) {
  constexpr int BK = 128;                  // keys per workgroup (4 waves x 32)
  constexpr int STAGE_E = 2 * TILE_E;      // Q tile, dO tile
  constexpr int IPT = 4;                   // Q/dO DMA instructions per wave per stage (+1 for waves 0, 1)
  static_assert(NS >= 2 && NS <= 4, "bad configuration");
  static_assert(NS * STAGE_E >= 8 * 32 * D, "the dK and dV blocks must fit the ring");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NS * STAGE_E];
  __shared__ __attribute__((aligned(1024))) float lds_l2[NS][256];   // per stage: lse2 of queries q0..q0+255
  __shared__ __attribute__((aligned(1024))) float lds_nd[NS][256];   // per stage: -D of the same queries

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i32 = lane & 31, g = lane >> 5;
  const int bhn = p.batch * p.heads;
  const int kb = blockIdx.x / bhn;          // key blocks in ascending order: the longest causal ones first
  const int bh = blockIdx.x - kb * bhn;
  const int b = bh / p.heads, h = bh - b * p.heads;
  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  const int k0 = kb * BK, kw0 = k0 + 32 * wave;
  const int kj = kw0 + i32;                 // this lane's key
  // query tiles the workgroup visits: causal ones start at the block's first key
  int qt_begin = p.causal ? k0 / BT : 0;
  int nqt = k0 < Lkv ? (Lq + BT - 1) / BT - qt_begin : 0;
  if (nqt < 0) nqt = 0;

  const __bf16* Qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* DOb = reinterpret_cast<const __bf16*>(p.dout) + b * p.dos_b + h * p.dos_h;
  const int64_t rows_all = (int64_t)bhn * p.n_q;
  const float* L2b = p.ld + (int64_t)bh * p.n_q;              // lse2 plane
  const float* NDb = p.ld + rows_all + (int64_t)bh * p.n_q;   // -D plane
  const uint32_t q_bytes = Lq > 0 ? (uint32_t)((int64_t)(Lq - 1) * p.qs_n * 2 + 128) : 0u;
  const uint32_t o_bytes = Lq > 0 ? (uint32_t)((int64_t)(Lq - 1) * p.dos_n * 2 + 128) : 0u;
  const uint32_t ld_bytes = (uint32_t)p.n_q * 4;

  // K and V fragments of the wave's 32 keys (B operands: lane = key, k = d);
  // keys past the length read as zeros.
  bf16x8 kf[4], vf[4];
  {
    const bool kvalid = kj < Lkv;
    const int jj = kvalid ? kj : 0;
    const __bf16* krow = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h + (int64_t)jj * p.ks_n;
    const __bf16* vrow = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h + (int64_t)jj * p.vs_n;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x8 kk = *reinterpret_cast<const bf16x8*>(krow + 16 * d + 8 * g);
      const bf16x8 vv = *reinterpret_cast<const bf16x8*>(vrow + 16 * d + 8 * g);
      kf[d] = kvalid ? kk : bf16x8{};
      vf[d] = kvalid ? vv : bf16x8{};
    }
    // consume them here: the wait for these loads happens once, before any DMA
#pragma unroll
    for (int d = 0; d < 4; ++d) asm volatile("" ::"v"(kf[d]), "v"(vf[d]));
  }

  // DMA offsets: instruction u (0..15) of a stage covers row block u & 7 of Q
  // (u < 8) or dO; the fifth instruction of each wave copies 128 (lse2, D)
  // pairs into the wave's own slot.
  uint32_t dma_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = wave * 4 + i;
    const bool is_o = u >= 8;
    const int r = 8 * (u & 7) + (lane >> 3);
    const int c = (lane & 7) ^ swz_qt(r);
    dma_off[i] = (uint32_t)(((int64_t)r * (is_o ? p.dos_n : p.qs_n) + c * 8) * 2);
  }
  auto issue_stage = [&](int j) {
    const int q0 = (qt_begin + j) * BT;
    const int64_t q_adv = (int64_t)q0 * p.qs_n, o_adv = (int64_t)q0 * p.dos_n;
    const i32x4 rq = make_rsrc(Qb + q_adv, (uint32_t)max<int64_t>(0, (int64_t)q_bytes - 2 * q_adv));
    const i32x4 ro = make_rsrc(DOb + o_adv, (uint32_t)max<int64_t>(0, (int64_t)o_bytes - 2 * o_adv));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = wave * 4 + i;
      const bool is_o = u >= 8;
      const __bf16* dst = smem + (j % NS) * STAGE_E + (is_o ? TILE_E : 0) + (u & 7) * 512;
      dma16(dma_off[i], is_o ? ro : rq, lds_addr(dst));
    }
    // the per-row terms of the tile's queries: wave 0 copies lse2, wave 1 -D
    if (wave < 2) {
      const i32x4 rl = make_rsrc((wave == 0 ? L2b : NDb) + q0,
                                 (uint32_t)max<int64_t>(0, (int64_t)ld_bytes - 4 * (int64_t)q0));
      dma16((uint32_t)(lane * 16), rl, lds_addr(wave == 0 ? &lds_l2[j % NS][0] : &lds_nd[j % NS][0]));
    }
  };

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nqt) issue_stage(j);

  f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};   // dK^T, dV^T: d 0..31 / 32..63, lane = key
  const float c2 = p.scale_log2;

  for (int t = 0; t < nqt; ++t) {
    if (wave < 2) wait_vmcnt_le<IPT + 1>(min(NS - 2, nqt - 1 - t) * (IPT + 1));
    else wait_vmcnt_le<IPT>(min(NS - 2, nqt - 1 - t) * IPT);
    barrier_lds();   // stage t visible; every wave is done with stage t-1
    if (t + NS - 1 < nqt) issue_stage(t + NS - 1);
    const int q0 = (qt_begin + t) * BT;
    if (p.causal && q0 + BT - 1 < kw0) continue;   // wave-uniform: every query before the wave's keys
    const __bf16* Qs = smem + (t % NS) * STAGE_E;
    const __bf16* Ds = Qs + TILE_E;
    const float* lt2 = &lds_l2[t % NS][0];
    const float* ltd = &lds_nd[t % NS][0];
    // Only the causal mask needs applying: rows past L_q have lse2 = +inf
    // (weight 0), rows past n_q and keys past L_kv read as zeros, so their dS
    // and dO are 0 and they add nothing to the legal keys' columns; the
    // columns of keys past L_kv are replaced by zeros at the store.
    const bool diag = p.causal && q0 < kw0 + 32;
    const int qlo = kj - q0 - 4 * g;   // legal: query offset (in the tile, less 4*g) >= qlo
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q K^T and dP - D = dO V^T - D for queries q0 + 32*qb + row(r):
      // lane = key; register r is query 32*qb + 8*(r/4) + 4*g + r%4 of the
      // tile, so the -D of four consecutive queries starts each register
      // group of the dP accumulator
      f32x16 s = {}, dp;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(ltd + 32 * qb + 8 * rg + 4 * g);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) dp[4 * rg + t4] = nd[t4];
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        s = mfma32(rows_frag(Qs, 32 * qb + i32, d, g), kf[d], s);
        dp = mfma32(rows_frag(Ds, 32 * qb + i32, d, g), vf[d], dp);
      }
      if (diag) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * qb + 8 * (r >> 2) + (r & 3) < qlo) s[r] = -INFINITY;
      }
      // P = 2^(s*c2 - lse2), dS = P (dP - D)
      float pv[16], dsv[16];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(lt2 + 32 * qb + 8 * rg + 4 * g);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const int r = 4 * rg + t4;
          const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l2[t4]));
          pv[r] = pr;
          dsv[r] = pr * dp[r];
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of this block
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 pf = pack8(pv + 8 * sb);
        const bf16x8 sf = pack8(dsv + 8 * sb);
        dv0 = mfma32(tr_frag(Ds, 0, qb, sb, lane), pf, dv0);
        dv1 = mfma32(tr_frag(Ds, 1, qb, sb, lane), pf, dv1);
        dk0 = mfma32(tr_frag(Qs, 0, qb, sb, lane), sf, dk0);
        dk1 = mfma32(tr_frag(Qs, 1, qb, sb, lane), sf, dk1);
      }
    }
  }

  // dK = scale dK^T, dV = dV^T, one rounding to bf16; register r of block cb
  // holds d = 32*cb + 8*(r/4) + 4*g + r%4 of key kj.  Each wave stages its
  // 32 x 64 blocks of dK and dV in its own 4 KiB pieces of the (now idle)
  // ring -- 16-byte chunk c of row r at position c ^ (r & 7) -- and writes
  // them out as whole 128-byte rows with write-through stores.
  const bool kvalid = kj < Lkv;   // the columns of keys past L_kv hold no gradient (maybe inf/NaN)
  barrier_lds();                  // every wave is past its last read of the ring
  __bf16* dKs = smem + wave * 32 * D;
  __bf16* dVs = smem + (4 + wave) * 32 * D;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    bf16x4 a0, a1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a0[t] = (__bf16)(kvalid ? dk0[4 * rg + t] * p.scale : 0.f);
      a1[t] = (__bf16)(kvalid ? dk1[4 * rg + t] * p.scale : 0.f);
    }
    *reinterpret_cast<u32x2*>(dKs + i32 * D + 8 * (rg ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, a0);
    *reinterpret_cast<u32x2*>(dKs + i32 * D + 8 * ((4 + rg) ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, a1);
  }
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    bf16x4 b0, b1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      b0[t] = (__bf16)(kvalid ? dv0[4 * rg + t] : 0.f);
      b1[t] = (__bf16)(kvalid ? dv1[4 * rg + t] : 0.f);
    }
    *reinterpret_cast<u32x2*>(dVs + i32 * D + 8 * (rg ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, b0);
    *reinterpret_cast<u32x2*>(dVs + i32 * D + 8 * ((4 + rg) ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, b1);
  }
  __bf16* dKb = reinterpret_cast<__bf16*>(p.dk) + b * p.dks_b + h * p.dks_h;
  __bf16* dVb = reinterpret_cast<__bf16*>(p.dv) + b * p.dvs_b + h * p.dvs_h;
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    if (kw0 + r < p.n_kv) {
      const int pos = 8 * (c ^ (r & 7));
      store_out(dKb + (int64_t)(kw0 + r) * p.dks_n + 8 * c, *reinterpret_cast<const u32x4*>(dKs + r * D + pos));
      store_out(dVb + (int64_t)(kw0 + r) * p.dvs_n + 8 * c, *reinterpret_cast<const u32x4*>(dVs + r * D + pos));
    }
  }
}

template <int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void sdpa_bwd_dq(const SdpaBwdParams p) {
  constexpr int BM = 128;                  // queries per workgroup (4 waves x 32)
  constexpr int STAGE_E = 2 * TILE_E;      // K tile, V tile
  constexpr int IPT = 4;
  static_assert(NS >= 2 && NS <= 4, "bad configuration");
  static_assert(NS * STAGE_E >= 4 * 32 * D, "the dQ blocks must fit the ring");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NS * STAGE_E];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i32 = lane & 31, g = lane >> 5;
  const int bhn = p.batch * p.heads;
  const int nqb = (p.n_q + BM - 1) / BM;
  const int qb_idx = blockIdx.x / bhn;
  const int bh = blockIdx.x - qb_idx * bhn;
  const int qb = p.causal ? nqb - 1 - qb_idx : qb_idx;   // causal: the longest blocks first
  const int b = bh / p.heads, h = bh - b * p.heads;
  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  const int q0 = qb * BM, qw0 = q0 + 32 * wave, qi = qw0 + i32;
  int kv_end = Lkv, wkv_end = Lkv;
  if (p.causal) {
    kv_end = min(kv_end, min(q0 + BM, Lq));
    wkv_end = min(wkv_end, min(qw0 + 32, Lq));
  }
  if (q0 >= Lq) kv_end = 0;
  if (qw0 >= Lq) wkv_end = 0;
  const int nblk = (kv_end + BT - 1) / BT;

  // Q and dO fragments of this lane's query (B operands: lane = query, k = d),
  // its lse2 = lse*log2(e) and D = dO . O (lanes l and l^32 hold the two
  // halves of d); padded rows and rows with no key read zeros and get
  // lse2 = +inf (weights 0).  lse2 and -D also go to the workspace planes,
  // where the dK/dV kernel, launched next, reads them.
  bf16x8 qf[4], df[4];
  float lse2 = INFINITY, dd = 0.f;
  {
    const bool qvalid = qi < Lq;
    const int ii = qvalid ? qi : 0;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h + (int64_t)ii * p.qs_n;
    const __bf16* drow = reinterpret_cast<const __bf16*>(p.dout) + b * p.dos_b + h * p.dos_h + (int64_t)ii * p.dos_n;
    const __bf16* orow = reinterpret_cast<const __bf16*>(p.o) + b * p.os_b + h * p.os_h + (int64_t)ii * p.os_n;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + 16 * d + 8 * g);
      const bf16x8 c = *reinterpret_cast<const bf16x8*>(drow + 16 * d + 8 * g);
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(orow + 16 * d + 8 * g);
      qf[d] = qvalid ? a : bf16x8{};
      df[d] = qvalid ? c : bf16x8{};
#pragma unroll
      for (int t = 0; t < 8; ++t) dot = fmaf((float)c[t], (float)o[t], dot);
    }
    dot = sum_with_partner(dot);
    const float lse = p.lse[(int64_t)bh * p.n_q + ii];
    if (qvalid && lse > -INFINITY) {
      lse2 = lse * LOG2E;
      dd = dot;
    }
    if (g == 0 && qi < p.n_q) {
      const int64_t row = (int64_t)bh * p.n_q + qi;
      p.ld[row] = lse2;                                    // lse2 plane
      p.ld[(int64_t)bhn * p.n_q + row] = -dd;              // -D plane
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) asm volatile("" ::"v"(qf[d]), "v"(df[d]));
    asm volatile("" ::"v"(lse2), "v"(dd));
  }

  const __bf16* Kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h;
  const __bf16* Vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h;
  const uint32_t k_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.ks_n * 2 + 128) : 0u;
  const uint32_t v_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.vs_n * 2 + 128) : 0u;
  uint32_t dma_off[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int u = wave * IPT + i;
    const bool is_v = u >= 8;
    const int r = 8 * (u & 7) + (lane >> 3);
    const int c = (lane & 7) ^ swz_qt(r);
    dma_off[i] = (uint32_t)(((int64_t)r * (is_v ? p.vs_n : p.ks_n) + c * 8) * 2);
  }
  auto issue_tile = [&](int t) {
    const int64_t k_adv = (int64_t)t * BT * p.ks_n, v_adv = (int64_t)t * BT * p.vs_n;
    const i32x4 rk = make_rsrc(Kb + k_adv, (uint32_t)max<int64_t>(0, (int64_t)k_bytes - 2 * k_adv));
    const i32x4 rv = make_rsrc(Vb + v_adv, (uint32_t)max<int64_t>(0, (int64_t)v_bytes - 2 * v_adv));
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = wave * IPT + i;
      const bool is_v = u >= 8;
      const __bf16* dst = smem + (t % NS) * STAGE_E + (is_v ? TILE_E : 0) + (u & 7) * 512;
      dma16(dma_off[i], is_v ? rv : rk, lds_addr(dst));
    }
  };
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nblk) issue_tile(t);

  f32x16 dq0 = {}, dq1 = {};   // dQ^T for d 0..31 / 32..63, lane = query
  const float c2 = p.scale_log2;
  constexpr int kFar = 1 << 30;
  for (int blk = 0; blk < nblk; ++blk) {
    wait_vmcnt_le<IPT>(min(NS - 2, nblk - 1 - blk) * IPT);
    barrier_lds();
    if (blk + NS - 1 < nblk) issue_tile(blk + NS - 1);
    const int key0 = blk * BT;
    if (key0 >= wkv_end) continue;
    const __bf16* Ks = smem + (blk % NS) * STAGE_E;
    const __bf16* Vs = Ks + TILE_E;
    // S^T = K Q^T and dP^T = V dO^T: sc/dp[jb] for keys 32*jb..; register r is
    // key key0 + 32*jb + 8*(r/4) + 4*g + r%4, lane column the query qi
    f32x16 sc[2] = {}, dp[2] = {};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        sc[jb] = mfma32(rows_frag(Ks, 32 * jb + i32, d, g), qf[d], sc[jb]);
        dp[jb] = mfma32(rows_frag(Vs, 32 * jb + i32, d, g), df[d], dp[jb]);
      }
    // keys past this lane's query (causal) or past L_kv get score -inf, so
    // weight 0 and dS 0 (rows past L_q already have lse2 = +inf)
    if (key0 + BT > Lkv || (p.causal && key0 + BT - 1 > qw0)) {
      const int krel = min(Lkv - 1, p.causal ? qi : kFar) - key0 - 4 * g;   // legal: offset <= krel
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * jb + 8 * (r >> 2) + (r & 3) > krel) sc[jb][r] = -INFINITY;
    }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sc[jb][r], c2, -lse2));
        dsv[r] = pr * (dp[jb][r] - dd);
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 sf = pack8(dsv + 8 * sb);
        dq0 = mfma32(tr_frag(Ks, 0, jb, sb, lane), sf, dq0);
        dq1 = mfma32(tr_frag(Ks, 1, jb, sb, lane), sf, dq1);
      }
    }
  }

  // dQ = scale dQ^T, one rounding to bf16 (rows past the length are zeros),
  // staged per wave in the idle ring and written as whole rows as above
  barrier_lds();   // every wave is past its last read of the ring
  __bf16* dQs = smem + wave * 32 * D;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    bf16x4 a0, a1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a0[t] = (__bf16)(dq0[4 * rg + t] * p.scale);
      a1[t] = (__bf16)(dq1[4 * rg + t] * p.scale);
    }
    *reinterpret_cast<u32x2*>(dQs + i32 * D + 8 * (rg ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, a0);
    *reinterpret_cast<u32x2*>(dQs + i32 * D + 8 * ((4 + rg) ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, a1);
  }
  __bf16* dQb = reinterpret_cast<__bf16*>(p.dq) + b * p.dqs_b + h * p.dqs_h;
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    if (qw0 + r < p.n_q)
      store_out(dQb + (int64_t)(qw0 + r) * p.dqs_n + 8 * c,
                *reinterpret_cast<const u32x4*>(dQs + r * D + 8 * (c ^ (r & 7))));
  }
}

}  // namespace

// Fixed scratch of the allocation-free backward entry point: the lse2 and -D
// planes, 8 bytes per query row of every (b, h), 2 M rows at most.  Each
// device holds one copy for the life of the process and every call on that
// device uses it.  In host code `scratch` only names the symbol: its device
// address is looked up per device (hipGetSymbolAddress, with the device
// current) and only that address is ever passed to a kernel.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lock;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* a = addr[dev].load(std::memory_order_acquire);
  if (!a) {
    std::lock_guard<std::mutex> g(lock);
    a = addr[dev].load(std::memory_order_relaxed);
    if (!a) {
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      addr[dev].store(a, std::memory_order_release);
    }
  }
  *ptr = a;
  return hipSuccess;
}

hipError_t launch_sdpa_bwd_bf16(const SdpaBwdParams& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.batch * p.heads;
  if (bh == 0) return hipSuccess;
  // dQ first: it also writes the lse2 and -D planes the dK/dV kernel reads
  if (p.n_q > 0) {
    const int64_t grid = (int64_t)((p.n_q + 127) / 128) * bh;
    const hipError_t e = launch_kernel(sdpa_bwd_dq<2>, dim3((unsigned)grid), dim3(256), stream, p);
    if (e != hipSuccess) return e;
  }
  if (p.n_kv > 0) {
    const int64_t grid = (int64_t)((p.n_kv + 127) / 128) * bh;
    return launch_kernel(sdpa_bwd_dkdv<2>, dim3((unsigned)grid), dim3(256), stream, p);
  }
  return hipSuccess;
}

}  // namespace attn
