// Scaled dot-product attention forward, bf16 storage, head size 64, gfx950.
//
// Computes O = softmax(Q K^T * scale) V per (batch, head) -- "Attention Is All
// You Need" section 3.2.1, Eq. 1 -- with the decoder's causal mask and key
// padding applied as -inf at the softmax input (section 3.2.3; the
// rockcohen.cc deep read, sections 5.3 and 6.3), without ever materialising
// the n_q x n_kv score matrix: the keys are streamed in tiles and the softmax
// is accumulated online with a running row max and row sum (the max shift is
// the shift invariance of the softmax, rockcohen.cc section 3.2).
//
// Work decomposition
//   workgroup = (batch, head, block of 32*NW queries); wave w owns 32 queries.
//   Per iteration the workgroup stages 64 keys of K and V (8 KiB each) in LDS
//   (double-buffered, one barrier per iteration) and every wave computes
//     S^T[64 keys x 32 queries] = K_tile . Q^T     (8 x mfma 32x32x16 bf16)
//     online softmax on S^T                        (VALU, exp2)
//     O^T[64 x 32] += V_tile^T . P^T               (8 x mfma 32x32x16 bf16)
//   Computing the transposes puts one query in each lane column of the
//   accumulators (lane l holds query l%32; lanes l and l^32 split the keys),
//   so the row max needs a single cross-lane swap per tile, the row sum stays
//   per lane until the end, and the S accumulator is already the P^T operand
//   of the second product without any data movement.  V stays row-major in
//   LDS; its transposed operand is read with ds_read_b64_tr_b16.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_bf16; checked by a probe on gfx950):
//   A[32 x 16]: lane l holds row l%32, k = 8*(l/32) + 0..7
//   B[16 x 32]: lane l holds col l%32, k = 8*(l/32) + 0..7
//   C[32 x 32]: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, col l%32
// ds_read_b64_tr_b16, per group of 16 lanes where lane k points at 4 values
// M[k][0..3]: lane i receives M[i/4][i%4], M[4+i/4][i%4], M[8+i/4][i%4],
// M[12+i/4][i%4].

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 64;         // head size (d_k = d_v)
constexpr int BN = 64;        // keys per iteration
constexpr int LDS_ROW = 72;   // bf16 per LDS row: 64 + 8 pad (144 B) -> conflict-free row reads
constexpr int TILE = BN * LDS_ROW;
constexpr float LN2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l^32, combined with the own value: {own, partner}.
__device__ __forceinline__ float max_with_partner(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 tr_read(const __bf16* lds_elem) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_elem));
  return __builtin_bit_cast(bf16x4, v);
}

// Workgroup id -> (batch*head index, query block).  Workgroups are handed to
// the 8 XCDs round-robin, so when batch*heads is a multiple of 8 all query
// blocks of one (b, h) land on the same XCD and share its L2 for K/V.  With a
// causal mask the longest query blocks are dispatched first.
__device__ __forceinline__ void map_block(int bid, int bh_total, int nqb, int causal, int& bh,
                                          int& qb) {
  int qb_idx;
  if ((bh_total & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, per = bh_total >> 3;
    qb_idx = slot / per;
    bh = (slot - qb_idx * per) * 8 + xcd;
  } else {
    qb_idx = bid / bh_total;
    bh = bid - qb_idx * bh_total;
  }
  qb = causal ? nqb - 1 - qb_idx : qb_idx;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_bf16_d64(const SdpaBf16Params p) {
  constexpr int BM = 32 * NW;          // queries per workgroup
  constexpr int NT = 64 * NW;          // threads per workgroup
  constexpr int CPT = (BN * D / 8) / NT;  // 16-byte chunks per thread per tile
  static_assert(CPT * NT == BN * D / 8, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * TILE];  // [buf][K, V][64][72]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, g = lane >> 5;

  int bh, qb;
  map_block(blockIdx.x, p.batch * p.heads, p.n_qblocks, p.causal, bh, qb);
  const int b = bh / p.heads, h = bh - b * p.heads;

  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + i32;

  // keys this workgroup / this wave needs
  int kv_end = Lkv, wkv_end = Lkv;
  if (p.causal) {
    kv_end = min(kv_end, q0 + BM);
    wkv_end = min(wkv_end, qw0 + 32);
  }
  if (q0 >= Lq) kv_end = 0;
  if (qw0 >= Lq) wkv_end = 0;
  const int nblk = (kv_end + BN - 1) / BN;

  const __bf16* Qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h;
  const __bf16* Vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h;

  // Q^T operand: lane holds query qi, d = 16*dstep + 8*g + 0..7.  Padded
  // query rows load zeros so their (discarded) columns stay finite.
  bf16x8 qf[4];
  {
    const bool qvalid = qi < Lq;
    const __bf16* qrow = Qb + (int64_t)qi * p.qs_n + 8 * g;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qvalid) raw = *reinterpret_cast<const u32x4*>(qrow + 16 * d);
      qf[d] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Staging: chunk c of a 64x64 tile is row c/8, columns 8*(c%8)..+7.
  // Key rows at or beyond the length are zero-filled, never read: zero
  // values keep 0 * V finite even where the padding holds NaN.
  u32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int blk) {
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
      const int c = tid + t * NT;
      const int row = c >> 3, col = (c & 7) * 8;
      const int j = blk * BN + row;
      if (j < Lkv) {
        kr[t] = *reinterpret_cast<const u32x4*>(Kb + (int64_t)j * p.ks_n + col);
        vr[t] = *reinterpret_cast<const u32x4*>(Vb + (int64_t)j * p.vs_n + col);
      } else {
        kr[t] = u32x4{0u, 0u, 0u, 0u};
        vr[t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* Ks = smem + buf * 2 * TILE;
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
      const int c = tid + t * NT;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * LDS_ROW + col) = kr[t];
      *reinterpret_cast<u32x4*>(Ks + TILE + row * LDS_ROW + col) = vr[t];
    }
  };

  f32x16 o0 = {}, o1 = {};     // O^T for value columns 0..31 and 32..63
  float m = -INFINITY;         // running max of scale*log2(e)*score
  float l = 0.f;               // running sum (this lane's half of the keys)
  const float c2 = p.scale_log2;

  // transposed-read addressing inside a 16-lane group
  const int k16 = lane & 15;
  const int chalf = (lane >> 4) & 1;
  const int tr_row = g * 4 + (k16 >> 2);
  const int tr_col = chalf * 16 + 4 * (k16 & 3);

  if (nblk > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nblk) load_tile(blk + 1);
    const int key0 = blk * BN;

    if (key0 < wkv_end) {  // wave-uniform: skip tiles entirely after this wave's queries
      const __bf16* Ks = smem + buf * 2 * TILE;
      const __bf16* Vs = Ks + TILE;

      // S^T = K . Q^T : s0 keys 0..31 of the tile, s1 keys 32..63
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + i32 * LDS_ROW + 16 * d + 8 * g);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (32 + i32) * LDS_ROW + 16 * d + 8 * g);
        s0 = mfma32(ka, qf[d], s0);
        s1 = mfma32(kb, qf[d], s1);
      }

      // -inf for illegal keys: only the tiles that cross the length or the diagonal
      if (key0 + BN > Lkv || (p.causal && key0 + BN - 1 > qw0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j0 = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const int j1 = j0 + 32;
          if (j0 >= Lkv || (p.causal && j0 > qi)) s0[r] = -INFINITY;
          if (j1 >= Lkv || (p.causal && j1 > qi)) s1[r] = -INFINITY;
        }
      }

      // online softmax
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = max_with_partner(mx);
      const float m_new = fmaxf(m, mx * c2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no legal key yet: avoid -inf - -inf
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -m_use));
        s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, -m_use));
        rs += s0[r] + s1[r];
      }
      l = fmaf(l, alpha, rs);
      m = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= alpha;
        o1[r] *= alpha;
      }

      // P^T operands: step (jb, s) covers keys 32*jb + 16*s + 0..15; lane's
      // element t is key 32*jb + 16*s + 8*(t/4) + 4*g + t%4 (the C layout).
      bf16x8 pf[2][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pf[0][s][t] = (__bf16)s0[8 * s + t];
          pf[1][s][t] = (__bf16)s1[8 * s + t];
        }
      }

      // O^T += V^T . P^T ; the A operand for (cb, jb, s) is V[key(t)][32*cb + lane%32]
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const __bf16* vrow = Vs + (32 * jb + 16 * s + tr_row) * LDS_ROW + tr_col;
          const bf16x4 a0lo = tr_read(vrow);
          const bf16x4 a0hi = tr_read(vrow + 8 * LDS_ROW);
          const bf16x4 a1lo = tr_read(vrow + 32);
          const bf16x4 a1hi = tr_read(vrow + 8 * LDS_ROW + 32);
          const bf16x8 va0 = __builtin_shufflevector(a0lo, a0hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 va1 = __builtin_shufflevector(a1lo, a1hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o0 = mfma32(va0, pf[jb][s], o0);
          o1 = mfma32(va1, pf[jb][s], o1);
        }
      }
    }

    if (blk + 1 < nblk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = O^T / l, rounded once to bf16; rows without a legal key or
  // beyond the query length are zeros.
  const float lt = sum_with_partner(l);
  if (qi < p.n_q) {
    const bool valid = (qi < Lq) && (lt > 0.f);
    const float inv = valid ? 1.f / lt : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.os_b + h * p.os_h + (int64_t)qi * p.os_n;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      bf16x4 w0, w1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w0[t] = (__bf16)(o0[4 * rg + t] * inv);
        w1[t] = (__bf16)(o1[4 * rg + t] * inv);
      }
      *reinterpret_cast<u32x2*>(orow + 8 * rg + 4 * g) = __builtin_bit_cast(u32x2, w0);
      *reinterpret_cast<u32x2*>(orow + 32 + 8 * rg + 4 * g) = __builtin_bit_cast(u32x2, w1);
    }
    if (p.lse && g == 0)
      p.lse[((int64_t)b * p.heads + h) * p.n_q + qi] = valid ? (m + __log2f(lt)) * LN2 : -INFINITY;
  }
}

}  // namespace

int sdpa_bf16_block_m(int batch, int heads, int n_q) {
  (void)batch;
  (void)heads;
  (void)n_q;
  return 128;
}

hipError_t launch_sdpa_bf16(const SdpaBf16Params& p_in, hipStream_t stream) {
  SdpaBf16Params p = p_in;
  const int bm = sdpa_bf16_block_m(p.batch, p.heads, p.n_q);
  p.n_qblocks = (p.n_q + bm - 1) / bm;
  const int64_t grid = (int64_t)p.n_qblocks * p.batch * p.heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(sdpa_fwd_bf16_d64<4>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
