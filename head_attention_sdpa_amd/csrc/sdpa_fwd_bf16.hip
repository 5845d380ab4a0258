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
// The MFMA and transposed-read lane layouts are listed in device_common.h.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int D = 64;         // head size (d_k = d_v)
constexpr int BN = 64;        // keys per iteration
constexpr float LN2 = 0.69314718055994530942f;

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



// One workgroup = (batch, head, 32*NW queries); wave w owns queries
// 32w..32w+31 of the block.  Per key tile the workgroup waits for its DMA,
// meets at one barrier, refills the stage the previous tile used, and every
// wave computes S^T, the masked online softmax and P.V for its queries.
// There is no software pipeline inside a wave: the waves of a SIMD (WPE of
// them, at most 512/WPE VGPRs each) interleave their vector and matrix work,
// and the NS-stage ring is small enough that WPE workgroups share a CU's LDS.
// BAND compiles the restricted-attention bounds in; without it the mask has
// one upper bound per lane (causal limit and key length), one compare per
// score on the tiles that cross it.
template <int NW, int NS, int WPE, bool BAND>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void sdpa_fwd_bf16_d64(const SdpaBf16Params p) {
  constexpr int BM = 32 * NW;
  constexpr int TILE_E = BN * D;
  constexpr int IPT = 16 / NW;
  static_assert(IPT * NW == 16 && NS >= 2 && NS <= 6, "bad configuration");
  static_assert(NW * 32 * D <= 2 * TILE_E, "the Q rows must fit in one ring stage");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NS * 2 * TILE_E];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // keys this workgroup / this wave needs: [kv_begin, kv_end) and
  // [wkv_begin, wkv_end) (queries >= Lq are zeros: need nothing)
  constexpr int kFar = 1 << 30;
  int kv_end = Lkv, wkv_end = Lkv, kv_begin = 0, wkv_begin = 0;
  if (p.causal) {
    kv_end = min(kv_end, min(q0 + BM, Lq));
    wkv_end = min(wkv_end, min(qw0 + 32, Lq));
  }
  const int window = BAND ? p.window : -1;  // BAND: restricted attention, keys |i - j| <= window
  if (BAND) {
    kv_begin = max(0, q0 - window);
    wkv_begin = max(0, qw0 - window);
    kv_end = min(kv_end, min(q0 + BM, Lq) + window);
    wkv_end = min(wkv_end, min(qw0 + 32, Lq) + window);
  }
  if (q0 >= Lq) kv_end = 0;
  if (qw0 >= Lq) wkv_end = 0;
  const int t_begin = kv_begin / BN;  // first key tile of the workgroup
  const int nblk = max(0, (kv_end + BN - 1) / BN - t_begin);

  const __bf16* Qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h;
  const __bf16* Vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h;
  const uint32_t q_bytes = Lq > 0 ? (uint32_t)((int64_t)(Lq - 1) * p.qs_n * 2 + 128) : 0u;
  const uint32_t k_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.ks_n * 2 + 128) : 0u;
  const uint32_t v_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.vs_n * 2 + 128) : 0u;

  const i32x4 rs_q = make_rsrc(Qb, q_bytes);

  uint32_t dma_off[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int u = wave * IPT + i;
    const bool is_v = u >= 8;
    const int r = 8 * (u & 7) + (lane >> 3);
    const int chunk = (lane & 7) ^ (is_v ? swz_v(r) : swz_k(r));
    dma_off[i] = (uint32_t)(((int64_t)r * (is_v ? p.vs_n : p.ks_n) + chunk * 8) * 2);
  }
  auto issue_tile = [&](int j) {  // the workgroup's j-th tile, key tile t_begin + j, into stage j % NS
    const int t = t_begin + j;
    const int64_t k_adv = (int64_t)t * BN * p.ks_n, v_adv = (int64_t)t * BN * p.vs_n;
    const i32x4 rk = make_rsrc(Kb + k_adv, (uint32_t)max<int64_t>(0, (int64_t)k_bytes - 2 * k_adv));
    const i32x4 rv = make_rsrc(Vb + v_adv, (uint32_t)max<int64_t>(0, (int64_t)v_bytes - 2 * v_adv));
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = wave * IPT + i;
      const bool is_v = u >= 8;
      const __bf16* dst = smem + (j % NS) * 2 * TILE_E + (is_v ? TILE_E : 0) + (u & 7) * 512;
      dma16(dma_off[i], is_v ? rv : rk, lds_addr(dst));
    }
  };

  // Q: each wave copies its 32 query rows (4 KiB) into the last ring stage,
  // which the prologue leaves free; the first refill of that stage is issued
  // after the barrier of the first iteration, when every wave has read its Q
  // fragments.  Q goes first, so once at most (prologue tiles) DMAs are in
  // flight Q has landed, while the prologue tiles may still be on their way.
  // With restricted attention each K/V tile also serves the neighbouring
  // query blocks on this XCD, so Q (read once) is copied with the
  // non-temporal hint and does not displace them in L2 (measured: window
  // 44.8 -> 42.4 us; with full attention the hint cost up to 3% on the
  // decoder, so there Q is copied plainly).
  const __bf16* Qs = smem + (NS - 1) * 2 * TILE_E + wave * 32 * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_k(r);
    const uint32_t voff = (uint32_t)(((int64_t)(qw0 + r) * p.qs_n + chunk * 8) * 2);
    if (BAND)
      dma16_nt(voff, rs_q, lds_addr(Qs + 8 * i * D));
    else
      dma16(voff, rs_q, lds_addr(Qs + 8 * i * D));
  }
  int prologue = 0;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nblk) {
      issue_tile(t);
      ++prologue;
    }
  wait_vmcnt_le<IPT>(prologue * IPT);
  // Q^T operand: lane holds query qi, d = 16*dstep + 8*g + 0..7
  bf16x8 qf[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int c = 2 * d + g;
    qf[d] = *reinterpret_cast<const bf16x8*>(Qs + i32 * D + 8 * (c ^ swz_k(i32)));
  }

  f32x16 o0 = {}, o1 = {};
  float m = -INFINITY;
  float l = 0.f;
  const float c2 = p.scale_log2;
  const int k16 = lane & 15;
  const int chalf = (lane >> 4) & 1;
  const int tr_row = g * 4 + (k16 >> 2);
  const int tr_chunk = 2 * chalf + ((k16 & 3) >> 1);
  const int tr_half = 4 * (k16 & 1);
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  for (int blk = 0; blk < nblk; ++blk) {
    // tile blk has landed once at most min(NS-2, nblk-1-blk) newer tiles are in flight
    wait_vmcnt_le<IPT>(min(NS - 2, nblk - 1 - blk) * IPT);
    barrier_lds();  // tile blk visible; every wave is done with tile blk-1
    if (blk + NS - 1 < nblk) issue_tile(blk + NS - 1);  // into the stage of tile blk-1
    const int key0 = (t_begin + blk) * BN;
    // wave-uniform: the tile holds no key this wave's queries may see
    if (key0 >= wkv_end || key0 + BN <= wkv_begin) continue;
    const __bf16* Ks = smem + (blk % NS) * 2 * TILE_E;
    const __bf16* Vs = Ks + TILE_E;
    f32x16 sc0 = {}, sc1 = {};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int c = 2 * d + g;
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + i32 * D + 8 * (c ^ swz_k(i32)));
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Ks + (32 + i32) * D + 8 * (c ^ swz_k(32 + i32)));
      sc0 = mfma32(ka, qf[d], sc0);
      sc1 = mfma32(kb, qf[d], sc1);
    }
    // -inf for illegal keys, only on tiles that cross a bound of some lane of
    // the wave (key length, diagonal, or the band |i - j| <= window): key
    // key0 + pos is legal iff thr_lo <= pos <= thr, where the lane's register
    // r holds pos = 8*(r/4) + 4*g + r%4 (+32 in sc1)
    const int hi_w = min(Lkv - 1, min(p.causal ? qw0 : kFar, BAND ? qw0 + window : kFar));
    const int lo_w = BAND ? qw0 + 31 - window : -kFar;
    if (key0 + BN - 1 > hi_w || key0 < lo_w) {
      const int lim = min(Lkv - 1, min(p.causal ? qi : kFar, BAND ? qi + window : kFar));
      const int thr = lim - key0 - 4 * g;
      const int thr_lo = BAND ? qi - window - key0 - 4 * g : -kFar;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = 8 * (r >> 2) + (r & 3);
        if (pos > thr || (BAND && pos < thr_lo)) sc0[r] = -INFINITY;
        if (pos + 32 > thr || (BAND && pos + 32 < thr_lo)) sc1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(sc0[0], sc1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, sc0[r]), sc1[r]);
    mx = max_with_partner(mx) * c2;
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m;
      // lanes that keep their shift use alpha = 1: exp2(m - m) would be NaN
      // for a lane with no legal key yet (m = -inf)
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // m = -inf: 0
      l *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= alpha;
        o1[r] *= alpha;
      }
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int blkq = 0; blkq < 4; ++blkq) {
      const int jb = blkq >> 1, s = blkq & 1;
      const f32x16& sc = jb ? sc1 : sc0;
      bf16x4 part[2][2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 32 * jb + 16 * s + 8 * hh + tr_row;
        const __bf16* vrow = Vs + row * D + tr_half;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          part[cb][hh] = tr_read(vrow + 8 * ((4 * cb + tr_chunk) ^ swz_v(row)));
      }
      bf16x2 pp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x2 e = {__builtin_amdgcn_exp2f(fmaf(sc[8 * s + 2 * t], c2, -m_use)),
                         __builtin_amdgcn_exp2f(fmaf(sc[8 * s + 2 * t + 1], c2, -m_use))};
        pp[t] = __builtin_convertvector(e, bf16x2);
        rs = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, rs, false);
      }
      const bf16x8 pf = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                                __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 va0 = __builtin_shufflevector(part[0][0], part[0][1], 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 va1 = __builtin_shufflevector(part[1][0], part[1][1], 0, 1, 2, 3, 4, 5, 6, 7);
      o0 = mfma32(va0, pf, o0);
      o1 = mfma32(va1, pf, o1);
    }
    l += rs;
  }

  // Epilogue: O = O^T / l, rounded once to bf16; rows without a legal key or
  // beyond the query length are zeros.  Each wave stages its 32 x 64 block in
  // its own 4 KiB of the (now idle) ring -- 16-byte chunk c of row r at
  // position c ^ (r & 7) -- and writes it out as whole 128-byte rows.
  const float lt = sum_with_partner(l);
  const bool valid = (qi < Lq) && (lt > 0.f);
  const float inv = valid ? 1.f / lt : 0.f;
  barrier_lds();  // every wave is past its last read of the ring
  __bf16* Os = smem + wave * 32 * D;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    bf16x4 w0, w1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w0[t] = (__bf16)(o0[4 * rg + t] * inv);
      w1[t] = (__bf16)(o1[4 * rg + t] * inv);
    }
    *reinterpret_cast<u32x2*>(Os + i32 * D + 8 * (rg ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, w0);
    *reinterpret_cast<u32x2*>(Os + i32 * D + 8 * ((4 + rg) ^ (i32 & 7)) + 4 * g) = __builtin_bit_cast(u32x2, w1);
  }
  if (p.lse && g == 0 && qi < p.n_q)
    store_out(p.lse + ((int64_t)b * p.heads + h) * p.n_q + qi, valid ? (m + __log2f(lt)) * LN2 : -INFINITY);
  __bf16* Ob = reinterpret_cast<__bf16*>(p.o) + b * p.os_b + h * p.os_h;
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    if (qw0 + r < p.n_q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Os + r * D + 8 * (c ^ (r & 7)));
      store_out(Ob + (int64_t)(qw0 + r) * p.os_n + 8 * c, v);
    }
  }
}

}  // namespace

int sdpa_bf16_block_m(int batch, int heads, int n_q) {
  (void)batch;
  (void)heads;
  (void)n_q;
  return 128;
}

// Four waves of 32 queries, a two-stage ring (32 KiB of LDS) and at most 128
// VGPRs: four workgroups (16 waves) per CU.  Measured on MI355X, this beats
// deeper rings (3-5 stages, fewer waves per SIMD) at every sequence length,
// the 256-key decoder included.
constexpr int kWaves = 4, kStages = 2, kWavesPerSimd = 4;

hipError_t launch_sdpa_bf16(const SdpaBf16Params& p_in, hipStream_t stream) {
  SdpaBf16Params p = p_in;
  const int bm = sdpa_bf16_block_m(p.batch, p.heads, p.n_q);
  static_assert(32 * kWaves == 128, "block size and kernel disagree");
  p.n_qblocks = (p.n_q + bm - 1) / bm;
  const int64_t grid = (int64_t)p.n_qblocks * p.batch * p.heads;
  if (grid == 0) return hipSuccess;
  if (p.window >= 0)
    return launch_kernel(sdpa_fwd_bf16_d64<kWaves, kStages, kWavesPerSimd, true>, dim3((unsigned)grid),
                         dim3(64 * kWaves), stream, p);
  return launch_kernel(sdpa_fwd_bf16_d64<kWaves, kStages, kWavesPerSimd, false>, dim3((unsigned)grid),
                       dim3(64 * kWaves), stream, p);
}

}  // namespace attn
