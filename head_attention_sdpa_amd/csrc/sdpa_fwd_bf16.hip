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
// Per 64-key tile every wave computes, for its 32 queries,
//     S^T[64 keys x 32 queries] = K_tile . Q^T     (8 x mfma 32x32x16 bf16)
//     online softmax on S^T                        (VALU, exp2)
//     O^T[64 x 32] += V_tile^T . P^T               (8 x mfma 32x32x16 bf16)
// Computing the transposes puts one query in each lane column of the
// accumulators (lane l holds query l%32; lanes l and l^32 split the keys), so
// the row max needs a single cross-lane swap per tile, the row sum stays per
// lane until the end, and the S accumulator is already the P^T operand of the
// second product without any data movement.  V stays row-major in LDS; its
// transposed operand is read with ds_read_b64_tr_b16.
//
// The streaming kernel below uses that tile step; the short-sequence kernel
// uses the same computation on 16 queries per wave (16x16x32 MFMAs).
// Kernels:
//   sdpa_fwd_bf16_d64           workgroup = (batch, head, 128 queries); the
//                               keys stream through a two-stage LDS ring.
//   sdpa_fwd_bf16_d64_resident  short sequences (n_q <= 256, n_kv <= 384):
//                               workgroup = (batch, head), 16 queries per
//                               wave; every key and value of the head is
//                               copied into LDS at once.
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
constexpr int BN = 64;        // keys per tile
constexpr int TILE_E = BN * D;
constexpr float LN2 = 0.69314718055994530942f;
constexpr int kFar = 1 << 30;

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

// Per-wave state: the 32 queries' output accumulators O^T (keys 0-31 and
// 32-63 of d in o0/o1 as the MFMA C layout holds them), the running shift m
// (log2 units) and the lane's part of the row sum l.
struct WaveState {
  f32x16 o0, o1;
  float m, l;
};

// Lane constants of the wave's reads.
struct Lanes {
  int i32, g;                     // query column, key half
  int tr_row, tr_chunk, tr_half;  // transposed V reads
};

__device__ __forceinline__ Lanes lanes_of(int lane) {
  Lanes L;
  L.i32 = lane & 31;
  L.g = lane >> 5;
  const int k16 = lane & 15, chalf = (lane >> 4) & 1;
  L.tr_row = L.g * 4 + (k16 >> 2);
  L.tr_chunk = 2 * chalf + ((k16 & 3) >> 1);
  L.tr_half = 4 * (k16 & 1);
  return L;
}

// Q^T operand from the wave's 32 staged query rows (K-tile swizzle): lane
// holds query i32, d = 16*dstep + 8*g + 0..7.
__device__ __forceinline__ void load_q(const __bf16* Qs, const Lanes& L, bf16x8 (&qf)[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int c = 2 * d + L.g;
    qf[d] = *reinterpret_cast<const bf16x8*>(Qs + L.i32 * D + 8 * (c ^ swz_k(L.i32)));
  }
}

// One 64-key tile (K at Ks, V at Vs in LDS) for the wave's 32 queries.
// `masked` (wave-uniform) says that some lane of the wave has an illegal key
// in the tile.  Register r of a lane holds key key0 + 4*g + pos with
// pos = 8*(r/4) + r%4 (+32 in sc1); that key is legal iff pos <= thr and,
// with BAND, pos >= thr_lo: the lane's bounds relative to key0 + 4*g.
template <bool BAND>
__device__ __forceinline__ void attend_tile(const __bf16* Ks, const __bf16* Vs, const bf16x8 (&qf)[4],
                                            bool masked, int thr, int thr_lo, float c2, const Lanes& L,
                                            WaveState& st) {
  f32x16 sc0 = {}, sc1 = {};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int c = 2 * d + L.g;
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + L.i32 * D + 8 * (c ^ swz_k(L.i32)));
    const bf16x8 kb =
        *reinterpret_cast<const bf16x8*>(Ks + (32 + L.i32) * D + 8 * (c ^ swz_k(32 + L.i32)));
    sc0 = mfma32(ka, qf[d], sc0);
    sc1 = mfma32(kb, qf[d], sc1);
  }
  if (masked) {
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
  // lazy rescale: the shift moves only when the tile max exceeds it by 8
  // (log2 units); exact by shift invariance, weights stay <= 2^8
  const bool grow = mx > st.m + 8.f;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = grow ? mx : st.m;
    // lanes that keep their shift use alpha = 1: exp2(m - m) would be NaN
    // for a lane with no legal key yet (m = -inf)
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;  // m = -inf: 0
    st.l *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st.o0[r] *= alpha;
      st.o1[r] *= alpha;
    }
    st.m = m_new;
  }
  const float m_use = (st.m == -INFINITY) ? 0.f : st.m;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float rs = 0.f;
#pragma unroll
  for (int blkq = 0; blkq < 4; ++blkq) {
    const int jb = blkq >> 1, s = blkq & 1;
    const f32x16& sc = jb ? sc1 : sc0;
    bf16x4 part[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 32 * jb + 16 * s + 8 * hh + L.tr_row;
      const __bf16* vrow = Vs + row * D + L.tr_half;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        part[cb][hh] = tr_read(vrow + 8 * ((4 * cb + L.tr_chunk) ^ swz_v(row)));
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
    st.o0 = mfma32(va0, pf, st.o0);
    st.o1 = mfma32(va1, pf, st.o1);
  }
  st.l += rs;
}

// Epilogue of one wave: O = O^T / l, rounded once to bf16; rows without a
// legal key or beyond the query length are zeros.  The wave stages its
// 32 x 64 block in 4 KiB of LDS that no other wave touches (16-byte chunk c of
// row r at position c ^ (r & 7)) and writes it out as whole 128-byte rows.
// Writes rows qw0 .. qw0+31 below n_q, and their lse when asked.
__device__ __forceinline__ void write_rows(const SdpaBf16Params& p, const WaveState& st, __bf16* Os,
                                           int b, int h, int qw0, int Lq, int lane, const Lanes& L) {
  const int qi = qw0 + L.i32;
  const float lt = sum_with_partner(st.l);
  const bool valid = (qi < Lq) && (lt > 0.f);
  const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    bf16x4 w0, w1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w0[t] = (__bf16)(st.o0[4 * rg + t] * inv);
      w1[t] = (__bf16)(st.o1[4 * rg + t] * inv);
    }
    *reinterpret_cast<u32x2*>(Os + L.i32 * D + 8 * (rg ^ (L.i32 & 7)) + 4 * L.g) =
        __builtin_bit_cast(u32x2, w0);
    *reinterpret_cast<u32x2*>(Os + L.i32 * D + 8 * ((4 + rg) ^ (L.i32 & 7)) + 4 * L.g) =
        __builtin_bit_cast(u32x2, w1);
  }
  if (p.lse && L.g == 0 && qi < p.n_q)
    store_out(p.lse + ((int64_t)b * p.heads + h) * p.n_q + qi,
              valid ? (st.m + __log2f(lt)) * LN2 : -INFINITY);
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

// Copies 32 query rows starting at row qw0 (K-tile swizzle) into Qs: 4 KiB,
// four 1 KiB copies of 8 rows.
template <bool NT_HINT>
__device__ __forceinline__ void copy_q(const i32x4& rs_q, int64_t qs_n, int qw0, int lane, const __bf16* Qs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_k(r);
    const uint32_t voff = (uint32_t)(((int64_t)(qw0 + r) * qs_n + chunk * 8) * 2);
    if (NT_HINT)
      dma16_nt(voff, rs_q, lds_addr(Qs + 8 * i * D));
    else
      dma16(voff, rs_q, lds_addr(Qs + 8 * i * D));
  }
}

// Byte offset and LDS slot of copy u (0..15) of a K/V tile for this lane:
// copies 0-7 are K rows 8u..8u+7, copies 8-15 V rows 8(u-8)..; each lane
// moves one 16-byte chunk, stored swizzled.
__device__ __forceinline__ uint32_t kv_copy_offset(int u, int lane, int64_t ks_n, int64_t vs_n) {
  const bool is_v = u >= 8;
  const int r = 8 * (u & 7) + (lane >> 3);
  const int chunk = (lane & 7) ^ (is_v ? swz_v(r) : swz_k(r));
  return (uint32_t)(((int64_t)r * (is_v ? vs_n : ks_n) + chunk * 8) * 2);
}
__device__ __forceinline__ int kv_copy_slot(int u) { return (u >= 8 ? TILE_E : 0) + (u & 7) * 512; }

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
  constexpr int IPT = 16 / NW;
  static_assert(IPT * NW == 16 && NS >= 2 && NS <= 6, "bad configuration");
  static_assert(NW * 32 * D <= 2 * TILE_E, "the Q rows must fit in one ring stage");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NS * 2 * TILE_E];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes L = lanes_of(lane);

  int bh, qb;
  map_block(blockIdx.x, p.batch * p.heads, p.n_qblocks, p.causal, bh, qb);
  const int b = bh / p.heads, h = bh - b * p.heads;

  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  const int q0 = qb * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + L.i32;
  // keys this workgroup / this wave needs: [kv_begin, kv_end) and
  // [wkv_begin, wkv_end) (queries >= Lq are zeros: need nothing)
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
  for (int i = 0; i < IPT; ++i) dma_off[i] = kv_copy_offset(wave * IPT + i, lane, p.ks_n, p.vs_n);
  auto issue_tile = [&](int j) {  // the workgroup's j-th tile, key tile t_begin + j, into stage j % NS
    const int t = t_begin + j;
    const int64_t k_adv = (int64_t)t * BN * p.ks_n, v_adv = (int64_t)t * BN * p.vs_n;
    const i32x4 rk = make_rsrc(Kb + k_adv, (uint32_t)max<int64_t>(0, (int64_t)k_bytes - 2 * k_adv));
    const i32x4 rv = make_rsrc(Vb + v_adv, (uint32_t)max<int64_t>(0, (int64_t)v_bytes - 2 * v_adv));
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = wave * IPT + i;
      dma16(dma_off[i], u >= 8 ? rv : rk, lds_addr(smem + (j % NS) * 2 * TILE_E + kv_copy_slot(u)));
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
  copy_q<BAND>(rs_q, p.qs_n, qw0, lane, Qs);
  int prologue = 0;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nblk) {
      issue_tile(t);
      ++prologue;
    }
  wait_vmcnt_le<IPT>(prologue * IPT);
  bf16x8 qf[4];
  load_q(Qs, L, qf);

  WaveState st;
  st.o0 = f32x16{};
  st.o1 = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  // -inf for illegal keys, only on tiles that cross a bound of some lane of
  // the wave (key length, diagonal, or the band |i - j| <= window)
  const int hi_w = min(Lkv - 1, min(p.causal ? qw0 : kFar, BAND ? qw0 + window : kFar));
  const int lo_w = BAND ? qw0 + 31 - window : -kFar;
  const int lim = min(Lkv - 1, min(p.causal ? qi : kFar, BAND ? qi + window : kFar));
  const int lim_lo = BAND ? qi - window : -kFar;

  for (int blk = 0; blk < nblk; ++blk) {
    // tile blk has landed once at most min(NS-2, nblk-1-blk) newer tiles are in flight
    wait_vmcnt_le<IPT>(min(NS - 2, nblk - 1 - blk) * IPT);
    barrier_lds();  // tile blk visible; every wave is done with tile blk-1
    if (blk + NS - 1 < nblk) issue_tile(blk + NS - 1);  // into the stage of tile blk-1
    const int key0 = (t_begin + blk) * BN;
    // wave-uniform: the tile holds no key this wave's queries may see
    if (key0 >= wkv_end || key0 + BN <= wkv_begin) continue;
    const __bf16* Ks = smem + (blk % NS) * 2 * TILE_E;
    const bool masked = key0 + BN - 1 > hi_w || key0 < lo_w;
    attend_tile<BAND>(Ks, Ks + TILE_E, qf, masked, lim - key0 - 4 * L.g, lim_lo - key0 - 4 * L.g,
                      p.scale_log2, L, st);
  }

  barrier_lds();  // every wave is past its last read of the ring
  write_rows(p, st, smem + wave * 32 * D, b, h, qw0, Lq, lane, L);
}

// ---------------------------------------------------------------------------
// Short sequences: 16 queries per wave on v_mfma_f32_16x16x32_bf16.
//
// Per 64-key tile a wave computes S^T[64 keys x 16 queries] as four 16-key
// blocks (8 MFMAs over d = 64), the online softmax on its 16 scores per lane,
// and O^T[64 d x 16 queries] += V^T . P^T (8 MFMAs over the 64 keys).  Lane l
// holds query l%16; the four lane groups G = l/16 hold keys 16*blk + 4*G + r
// (register r of block blk), so the row max needs two cross-lane swaps (l^16,
// l^32).  In the second product the keys of a 32-key step are taken in the
// order the S accumulator holds them (block 2s then 2s+1, registers 0..3 of
// lane group G), so P^T needs no data movement; the V^T operand is read in
// the same key order with two ds_read_b64_tr_b16 per d-block.
// ---------------------------------------------------------------------------

// V tile swizzle of this kernel: the transposed reads of one instruction
// touch 16 rows x 32 bytes, so 32-byte slots are permuted by (r >> 2) & 3.
__device__ __forceinline__ int swz_v16(int r) { return ((r >> 2) & 3) << 1; }

struct WaveState16 {
  f32x4 o[4];  // O^T d-blocks: lane l, register r holds d = 16*db + 4*(l/16) + r of query l%16
  float m, l;
};

// One 64-key tile for the wave's 16 queries.  `masked` (wave-uniform): some
// lane has an illegal key in the tile; register r of block blk holds key
// key0 + 4*G + 16*blk + r, legal iff 16*blk + r <= thr (the lane's bound
// relative to key0 + 4*G).
__device__ __forceinline__ void attend_tile16(const __bf16* Ks, const __bf16* Vs, const bf16x8 (&qf)[2],
                                              bool masked, int thr, float c2, int q16, int G,
                                              WaveState16& st) {
  f32x4 sc[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int row = 16 * blk + q16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + row * D + 8 * ((4 * kk + G) ^ swz_k(row)));
      sc[blk] = mfma16(ka, qf[kk], sc[blk]);
    }
  }
  if (masked) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * blk + r > thr) sc[blk][r] = -INFINITY;
  }
  const float m01 = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                          fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  const float m23 = fmaxf(fmaxf(fmaxf(sc[2][0], sc[2][1]), fmaxf(sc[2][2], sc[2][3])),
                          fmaxf(fmaxf(sc[3][0], sc[3][1]), fmaxf(sc[3][2], sc[3][3])));
  const float mx = max_with_partner(max_with_lane16(fmaxf(m01, m23))) * c2;
  // lazy rescale, as in the 32-query tile step
  const bool grow = mx > st.m + 8.f;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = grow ? mx : st.m;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
    st.m = m_new;
  }
  const float m_use = (st.m == -INFINITY) ? 0.f : st.m;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x2 pp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4& sb = sc[2 * ks + (t >> 1)];
      const int r = 2 * (t & 1);
      const f32x2 e = {__builtin_amdgcn_exp2f(fmaf(sb[r], c2, -m_use)),
                       __builtin_amdgcn_exp2f(fmaf(sb[r + 1], c2, -m_use))};
      pp[t] = __builtin_convertvector(e, bf16x2);
      if (t & 1)
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, rs1, false);
      else
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones, rs0, false);
    }
    const bf16x8 pf = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                              __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3),
                                              0, 1, 2, 3, 4, 5, 6, 7);
    // V^T rows d = 16*db + q16, keys 32*ks + 4*G + 0..3 and 32*ks + 16 + 4*G + 0..3
    const int row0 = 32 * ks + 4 * G + (q16 >> 2), row1 = row0 + 16;
    const int cq = (q16 & 3) >> 1, hq = 4 * (q16 & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int c = 2 * db + cq;
      const bf16x4 v0 = tr_read(Vs + row0 * D + 8 * (c ^ swz_v16(row0)) + hq);
      const bf16x4 v1 = tr_read(Vs + row1 * D + 8 * (c ^ swz_v16(row1)) + hq);
      st.o[db] = mfma16(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7), pf, st.o[db]);
    }
  }
  st.l += rs0 + rs1;
}

// Epilogue of a 16-query wave: O = O^T / l rounded once to bf16 (zeros for
// rows without a legal key or beyond the query length), staged in the wave's
// 2 KiB of LDS (chunk c of row r at c ^ (r & 7)) and written as whole rows.
__device__ __forceinline__ void write_rows16(const SdpaBf16Params& p, const WaveState16& st, __bf16* Os,
                                             int b, int h, int qw0, int Lq, int lane) {
  const int q16 = lane & 15, G = lane >> 4;
  const int qi = qw0 + q16;
  const float lt = sum_with_partner(sum_with_lane16(st.l));
  const bool valid = (qi < Lq) && (lt > 0.f);
  const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    bf16x4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = (__bf16)(st.o[db][r] * inv);
    const int c = 2 * db + (G >> 1);
    *reinterpret_cast<u32x2*>(Os + q16 * D + 8 * (c ^ (q16 & 7)) + 4 * (G & 1)) = __builtin_bit_cast(u32x2, w);
  }
  if (p.lse && G == 0 && qi < p.n_q)
    store_out(p.lse + ((int64_t)b * p.heads + h) * p.n_q + qi,
              valid ? (st.m + __log2f(lt)) * LN2 : -INFINITY);
  __bf16* Ob = reinterpret_cast<__bf16*>(p.o) + b * p.os_b + h * p.os_h;
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    if (qw0 + r < p.n_q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Os + r * D + 8 * (c ^ (r & 7)));
      store_out(Ob + (int64_t)(qw0 + r) * p.os_n + 8 * c, v);
    }
  }
}

// One workgroup = one (batch, head) of a short sequence: NW waves of 16
// queries (n_q <= 16*NW), every key tile of the head resident in LDS (NT
// tiles of 64 keys, n_kv <= 64*NT), nothing ever refilled.
//
// Copies: Q and tile 0 at the start, then tile t+1 right after the barrier
// that publishes tile t, so one tile per head is in flight while tile t is
// computed.  Measured on the decoder shape [32,8,256,64], issuing more at
// once is slower, down to everything at the start (9.7 -> 11.1 us): all 256
// heads' requests then interleave in HBM and tile 0 of a head completes only
// near the end of the whole load, while with one tile in flight the tiles
// arrive in the order they are needed.  A tile is copied only by the waves
// that need it (its 16 copies of 1 KiB dealt round-robin over them), so a
// wave's only outstanding copies when it waits for tile t are its copies of
// tile t: it waits for all of them (vmcnt 0), then the waves meet at the
// barrier.  A wave writes its rows right after its last tile and then only
// meets the remaining barriers, never waiting on the vector memory counter
// again -- the output stores count there too, and a wait on them would hold
// up the others at the next barrier.
//
// With the causal mask group g needs tiles 0..g/4 (at least as many as group
// g-1); the waves that share a SIMD (w, w+4, w+8, w+12) then get the same
// number of tile steps, 1+2+3+4 at n = 256.
template <int NT, int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_bf16_d64_resident(const SdpaBf16Params p) {
  static_assert(NT >= 1 && NT <= 6 && (NW == 8 || NW == 16), "bad configuration");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[NT * 2 * TILE_E + NW * 16 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q16 = lane & 15, G = lane >> 4;

  const int bh = blockIdx.x;
  const int b = bh / p.heads, h = bh - b * p.heads;
  int Lq = p.n_q, Lkv = p.n_kv;
  if (p.seqlens_q) Lq = min(max(p.seqlens_q[b], 0), p.n_q);
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);

  const int qw0 = 16 * wave;
  const int qi = qw0 + q16;
  // tiles of the workgroup and of this wave (queries >= Lq need none)
  const int kv_end = Lq == 0 ? 0 : (p.causal ? min(Lkv, Lq) : Lkv);
  const int nt = (kv_end + BN - 1) / BN;
  const int wkv_end = qw0 >= Lq ? 0 : (p.causal ? min(Lkv, min(qw0 + 16, Lq)) : Lkv);
  const int wnt = (wkv_end + BN - 1) / BN;
  // the waves that need tile t < nt are groups [first(t), gact): every
  // active group without the mask, groups from 4t on with it (for t < nt,
  // 64t < min(Lkv, Lq), so group g needs tile t iff 16g + 16 > 64t)
  const int gact = min(NW, (Lq + 15) / 16);

  const __bf16* Qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h;
  const __bf16* Vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h;
  const uint32_t q_bytes = Lq > 0 ? (uint32_t)((int64_t)(Lq - 1) * p.qs_n * 2 + 128) : 0u;
  const uint32_t k_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.ks_n * 2 + 128) : 0u;
  const uint32_t v_bytes = Lkv > 0 ? (uint32_t)((int64_t)(Lkv - 1) * p.vs_n * 2 + 128) : 0u;
  const i32x4 rk = make_rsrc(Kb, k_bytes);
  const i32x4 rv = make_rsrc(Vb, v_bytes);

  // this wave's copies of tile t: copy u (0-7 K rows 8u.., 8-15 V rows
  // 8(u-8)..) for u = rank, rank + count, ... below 16
  auto copy_tile = [&](int t) {
    const int first = p.causal ? 4 * t : 0;
    const int count = gact - first, rank = wave - first;
    for (int u = rank; u < 16; u += count) {
      const bool is_v = u >= 8;
      const int r = 8 * (u & 7) + (lane >> 3);
      const int chunk = (lane & 7) ^ (is_v ? swz_v16(r) : swz_k(r));
      const int64_t stride = is_v ? p.vs_n : p.ks_n;
      dma16((uint32_t)((((int64_t)t * BN + r) * stride + chunk * 8) * 2), is_v ? rv : rk,
            lds_addr(smem + t * 2 * TILE_E + (is_v ? TILE_E : 0) + (u & 7) * 512));
    }
  };

  // Q rows qw0..qw0+15 (two copies of 8 rows, K-tile swizzle), then tile 0
  __bf16* Qs = smem + NT * 2 * TILE_E + wave * 16 * D;
  if (wnt > 0) {
    const i32x4 rs_q = make_rsrc(Qb, q_bytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ swz_k(r);
      dma16((uint32_t)(((int64_t)(qw0 + r) * p.qs_n + chunk * 8) * 2), rs_q, lds_addr(Qs + 8 * i * D));
    }
    copy_tile(0);
  }

  WaveState16 st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  const int hi_w = min(Lkv - 1, p.causal ? qw0 : kFar);
  const int lim = min(Lkv - 1, p.causal ? qi : kFar);
  bf16x8 qf[2];
  if (wnt == 0) write_rows16(p, st, Qs, b, h, qw0, Lq, lane);  // nothing to attend: zero rows
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nt) {
      if (t < wnt) wait_vmcnt<0>();  // this wave's copies of tile t (and, for t = 0, of Q) have landed
      barrier_lds();                 // every copy of tile t has landed
      if (t + 1 < wnt) copy_tile(t + 1);
      if (t < wnt) {
        if (t == 0) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(Qs + q16 * D + 8 * ((4 * kk + G) ^ swz_k(q16)));
        }
        const int key0 = t * BN;
        const __bf16* Ks = smem + t * 2 * TILE_E;
        attend_tile16(Ks, Ks + TILE_E, qf, key0 + BN - 1 > hi_w, lim - key0 - 4 * G, p.scale_log2, q16, G,
                      st);
        if (t == wnt - 1) write_rows16(p, st, Qs, b, h, qw0, Lq, lane);
      }
    }
  }
}

}  // namespace

// Queries per workgroup of the streaming kernel.
int sdpa_bf16_block_m(int batch, int heads, int n_q) {
  (void)batch;
  (void)heads;
  (void)n_q;
  return 128;
}

// Shapes the resident kernel takes: no band, at most 256 queries and 6 key
// tiles (K, V and Q then need at most 128 KiB of LDS).
bool sdpa_bf16_resident(int n_q, int n_kv, int window) {
  return window < 0 && n_q <= 256 && n_kv <= 6 * BN;
}

// Four waves of 32 queries, a two-stage ring (32 KiB of LDS) and at most 128
// VGPRs: four workgroups (16 waves) per CU.  Measured on MI355X, this beats
// deeper rings (3-5 stages, fewer waves per SIMD) at every sequence length.
constexpr int kWaves = 4, kStages = 2, kWavesPerSimd = 4;

template <int NT>
static hipError_t launch_resident(const SdpaBf16Params& p, dim3 grid, hipStream_t stream) {
  if (p.n_q <= 128)
    return launch_kernel(sdpa_fwd_bf16_d64_resident<NT, 8>, grid, dim3(512), stream, p);
  return launch_kernel(sdpa_fwd_bf16_d64_resident<NT, 16>, grid, dim3(1024), stream, p);
}

hipError_t launch_sdpa_bf16(const SdpaBf16Params& p_in, hipStream_t stream) {
  SdpaBf16Params p = p_in;
  if (sdpa_bf16_resident(p.n_q, p.n_kv, p.window)) {
    const int64_t grid = (int64_t)p.batch * p.heads;
    if (grid == 0 || p.n_q == 0) return hipSuccess;
    const int tiles = (p.n_kv + BN - 1) / BN;
    p.n_qblocks = 1;
    if (tiles <= 2) return launch_resident<2>(p, dim3((unsigned)grid), stream);
    if (tiles <= 4) return launch_resident<4>(p, dim3((unsigned)grid), stream);
    return launch_resident<6>(p, dim3((unsigned)grid), stream);
  }
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
