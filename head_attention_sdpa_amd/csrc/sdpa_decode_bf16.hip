// One decoding step over a key/value cache, bf16 storage, head size 64, gfx950.
//
// Autoregressive generation evaluates the decoder one position at a time
// ("Attention Is All You Need" section 3.2.3; attention-paper-guide sections
// 05 and 07+; the csdn blog, section 3.6): the n_q newest queries of each
// sequence, at positions L_kv - n_q + i, attend to the cached keys and values
// up to and including their own position (the causal mask, aligned at the end
// of the cache).  With few queries and a long cache the work is a stream over
// K and V (256 bytes per key), so the keys of each (batch, head) are split
// into chunks, one wave per chunk; the wave's 32 lane columns are the (up to
// 32) queries.  K/V tiles of 64 keys stream through an LDS-DMA ring of the
// wave's own -- no barrier, only the wave's own vmcnt waits -- and each tile
// runs the same transposed MFMA products and online softmax as the prefill
// kernel.  A chunk ends with sum_j 2^(s_j - m) V_j, its shift m (log2 units)
// and sum l, and the chunks are merged: O = sum_c 2^(m_c - M) O_c / L with
// L = sum_c 2^(m_c - M) l_c, rounded to bf16 once, plus the log-sum-exp (the
// shift cancels in O, rockcohen.cc section 3.2).
//
//   up to four chunks per (b, h): sdpa_decode_partial_bf16<NS, W> with one
//     workgroup per (batch, head) and W = chunks waves, merged through LDS;
//   more chunks: sdpa_decode_partial_bf16<NS, 0> with one single-wave
//     workgroup per (batch, head, chunk), leaving its partial result in the
//     workspace, then sdpa_decode_combine, one workgroup per (batch, head,
//     query).

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
// Chunks x (b, h) to aim for, and the ring depth.  Measured on MI355X: a
// two-stage ring (32 KiB, five single-wave workgroups per CU) streams the
// cache faster than deeper rings with fewer workgroups per CU; and fewer,
// longer chunks stream faster than many short ones (16 x 16 heads over a
// 4096-key cache with lengths U{1024..4096}: 37.0 us at 1024 workgroups
// against 42.4 us at 2048, 45.1 us at 4096 and 41.5 us at 512).
constexpr int kTargetGroups = 1024;
constexpr int kStages = 2;

// W = 0: one wave per (b, h, chunk), which leaves its partial result in the
// workspace for sdpa_decode_combine.  W = 1..4: one workgroup per (b, h) with
// one wave per chunk (W = n_chunks); the waves merge their results through
// LDS and wave 0 writes O and the log-sum-exp itself, so no second kernel
// runs.  Either way each wave streams its chunk through a ring of its own and
// waits only for its own copies.
template <int NS, int W>
__global__ __launch_bounds__(64 * (W > 0 ? W : 1)) void sdpa_decode_partial_bf16(const SdpaDecodeParams p) {
  static_assert(NS >= 2 && NS <= 6 && W >= 0 && W <= 4, "bad configuration");
  constexpr int NWAVE = W > 0 ? W : 1;
  constexpr int IPT = 16;  // DMA instructions per tile (8 K + 8 V row blocks of 8 rows)
  constexpr int RING_E = NS * 2 * TILE_E;  // one wave's ring
  __shared__ __attribute__((aligned(1024))) __bf16 lds_all[NWAVE * RING_E];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __bf16* const smem = lds_all + wave * RING_E;
  const int i32 = lane & 31, g = lane >> 5;
  const int chunk = W > 0 ? wave : (int)(blockIdx.x % (unsigned)p.n_chunks);   // W = 0: workgroup = bh * n_chunks + chunk
  const int bh = W > 0 ? (int)blockIdx.x : (int)(blockIdx.x / (unsigned)p.n_chunks);
  const int b = bh / p.heads, h = bh - b * p.heads;

  int Lkv = p.n_kv;
  if (p.seqlens_kv) Lkv = min(max(p.seqlens_kv[b], 0), p.n_kv);
  const int qi = i32;                         // query of this lane column
  const int pos = Lkv - p.n_q + qi;           // its position in the sequence
  const int kbeg = chunk * p.chunk_tiles * BN;
  const int kend = min(kbeg + p.chunk_tiles * BN, Lkv);   // this chunk's keys: [kbeg, kend)
  const int nblk = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const __bf16* Qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qs_b + h * p.qs_h;
  const __bf16* Kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ks_b + h * p.ks_h + (int64_t)kbeg * p.ks_n;
  const __bf16* Vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vs_b + h * p.vs_h + (int64_t)kbeg * p.vs_n;
  // descriptor ranges end with the last query / the chunk's last key: rows
  // past them read as zeros (the cache beyond L_kv may hold anything)
  const uint32_t q_bytes = (uint32_t)((int64_t)(p.n_q - 1) * p.qs_n * 2 + 128);
  const int nk = kend - kbeg;
  const uint32_t k_bytes = nk > 0 ? (uint32_t)((int64_t)(nk - 1) * p.ks_n * 2 + 128) : 0u;
  const uint32_t v_bytes = nk > 0 ? (uint32_t)((int64_t)(nk - 1) * p.vs_n * 2 + 128) : 0u;
  const i32x4 rs_q = make_rsrc(Qb, q_bytes);

  // DMA instruction u of a tile: row block u & 7 of K (u < 8) or V; lane l
  // fills row 8*(u&7) + l/8 at chunk position l%8 with the global chunk the
  // swizzle maps there.
  uint32_t dma_off[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const bool is_v = u >= 8;
    const int r = 8 * (u & 7) + (lane >> 3);
    const int c = (lane & 7) ^ (is_v ? swz_v(r) : swz_k(r));
    dma_off[u] = (uint32_t)(((int64_t)r * (is_v ? p.vs_n : p.ks_n) + c * 8) * 2);
  }
  auto issue_tile = [&](int t) {
    const int64_t k_adv = (int64_t)t * BN * p.ks_n, v_adv = (int64_t)t * BN * p.vs_n;
    const i32x4 rk = make_rsrc(Kb + k_adv, (uint32_t)max<int64_t>(0, (int64_t)k_bytes - 2 * k_adv));
    const i32x4 rv = make_rsrc(Vb + v_adv, (uint32_t)max<int64_t>(0, (int64_t)v_bytes - 2 * v_adv));
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const bool is_v = u >= 8;
      const __bf16* dst = smem + (t % NS) * 2 * TILE_E + (is_v ? TILE_E : 0) + (u & 7) * 512;
      dma16(dma_off[u], is_v ? rv : rk, lds_addr(dst));
    }
  };

  // Q (32 rows, rows >= n_q zero) into the last stage, then the prologue
  // tiles; the wave reads Q once at most (prologue tiles) DMAs are in flight.
  const __bf16* Qs = smem + (NS - 1) * 2 * TILE_E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_k(r);
    dma16((uint32_t)(((int64_t)r * p.qs_n + c * 8) * 2), rs_q, lds_addr(Qs + 8 * i * D));
  }
  int prologue = 0;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nblk) {
      issue_tile(t);
      ++prologue;
    }
  wait_vmcnt_le<IPT>(prologue * IPT);
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
  // key j is legal for this lane's query iff j <= pos and j < kend (the next
  // chunk's keys are counted there)
  const int lim = min(pos, kend - 1);

  for (int t = 0; t < nblk; ++t) {
    // tile t has landed once at most min(NS-2, nblk-1-t) newer tiles are in
    // flight; the wave's reads of tile t-1 are done before its stage refills
    // (the ring is the wave's own: no barrier)
    wait_vmcnt_le<IPT>(min(NS - 2, nblk - 1 - t) * IPT);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (t + NS - 1 < nblk) issue_tile(t + NS - 1);
    const int key0 = kbeg + t * BN;
    const __bf16* Ks = smem + (t % NS) * 2 * TILE_E;
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
    // -inf for illegal keys, only on tiles that reach the chunk end or the
    // newest positions: register r holds key key0 + 8*(r/4) + 4*g + r%4 (+32)
    if (key0 + BN > kend || key0 + BN - 1 > Lkv - p.n_q) {
      const int thr = lim - key0 - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = 8 * (r >> 2) + (r & 3);
        if (kp > thr) sc0[r] = -INFINITY;
        if (kp + 32 > thr) sc1[r] = -INFINITY;
      }
    }
    // online softmax with lazy, per-lane rescaling (as in the prefill kernel)
    float mx = fmaxf(sc0[0], sc1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, sc0[r]), sc1[r]);
    mx = max_with_partner(mx) * c2;
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
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
      for (int tt = 0; tt < 4; ++tt) {
        const f32x2 e = {__builtin_amdgcn_exp2f(fmaf(sc[8 * s + 2 * tt], c2, -m_use)),
                         __builtin_amdgcn_exp2f(fmaf(sc[8 * s + 2 * tt + 1], c2, -m_use))};
        pp[tt] = __builtin_convertvector(e, bf16x2);
        rs = __builtin_amdgcn_fdot2_f32_bf16(pp[tt], ones, rs, false);
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

  if constexpr (W > 0) {
    // Merge the W chunks in LDS: waves 1..W-1 leave O (32 fp32 per lane, in
    // the lane's accumulator layout), the shift m and the lane's sum l in
    // their own ring; wave 0 scales each part by 2^(m_c - M), M the largest
    // shift (a part without a legal key, m = -inf, weighs 0).
    constexpr int CMB = 32 * 64 + 128;  // floats per wave
    static_assert(CMB * 4 <= RING_E * 2, "merge area exceeds a ring");
    if constexpr (W > 1) {
      if (wave > 0) {
        float* cmb = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          *reinterpret_cast<f32x4*>(cmb + 4 * (k * 64 + lane)) = f32x4{o0[4 * k], o0[4 * k + 1], o0[4 * k + 2], o0[4 * k + 3]};
          *reinterpret_cast<f32x4*>(cmb + 4 * ((4 + k) * 64 + lane)) =
              f32x4{o1[4 * k], o1[4 * k + 1], o1[4 * k + 2], o1[4 * k + 3]};
        }
        cmb[2048 + lane] = m;
        cmb[2048 + 64 + lane] = l;
      }
      barrier_lds();
      if (wave > 0) return;
      float mm = m;
#pragma unroll
      for (int w = 1; w < W; ++w) mm = fmaxf(mm, reinterpret_cast<const float*>(lds_all + w * RING_E)[2048 + lane]);
      const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
      l *= a0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= a0;
        o1[r] *= a0;
      }
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float* cmb = reinterpret_cast<const float*>(lds_all + w * RING_E);
        const float mw = cmb[2048 + lane];
        const float aw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        l = fmaf(aw, cmb[2048 + 64 + lane], l);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(cmb + 4 * (k * 64 + lane));
          const f32x4 y = *reinterpret_cast<const f32x4*>(cmb + 4 * ((4 + k) * 64 + lane));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            o0[4 * k + t] = fmaf(aw, x[t], o0[4 * k + t]);
            o1[4 * k + t] = fmaf(aw, y[t], o1[4 * k + t]);
          }
        }
      }
      m = mm;
    }
    // O = O^T / l, rounded once to bf16; a query with no legal key gets zeros
    // and lse = -inf.  Lane (query qi, half g) holds d = 8*rg + 4*g + 0..3
    // (+32 in o1): 8-byte stores.
    const float lt = sum_with_partner(l);
    const bool valid = lt > 0.f;
    const float inv = valid ? 1.f / lt : 0.f;
    if (qi < p.n_q) {
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
      if (p.lse && g == 0) p.lse[(int64_t)bh * p.n_q + qi] = valid ? (m + __log2f(lt)) * LN2 : -INFINITY;
    }
    return;
  }

  // partial result of this chunk (a chunk without keys leaves m = -inf, l = 0)
  const float lt = sum_with_partner(l);
  if (qi < p.n_q) {
    const int64_t row = ((int64_t)bh * p.n_chunks + chunk) * p.n_q + qi;
    float* po = p.part_o + row * D;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      *reinterpret_cast<f32x4*>(po + 8 * rg + 4 * g) =
          f32x4{o0[4 * rg], o0[4 * rg + 1], o0[4 * rg + 2], o0[4 * rg + 3]};
      *reinterpret_cast<f32x4*>(po + 32 + 8 * rg + 4 * g) =
          f32x4{o1[4 * rg], o1[4 * rg + 1], o1[4 * rg + 2], o1[4 * rg + 3]};
    }
    if (g == 0) *reinterpret_cast<f32x2*>(p.part_ml + 2 * row) = f32x2{m, lt};
  }
}

// One workgroup of 64 threads per (b, h, query): thread d owns output column d.
__global__ __launch_bounds__(64) void sdpa_decode_combine(const SdpaDecodeParams p) {
  const int d = threadIdx.x;
  const int64_t idx = blockIdx.x;               // (b*H + h)*n_q + i
  const int i = (int)(idx % p.n_q);
  const int64_t bh = idx / p.n_q;
  const int b = (int)(bh / p.heads), h = (int)(bh - (int64_t)b * p.heads);
  const float* ml = p.part_ml + 2 * (bh * p.n_chunks * p.n_q + i);
  float mm = -INFINITY;
  for (int c = 0; c < p.n_chunks; ++c) mm = fmaxf(mm, ml[2 * (int64_t)c * p.n_q]);
  float L = 0.f, acc = 0.f;
  if (mm != -INFINITY) {
    const float* po = p.part_o + (bh * p.n_chunks * p.n_q + i) * D + d;
    for (int c = 0; c < p.n_chunks; ++c) {
      const float mc = ml[2 * (int64_t)c * p.n_q];
      if (mc == -INFINITY) continue;            // no legal key in this chunk
      const float f = __builtin_amdgcn_exp2f(mc - mm);
      L = fmaf(f, ml[2 * (int64_t)c * p.n_q + 1], L);
      acc = fmaf(f, po[(int64_t)c * p.n_q * D], acc);
    }
  }
  const bool valid = L > 0.f;
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.os_b + h * p.os_h + (int64_t)i * p.os_n;
  orow[d] = (__bf16)(valid ? acc / L : 0.f);
  if (p.lse && d == 0) p.lse[idx] = valid ? (mm + __log2f(L)) * LN2 : -INFINITY;
}

}  // namespace

void sdpa_decode_plan(int batch, int heads, int n_kv, int* chunk_tiles, int* n_chunks) {
  const int tiles = n_kv > 0 ? (n_kv + BN - 1) / BN : 1;
  const int64_t bh = (int64_t)batch * heads;
  int64_t want = (kTargetGroups + bh - 1) / bh;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  const int ct = (int)((tiles + want - 1) / want);
  *chunk_tiles = ct;
  *n_chunks = (tiles + ct - 1) / ct;
}

hipError_t launch_sdpa_decode_bf16(const SdpaDecodeParams& p, hipStream_t stream) {
  const int64_t bh = (int64_t)p.batch * p.heads;
  if (bh == 0 || p.n_q == 0) return hipSuccess;
  // up to four chunks per (b, h): one workgroup per (b, h), merged in LDS
  const dim3 g1((unsigned)bh);
  switch (p.n_chunks) {
    case 1: return launch_kernel(sdpa_decode_partial_bf16<kStages, 1>, g1, dim3(64), stream, p);
    case 2: return launch_kernel(sdpa_decode_partial_bf16<kStages, 2>, g1, dim3(128), stream, p);
    case 3: return launch_kernel(sdpa_decode_partial_bf16<kStages, 3>, g1, dim3(192), stream, p);
    case 4: return launch_kernel(sdpa_decode_partial_bf16<kStages, 4>, g1, dim3(256), stream, p);
    default: break;
  }
  const hipError_t e =
      launch_kernel(sdpa_decode_partial_bf16<kStages, 0>, dim3((unsigned)(bh * p.n_chunks)), dim3(64), stream, p);
  if (e != hipSuccess) return e;
  return launch_kernel(sdpa_decode_combine, dim3((unsigned)(bh * p.n_q)), dim3(64), stream, p);
}

}  // namespace attn
