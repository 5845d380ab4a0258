// bf16 GEMM for the projections of multi-head attention, gfx950.
//
// C[M, N] = A[M, K] . B[K, N]  (A = activations, row-major; B = weights,
// row-major [in, out] so that the product is X.W as in the projections
// X W_i^Q, X W_i^K, X W_i^V and Concat(...) W^O of "Attention Is All You
// Need" section 3.2.2).  bf16 inputs, fp32 accumulation, one RNE rounding to
// bf16 at the store.  B may be given as up to three column panels so that the
// Q, K and V projections of self-attention run as one launch.
//
// Both kernels compute the transpose D = B^T . A^T on MFMA 32x32x16 bf16:
//   A-operand (B^T rows = output columns n): read transposed from the
//     row-major B tile in LDS with ds_read_b64_tr_b16;
//   B-operand (A^T columns = output rows m): contiguous 16-byte LDS reads;
//   accumulator lane l holds output row m = l%32 and four consecutive output
//     columns per register group.
// gemm_bf16_dma_kernel (panels a multiple of 256 wide, K a multiple of 32)
// takes the projections of the attention block; gemm_bf16_kernel (128 x 128 x
// 64 tiles staged through registers, any M, N a multiple of 8, K a multiple of
// 64) takes every other shape.  Rows m >= M are zero-filled on load and not
// stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {


constexpr int BM = 128, BNt = 128, BK = 64;
constexpr int A_ROW = BK + 8;        // 72 bf16 = 144 B per A row in LDS
constexpr int B_ROW = BNt + 16;      // 144 bf16 = 288 B per B row in LDS
constexpr int A_TILE = BM * A_ROW;
constexpr int B_TILE = BK * B_ROW;
constexpr int NT = 256;

// General-shape kernel: workgroup tile 128 (m) x 128 (n) x 64 (k), four waves
// in a 2x2 arrangement of 64x64 wave tiles, A and B tiles loaded through
// registers and double-buffered in LDS with one barrier per k-step; columns
// n >= N are zero-filled on load and not stored.  C is stored as 8-byte row
// segments.
__global__ __launch_bounds__(NT) void gemm_bf16_kernel(const GemmBf16Params p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (A_TILE + B_TILE)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;   // wave tile position (64 x 64 each)

  // Workgroup -> tile.  Workgroups go to the 8 XCDs round-robin; each XCD
  // gets a contiguous range of tiles, walked in groups of GM row tiles x all
  // column tiles so that the A rows of a group and a few B column tiles stay
  // in that XCD's L2 while the group is in flight.
  constexpr int GM = 8;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BNt - 1) / BNt;
  const int total = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((total & 7) == 0) tile = (tile & 7) * (total >> 3) + (tile >> 3);
  const int grp = tile / (GM * tiles_n);
  const int rem = tile - grp * (GM * tiles_n);
  const int gm_here = min(GM, tiles_m - grp * GM);
  const int tn = rem / gm_here, tm = grp * GM + (rem - (rem / gm_here) * gm_here);
  const int m0 = tm * BM, n0 = tn * BNt;

  const __bf16* A = reinterpret_cast<const __bf16*>(p.a);

  // staging: A tile 128x64 -> 1024 chunks of 8 bf16; B tile 64x128 -> 1024 chunks
  u32x4 ar[4], br[4];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = tid + t * NT;
      const int row = c >> 3, col = (c & 7) * 8;     // A: 128 rows x 8 chunks
      const int m = m0 + row;
      ar[t] = (m < p.M) ? *reinterpret_cast<const u32x4*>(A + (int64_t)m * p.lda + k0 + col)
                        : u32x4{0u, 0u, 0u, 0u};
      const int brow = c >> 4, bcol = (c & 15) * 8;  // B: 64 rows x 16 chunks
      const int n = n0 + bcol;
      if (n < p.N) {
        const int panel = n / p.n_panel, ncol = n - panel * p.n_panel;
        const __bf16* Bp = reinterpret_cast<const __bf16*>(p.b[panel]);
        br[t] = *reinterpret_cast<const u32x4*>(Bp + (int64_t)(k0 + brow) * p.n_panel + ncol);
      } else {
        br[t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tiles = [&](int buf) {
    __bf16* As = smem + buf * (A_TILE + B_TILE);
    __bf16* Bs = As + A_TILE;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = tid + t * NT;
      *reinterpret_cast<u32x4*>(As + (c >> 3) * A_ROW + (c & 7) * 8) = ar[t];
      *reinterpret_cast<u32x4*>(Bs + (c >> 4) * B_ROW + (c & 15) * 8) = br[t];
    }
  };

  f32x16 acc[2][2] = {};   // [n block][m block] of the wave's 64x64 (n x m) tile

  const int k16 = lane & 15, chalf = (lane >> 4) & 1;
  // both operands must pair the same k with a given (lane group, element):
  // element t of lane group g is k = 16*ks + 8*g + t on both sides
  const int tr_row = g * 8 + (k16 >> 2);
  const int tr_col = chalf * 16 + 4 * (k16 & 3);

  const int nk = p.K / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
    const __bf16* As = smem + buf * (A_TILE + B_TILE);
    const __bf16* Bs = As + A_TILE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // B-operand (A^T): lane holds output row m, k = 16*ks + 8*g + 0..7
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + mb * 32 + l32) * A_ROW + 16 * ks + 8 * g);
      // A-operand (B^T): lane holds output column n = lane%32 of the block,
      // k = 16*ks + 8*g + 0..7, read transposed from row-major B
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const __bf16* bp = Bs + (16 * ks + tr_row) * B_ROW + wn * 64 + nb * 32 + tr_col;
        const bf16x4 lo = tr_read(bp);
        const bf16x4 hi = tr_read(bp + 4 * B_ROW);
        bfr[nb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32(bfr[nb], af[mb], acc[nb][mb]);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // store: acc[nb][mb] register r -> n = n0 + wn*64 + nb*32 + 8*(r/4) + 4*g + r%4,
  //                                   m = m0 + wm*64 + mb*32 + lane%32
  __bf16* C = reinterpret_cast<__bf16*>(p.c);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= p.M) continue;
    __bf16* crow = C + (int64_t)m * p.ldc;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n0 + wn * 64 + nb * 32 + 8 * rg + 4 * g;
        if (n >= p.N) continue;
        bf16x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = (__bf16)acc[nb][mb][4 * rg + t];
        *reinterpret_cast<u32x2*>(crow + n) = __builtin_bit_cast(u32x2, w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel for the common shapes (column panels a multiple of 256 wide, K
// a multiple of 32): workgroup tile 256 (m) x 256 (n), eight waves (two per
// SIMD) in a 2 x 4 arrangement of 128 (m) x 64 (n) wave tiles (8 MFMA
// accumulators per wave: 8 MFMAs per 4 + 4 LDS reads).  K advances 32 at a
// time: the X and W slices of one step (16 KiB each) are copied global -> LDS
// by buffer_load ... lds into an S-stage ring, so S-1 steps are in flight
// while one is computed; rows past M read as zeros from the buffer range.
// LDS layouts are XOR-swizzled (no padding):
//   X slice [256 m][32 k], 64-byte rows: 16-byte chunk c of row r at position
//     c ^ ((r>>2)&3) (16 consecutive rows read one chunk each: distinct banks)
//   W slice, two halves of [32 k][128 n]: chunk c of row r at position
//     c ^ (4*(r&3)) (transposed reads touch 4 consecutive rows x 2 or 4 chunks)
constexpr int M2 = 256, N2 = 256, K2 = 32;
constexpr int X_SLICE = M2 * K2;         // bf16 elements (16 KiB)
constexpr int W_HALF = K2 * 128;         // one [32 k][128 n] half of the W slice (8 KiB)
constexpr int STAGE = X_SLICE + 2 * W_HALF;
constexpr int NWAVES = 8;
constexpr int IPW = STAGE * 2 / 1024 / NWAVES;   // 1 KiB DMA instructions per wave per stage (4)

__device__ __forceinline__ int swz_x(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_w(int r) { return 4 * (r & 3); }

template <int S>
__global__ __launch_bounds__(64 * NWAVES) void gemm_bf16_dma_kernel(const GemmBf16Params p) {
  static_assert(S >= 4 && S <= 5, "bad configuration");
  static_assert(S * STAGE >= M2 * N2, "the output tile must fit the ring");
  __shared__ __attribute__((aligned(1024))) __bf16 smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;   // wave tile: rows 128*wm.., cols 64*wn..

  // Tile order: each XCD (workgroups are dealt to the 8 XCDs round-robin)
  // gets a contiguous range of tiles, walked in groups of GM row tiles x all
  // column tiles, so the workgroups running together on one XCD share X rows
  // and W columns in its L2.
  constexpr int GM = 8;
  const int tiles_m = (p.M + M2 - 1) / M2;
  const int tiles_n = p.N / N2;
  const int total = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((total & 7) == 0) tile = (tile & 7) * (total >> 3) + (tile >> 3);
  const int grp = tile / (GM * tiles_n);
  const int rem = tile - grp * (GM * tiles_n);
  const int gm_here = min(GM, tiles_m - grp * GM);
  const int tn = rem / gm_here, tm = grp * GM + (rem - (rem / gm_here) * gm_here);
  const int m0 = tm * M2, n0 = tn * N2;

  // descriptors: X rows m0.. (rows >= M read as zeros); W panel columns n0..
  const __bf16* Xb = reinterpret_cast<const __bf16*>(p.a) + (int64_t)m0 * p.lda;
  const int rows_here = min(M2, p.M - m0);
  const uint32_t x_bytes = (uint32_t)((int64_t)(rows_here - 1) * p.lda * 2 + (int64_t)p.K * 2);
  const int panel = n0 / p.n_panel;
  // (explicit selection keeps the kernel-argument array in scalar registers)
  const uint16_t* wpanel = panel == 0 ? p.b[0] : (panel == 1 ? p.b[1] : p.b[2]);
  const __bf16* Wb = reinterpret_cast<const __bf16*>(wpanel) + (n0 - panel * p.n_panel);
  const uint32_t w_bytes = (uint32_t)((int64_t)(p.K - 1) * p.n_panel * 2 + N2 * 2);

  // per-lane DMA offsets (relative to the k-step base).  Instruction u of a
  // stage: u < 16 copies X rows 16u..16u+15 (four 16-byte chunks each);
  // otherwise w = u - 16 copies rows 4*(w%8).. of W half w/8 (columns
  // 128*(w/8)..).
  uint32_t off[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int u = wave * IPW + i;
    if (u < 16) {
      const int r = 16 * u + (lane >> 2);
      const int c = (lane & 3) ^ swz_x(r);
      off[i] = (uint32_t)(((int64_t)r * p.lda + c * 8) * 2);
    } else {
      const int w = u - 16, half = w >> 3;
      const int r = 4 * (w & 7) + (lane >> 4);
      const int c = (lane & 15) ^ swz_w(r);
      off[i] = (uint32_t)(((int64_t)r * p.n_panel + 128 * half + c * 8) * 2);
    }
  }
  const int nk = p.K / K2;
  auto issue = [&](int kt) {
    const i32x4 rx = make_rsrc(Xb + kt * K2, x_bytes > (uint32_t)(kt * K2 * 2) ? x_bytes - kt * K2 * 2 : 0u);
    const int64_t w_adv = (int64_t)kt * K2 * p.n_panel;
    const i32x4 rw = make_rsrc(Wb + w_adv, (uint32_t)((int64_t)w_bytes - w_adv * 2));
    __bf16* st = smem + (kt % S) * STAGE;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int u = wave * IPW + i;   // wave-uniform: selects, no branches
      const bool x = u < 16;
      const int w = u - 16;
      dma16(off[i], x ? rx : rw, lds_addr(st + (x ? u * 512 : X_SLICE + (w >> 3) * W_HALF + (w & 7) * 512)));
    }
  };

  f32x16 acc[2][4] = {};   // [n block][m block]

  const int k16 = lane & 15, chalf = (lane >> 4) & 1;
  const int tr_row = g * 8 + (k16 >> 2);           // + 16*ks (+4 for the second half)
  const int tr_chunk = 2 * chalf + ((k16 & 3) >> 1);  // + 4*nb + 8*(wn&1)
  const int tr_half = 4 * (k16 & 1);

  // fragments of one 16-wide k-step: X rows (MFMA B operand) and W^T rows
  // (MFMA A operand, transposed reads of the row-major W slice)
  auto load_frags = [&](int kt, int ks, bf16x8 (&xf)[4], bf16x8 (&wf)[2]) {
    const __bf16* Xs = smem + (kt % S) * STAGE;
    const __bf16* Ws = Xs + X_SLICE + (wn >> 1) * W_HALF;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 128 + mb * 32 + l32;
      const int c = 2 * ks + g;
      xf[mb] = *reinterpret_cast<const bf16x8*>(Xs + r * K2 + 8 * (c ^ swz_x(r)));
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int c = 8 * (wn & 1) + 4 * nb + tr_chunk;
      const int r0 = 16 * ks + tr_row, r1 = r0 + 4;
      const bf16x4 lo = tr_read(Ws + r0 * 128 + 8 * (c ^ swz_w(r0)) + tr_half);
      const bf16x4 hi = tr_read(Ws + r1 * 128 + 8 * (c ^ swz_w(r1)) + tr_half);
      wf[nb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // Prologue: the whole ring in flight.  In the loop, the fragments of the
  // next k-step are read before the MFMAs of the current one; the barrier of
  // step kt sits after every fragment of the step is in registers, so it also
  // frees that step's stage for step kt + S.
  int pro = 0;
#pragma unroll
  for (int t = 0; t < S; ++t)
    if (t < nk) {
      issue(t);
      ++pro;
    }
  wait_vmcnt_le<IPW>((pro - 1) * IPW);
  barrier_lds();
  bf16x8 xa[4], wa[2], xb[4], wb[2];
  load_frags(0, 0, xa, wa);
  auto mfmas = [&](const bf16x8 (&xf)[4], const bf16x8 (&wf)[2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma32(wf[nb], xf[mb], acc[nb][mb]);
  };
  for (int kt = 0; kt < nk; ++kt) {
    load_frags(kt, 1, xb, wb);
    mfmas(xa, wa);
    if (kt + 1 < nk) {
      // step kt+1 landed once at most min(S-2, nk-2-kt) newer steps are in flight
      wait_vmcnt_le<IPW>(min(S - 2, nk - 2 - kt) * IPW);
      barrier_lds();                    // every wave holds all of step kt: its stage is free
      if (kt + S < nk) issue(kt + S);   // into the stage of step kt
      load_frags(kt + 1, 0, xa, wa);
    }
    mfmas(xb, wb);
  }

  // Epilogue through LDS (the ring is idle once every wave is past the last
  // step): the tile is staged as [256 m][256 n] bf16, 512-byte rows, 16-byte
  // chunk q of row m at position q ^ (m & 31), then written out as whole rows,
  // 16 bytes per lane, 1 KiB per store instruction.
  // acc[nb][mb] register r -> n = 64*wn + 32*nb + 8*(r/4) + 4*g + r%4,
  //                           m = 128*wm + 32*mb + lane%32 (inside the tile)
  barrier_lds();
  __bf16* Cs = smem;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ml = wm * 128 + mb * 32 + l32;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = (__bf16)acc[nb][mb][4 * rg + t];
        const int q = 8 * wn + 4 * nb + rg;
        *reinterpret_cast<u32x2*>(Cs + ml * N2 + 8 * (q ^ (ml & 31)) + 4 * g) = __builtin_bit_cast(u32x2, w);
      }
    }
  }
  barrier_lds();
  __bf16* C = reinterpret_cast<__bf16*>(p.c);
  const int c = lane & 31;
#pragma unroll
  for (int i = 0; i < M2 / 2 / NWAVES; ++i) {
    const int row = 2 * (wave * (M2 / 2 / NWAVES) + i) + (lane >> 5);
    if (m0 + row < p.M) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Cs + row * N2 + 8 * (c ^ (row & 31)));
      *reinterpret_cast<u32x4*>(C + (int64_t)(m0 + row) * p.ldc + n0 + 8 * c) = v;
    }
  }
}

}  // namespace

constexpr int kStages = 4;   // three 32-k steps in flight; the output tile reuses the 128 KiB ring

bool gemm_bf16_main_supported(const GemmBf16Params& p) {
  // whole 256-column tiles inside one panel, K in 32-steps, and per-tile
  // buffer ranges within 32-bit offsets
  return p.n_panel % N2 == 0 && p.N % N2 == 0 && p.K % K2 == 0 && (int64_t)M2 * p.lda * 2 < 0x7fffffffLL &&
         (int64_t)p.K * p.n_panel * 2 < 0x7fffffffLL && p.ldc % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(p.c) & 15) == 0;   // 16-byte output stores
}

hipError_t launch_gemm_bf16(const GemmBf16Params& p, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (gemm_bf16_main_supported(p)) {
    const int64_t tiles = (int64_t)((p.M + M2 - 1) / M2) * (p.N / N2);
    return launch_kernel(gemm_bf16_dma_kernel<kStages>, dim3((unsigned)tiles), dim3(64 * NWAVES), stream, p);
  }
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BNt - 1) / BNt);
  return launch_kernel(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(NT), stream, p);
}

}  // namespace attn
