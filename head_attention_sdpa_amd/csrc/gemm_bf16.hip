// bf16 GEMM for the projections of multi-head attention, gfx950.
//
// C[M, N] = A[M, K] . B[K, N]  (A = activations, row-major; B = weights,
// row-major [in, out] so that the product is X.W as in the projections
// X W_i^Q, X W_i^K, X W_i^V and Concat(...) W^O of "Attention Is All You
// Need" section 3.2.2).  bf16 inputs, fp32 accumulation, one RNE rounding to
// bf16 at the store.  B may be given as up to three column panels so that the
// Q, K and V projections of self-attention run as one launch.
//
// The kernel computes the transpose D = B^T . A^T on MFMA 32x32x16 bf16:
//   A-operand (B^T rows = output columns n): read transposed from the
//     row-major B tile in LDS with ds_read_b64_tr_b16;
//   B-operand (A^T columns = output rows m): contiguous 16-byte LDS reads;
//   accumulator lane l holds output row m = l%32 and four consecutive output
//     columns per register group, so C is stored as 8-byte row segments.
// Workgroup tile 128 (m) x 128 (n) x 64 (k), four waves in a 2x2 arrangement
// of 64x64 wave tiles, A and B tiles double-buffered in LDS with one barrier
// per k-step.  Rows m >= M and columns n >= N are zero-filled on load and not
// stored; K must be a multiple of 64 and N a multiple of 8.

#include <hip/hip_runtime.h>
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

constexpr int BM = 128, BNt = 128, BK = 64;
constexpr int A_ROW = BK + 8;        // 72 bf16 = 144 B per A row in LDS
constexpr int B_ROW = BNt + 16;      // 144 bf16 = 288 B per B row in LDS
constexpr int A_TILE = BM * A_ROW;
constexpr int B_TILE = BK * B_ROW;
constexpr int NT = 256;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 tr_read(const __bf16* lds_elem) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_elem));
  return __builtin_bit_cast(bf16x4, v);
}

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

}  // namespace

hipError_t launch_gemm_bf16(const GemmBf16Params& p, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BNt - 1) / BNt);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
