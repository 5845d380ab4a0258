// Device helpers shared by the library's gfx950 kernels (not installed).
//
//   - vector types of the MFMA operands and accumulators;
//   - the MFMA 32x32x16 and 16x16x32 bf16 products and the transposed LDS
//     read;
//   - global -> LDS copies (LDS DMA): 16 bytes per lane, lane i of the wave
//     lands at M0 + 16*i, addressed through a raw buffer descriptor whose
//     range makes reads past it return zeros.  They are issued from inline
//     assembly and waited for with explicit vmcnt counts, so the compiler
//     never inserts its own conservative "all DMA done" waits in front of
//     LDS reads, which would drain a prefetch ring every iteration;
//   - cross-lane reductions between lanes l and l^32 or l^16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16 (lane layouts checked by a probe on gfx950):
//   A[32 x 16]: lane l holds row l%32, k = 8*(l/32) + 0..7
//   B[16 x 32]: lane l holds col l%32, k = 8*(l/32) + 0..7
//   C[32 x 32]: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, col l%32
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 (lane layouts checked by a probe on gfx950):
//   A[16 x 32]: lane l holds row l%16, k = 8*(l/16) + 0..7
//   B[32 x 16]: lane l holds col l%16, k = 8*(l/16) + 0..7
//   C[16 x 16]: lane l, register r holds row 4*(l/16) + r, col l%16
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: per group of 16 lanes where lane k points at 4 values
// M[k][0..3], lane i receives M[i/4][i%4], M[4+i/4][i%4], M[8+i/4][i%4],
// M[12+i/4][i%4].
__device__ __forceinline__ bf16x4 tr_read(const __bf16* lds_elem) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_elem));
  return __builtin_bit_cast(bf16x4, v);
}

// Raw buffer descriptor: 48-bit base, stride 0, range in bytes; reads at or
// past the range return zeros.  The descriptor must live in scalar registers:
// every input is wave-uniform, and readfirstlane says so to the compiler.
// When the compiler computes a word with a vector instruction it moves it to
// a scalar register with v_readfirstlane, and a buffer instruction that reads
// a scalar register written by a vector instruction needs five wait states
// first (GFX9 family).  The copies below are issued from inline assembly,
// where the compiler cannot add them, so every word is passed through a
// scalar move: its last writer is then a scalar instruction.
__device__ __forceinline__ int sgpr_word(int x) {
  int y;
  asm volatile("s_mov_b32 %0, %1" : "=s"(y) : "s"(x));
  return y;
}
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{sgpr_word(__builtin_amdgcn_readfirstlane((int)(uint32_t)a)),
               sgpr_word(__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff)),
               sgpr_word(__builtin_amdgcn_readfirstlane((int)bytes)), 0x00020000};
}

// One global -> LDS copy: this lane's 16 bytes at buffer offset voff land at
// LDS address lds_addr + 16 * lane.  The wait state between the write of M0
// and the copy that reads it is the one the GFX9 family asks for (the
// compiler does not look into the assembly to add it).
__device__ __forceinline__ void dma16(uint32_t voff, i32x4 rsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

// The same copy with the non-temporal hint: the lines are marked for early
// eviction from L2, for data read once that should not displace data that
// other workgroups are about to read again.
__device__ __forceinline__ void dma16_nt(uint32_t voff, i32x4 rsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               ::"v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n (a multiple of Step, n <= 6*Step) copies are in flight
template <int Step>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n <= 0) wait_vmcnt<0>();
  else if (n <= Step) wait_vmcnt<Step>();
  else if (n <= 2 * Step) wait_vmcnt<2 * Step>();
  else if (n <= 3 * Step) wait_vmcnt<3 * Step>();
  else if (n <= 4 * Step) wait_vmcnt<4 * Step>();
  else if (n <= 5 * Step) wait_vmcnt<5 * Step>();
  else wait_vmcnt<6 * Step>();
}
// The wave's own LDS accesses are complete, then all waves meet.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Value held by lane l^32, combined with the own value.
__device__ __forceinline__ float max_with_partner(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The same with lane l^16 (gfx950 v_permlane16_swap).
__device__ __forceinline__ float max_with_lane16(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_lane16(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_with_partner(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Stores of a kernel's outputs with the "nt sc1" cache policy: device-scope
// write-through with a streaming hint.  A plain store leaves the line dirty in
// the XCD's L2 until the writeback at the end of the kernel, which then sits
// at the tail of a short kernel; these stores send the line on its way at
// once.  The attention forward writes O and the lse with them (measured,
// cold: decoder [32,8,256,64] causal 11.7 -> 10.9 us, encoder [32,8,128,64]
// 7.1 -> 6.1 us; no change inside the projection block).  For the 8-byte
// partial-row stores of the backward and decode kernels and for the GEMM
// outputs they were slower, so those keep plain stores.  The stores are
// issued from inline assembly, so the compiler does not count them among its
// own memory operations: a kernel issues them after its last global load, so
// that no wait the compiler inserts has to cover them, and only for final
// results that the same kernel does not read back.  The compiler's hazard
// checks do not see into the assembly either: a store of more than 64 bits
// must be followed by two wait states before a vector ALU instruction may
// overwrite its data registers, so the 16-byte form carries its own s_nop.
__device__ __forceinline__ void store_out(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_out(void* p, u32x2 v) {
  asm volatile("global_store_dwordx2 %0, %1, off nt sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_out(void* p, float v) {
  asm volatile("global_store_dword %0, %1, off nt sc1" ::"v"(p), "v"(v) : "memory");
}

// Attention K/V tile layout in LDS: 64 rows x 128 B, no padding; the 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r), so that the lane
// patterns of the two readers hit distinct banks:
//   K (rows of 16 consecutive keys, one chunk each):  swz = (r >> 1) & 7
//   V (transposed reads of 4 rows x 2 or 4 chunks):    swz = ((r >> 1) & 1) << 2
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v(int r) { return ((r >> 1) & 1) << 2; }

}  // namespace
}  // namespace attn
