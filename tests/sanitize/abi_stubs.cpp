// Host-only stand-ins for the library's kernel launchers and device helpers,
// so that the C ABI's host code (validation, stride and workspace
// bookkeeping in abi.cpp) can run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Each launcher
// records the parameters it was given and reports success; nothing here
// computes attention.
#include <stdint.h>

#include "internal.h"
#include "abi_stubs.h"

namespace attn {

Recorded g_rec;

hipError_t launch_sdpa_bf16(const SdpaBf16Params& p, hipStream_t) {
  g_rec.sdpa_bf16 = p;
  ++g_rec.n_sdpa_bf16;
  return hipSuccess;
}
hipError_t launch_sdpa_f32(const SdpaF32Params& p, hipStream_t) {
  g_rec.sdpa_f32 = p;
  ++g_rec.n_sdpa_f32;
  return hipSuccess;
}
hipError_t launch_sdpa_decode_bf16(const SdpaDecodeParams& p, hipStream_t) {
  g_rec.decode = p;
  ++g_rec.n_decode;
  return hipSuccess;
}
hipError_t launch_sdpa_bwd_bf16(const SdpaBwdParams& p, hipStream_t) {
  g_rec.bwd = p;
  ++g_rec.n_bwd;
  return hipSuccess;
}
hipError_t launch_gemm_bf16(const GemmBf16Params& p, hipStream_t) {
  g_rec.gemm = p;
  ++g_rec.n_gemm;
  return hipSuccess;
}
hipError_t launch_pe_add_bf16(const PeAddParams& p, hipStream_t) {
  g_rec.pe = p;
  ++g_rec.n_pe;
  return hipSuccess;
}
hipError_t launch_gemm_bf16_ln(const GemmLnParams& p, hipStream_t) {
  g_rec.ln = p;
  ++g_rec.n_ln;
  return hipSuccess;
}
bool gemm_bf16_main_supported(const GemmBf16Params&) { return true; }
int sdpa_bf16_block_m(int, int, int) { return 128; }
bool sdpa_bf16_resident(int n_q, int n_kv, int window) { return window < 0 && n_q <= 256 && n_kv <= 384; }

// One chunk of up to 16 key tiles per (b, h): any consistent plan exercises
// the workspace bookkeeping.
void sdpa_decode_plan(int, int, int n_kv, int* chunk_tiles, int* n_chunks) {
  const int tiles = (n_kv + 63) / 64;
  *chunk_tiles = 16;
  *n_chunks = tiles > 0 ? (tiles + 15) / 16 : 1;
}

// The fixed scratch of the allocation-free backward: a host array here.
alignas(256) static char g_scratch[kBwdScratchBytes];
hipError_t bwd_scratch(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}

}  // namespace attn

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }
