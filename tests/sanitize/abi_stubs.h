// What the stand-in launchers of abi_stubs.cpp were last given.
#pragma once
#include "internal.h"

namespace attn {
struct Recorded {
  SdpaBf16Params sdpa_bf16;
  SdpaF32Params sdpa_f32;
  SdpaDecodeParams decode;
  SdpaBwdParams bwd;
  GemmBf16Params gemm;
  PeAddParams pe;
  GemmLnParams ln;
  int n_sdpa_bf16 = 0, n_sdpa_f32 = 0, n_decode = 0, n_bwd = 0, n_gemm = 0, n_pe = 0, n_ln = 0;
};
extern Recorded g_rec;
}  // namespace attn
