// Drives every entry point of include/attn_sdpa.h through its host code with
// valid and invalid arguments, against the stand-in launchers of
// abi_stubs.cpp (no GPU).  Built with -fsanitize=address,undefined: any
// out-of-bounds access, use of uninitialised stride state, signed overflow
// in the size and offset arithmetic, misaligned access and the like is
// reported by the sanitizers; a wrong status or a wrongly marshalled launch
// is reported here.  Prints "abi driver: ok" and exits 0 when every check
// holds.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/attn_sdpa.h"
#include "abi_stubs.h"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "abi driver: check failed at line %d: %s\n", __LINE__, #cond); \
      g_fail = 1;                                                     \
    }                                                                 \
  } while (0)

// Device pointers are only carried, never dereferenced: distinct 256-byte
// aligned addresses stand in for them.
static void* dev(int i) { return reinterpret_cast<void*>((uintptr_t)0x100000 * (uintptr_t)(i + 1)); }

using attn::g_rec;

static void sdpa_calls() {
  const int B = 2, H = 3, nq = 100, nkv = 130;
  int32_t lens[2] = {100, 50};  // host memory: the library must not read lengths on the host
  // contiguous bf16, causal, with lengths and lse
  const int before = g_rec.n_sdpa_bf16;
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                      0.f, ATTN_MASK_CAUSAL, lens, lens, (float*)dev(4), NULL) == ATTN_OK);
  CHECK(g_rec.n_sdpa_bf16 == before + 1);
  CHECK(g_rec.sdpa_bf16.qs_n == 64 && g_rec.sdpa_bf16.qs_h == nq * 64 && g_rec.sdpa_bf16.qs_b == (int64_t)H * nq * 64);
  CHECK(g_rec.sdpa_bf16.ks_h == nkv * 64 && g_rec.sdpa_bf16.causal == 1 && g_rec.sdpa_bf16.window == -1);
  CHECK(g_rec.sdpa_bf16.scale_log2 > 0.18f && g_rec.sdpa_bf16.scale_log2 < 0.181f);  // (1/8) log2(e)
  // strided (a packed [B, n, H, 64] view)
  attn_strides st = {(int64_t)nq * H * 64, 64, (int64_t)H * 64};
  attn_strides sk = {(int64_t)nkv * H * 64, 64, (int64_t)H * 64};
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), &st, dev(1), &sk, dev(2), &sk, dev(3), &st, 0.5f,
                      ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_OK);
  CHECK(g_rec.sdpa_bf16.qs_n == H * 64 && g_rec.sdpa_bf16.vs_b == (int64_t)nkv * H * 64);
  // fp32 small head sizes
  CHECK(attn_sdpa_fwd(ATTN_F32, 1, 1, 16, 16, 5, 7, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL, 0.125f,
                      ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_OK);
  CHECK(g_rec.sdpa_f32.d_k == 5 && g_rec.sdpa_f32.d_v == 7 && g_rec.sdpa_f32.os_h == 16 * 7);
  // errors, nothing enqueued
  const int n0 = g_rec.n_sdpa_bf16;
  CHECK(attn_sdpa_fwd((attn_dtype)9, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                      0.f, ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_INVALID);
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, NULL, NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL, 0.f,
                      ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_INVALID);
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 32, 32, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL, 0.f,
                      ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, (char*)dev(0) + 2, NULL, dev(1), NULL, dev(2), NULL, dev(3),
                      NULL, 0.f, ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_ALIGN);
  CHECK(attn_sdpa_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                      -1.f, ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_INVALID);
  // sizes at the limits of the 32-bit offsets and of int
  CHECK(attn_sdpa_fwd(ATTN_BF16, 1, 1, INT_MAX, INT_MAX, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3),
                      NULL, 0.f, ATTN_MASK_CAUSAL, NULL, NULL, NULL, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(attn_sdpa_fwd(ATTN_BF16, INT_MAX, INT_MAX, 64, 64, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3),
                      NULL, 0.f, ATTN_MASK_NONE, NULL, NULL, NULL, NULL) == ATTN_E_UNSUPPORTED);
  CHECK(g_rec.n_sdpa_bf16 == n0);
  // restricted attention: a radius beyond every |i - j| is clamped
  CHECK(attn_sdpa_window_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                             0.f, ATTN_MASK_CAUSAL, INT_MAX, NULL, NULL, NULL, NULL) == ATTN_OK);
  CHECK(g_rec.sdpa_bf16.window == nkv);
  CHECK(attn_sdpa_window_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                             0.f, ATTN_MASK_NONE, 17, NULL, NULL, NULL, NULL) == ATTN_OK);
  CHECK(g_rec.sdpa_bf16.window == 17);
  CHECK(attn_sdpa_window_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                             0.f, ATTN_MASK_NONE, -1, NULL, NULL, NULL, NULL) == ATTN_E_INVALID);
}

static void mha_calls() {
  const int B = 2, n = 300, dm = 256, H = 4;
  const size_t ws = attn_mha_workspace_bytes(ATTN_BF16, B, n, n, dm, H, 64, 64);
  CHECK(ws == (size_t)B * n * dm * 2 * 4);
  const int g0 = g_rec.n_gemm, s0 = g_rec.n_sdpa_bf16;
  CHECK(attn_mha_fwd(ATTN_BF16, B, n, n, dm, H, 64, 64, dev(0), dev(0), dev(1), dev(2), dev(3), dev(4), dev(5), 0.f,
                     ATTN_MASK_CAUSAL, NULL, NULL, dev(6), ws, NULL) == ATTN_OK);
  CHECK(g_rec.n_gemm == g0 + 2 && g_rec.n_sdpa_bf16 == s0 + 1);   // fused QKV, then W^O
  CHECK(g_rec.sdpa_bf16.qs_n == 3 * H * 64 && g_rec.sdpa_bf16.os_n == H * 64);
  CHECK(g_rec.gemm.M == B * n && g_rec.gemm.N == dm && g_rec.gemm.K == H * 64);
  // cross-attention: separate Q and KV projections
  const size_t wsx = attn_mha_workspace_bytes(ATTN_BF16, B, n, 170, dm, H, 64, 64);
  CHECK(attn_mha_fwd(ATTN_BF16, B, n, 170, dm, H, 64, 64, dev(0), dev(7), dev(1), dev(2), dev(3), dev(4), dev(5), 0.f,
                     ATTN_MASK_NONE, NULL, NULL, dev(6), wsx, NULL) == ATTN_OK);
  CHECK(g_rec.sdpa_bf16.ks_n == 2 * H * 64 && g_rec.sdpa_bf16.n_kv == 170);
  // the head split, the workspace and the offset limits
  CHECK(attn_mha_fwd(ATTN_BF16, B, n, n, 128, H, 64, 64, dev(0), dev(0), dev(1), dev(2), dev(3), dev(4), dev(5), 0.f,
                     ATTN_MASK_CAUSAL, NULL, NULL, dev(6), ws, NULL) == ATTN_E_INVALID);
  CHECK(attn_mha_fwd(ATTN_BF16, B, n, n, dm, H, 64, 64, dev(0), dev(0), dev(1), dev(2), dev(3), dev(4), dev(5), 0.f,
                     ATTN_MASK_CAUSAL, NULL, NULL, dev(6), ws - 1, NULL) == ATTN_E_WORKSPACE);
  CHECK(attn_mha_workspace_bytes(ATTN_BF16, 1, INT_MAX, INT_MAX, 4096, 64, 64, 64) == 0);
  CHECK(attn_mha_workspace_bytes(ATTN_BF16, INT_MAX, INT_MAX, INT_MAX, 1024, 16, 64, 64) == 0);
  // the sublayer with the encoding: PE pass, projections, SDPA, W^O + LayerNorm
  const size_t wsb = attn_mha_block_workspace_bytes(ATTN_BF16, B, n, n, dm, H, 64, 64, 1);
  CHECK(wsb == ws + (size_t)B * n * dm * 2);
  const int p0 = g_rec.n_pe, l0 = g_rec.n_ln;
  CHECK(attn_mha_block_fwd(ATTN_BF16, B, n, n, dm, H, 64, 64, dev(0), dev(0), 1, dev(1), dev(2), dev(3), dev(4),
                           dev(8), dev(9), 1e-5f, dev(5), 0.f, ATTN_MASK_CAUSAL, NULL, NULL, dev(6), wsb,
                           NULL) == ATTN_OK);
  CHECK(g_rec.n_pe == p0 + 1 && g_rec.n_ln == l0 + 1 && g_rec.ln.N == dm && g_rec.ln.M == B * n);
  CHECK(attn_mha_block_fwd(ATTN_BF16, B, n, n, dm, H, 64, 64, dev(0), dev(7), 1, dev(1), dev(2), dev(3), dev(4),
                           dev(8), dev(9), 1e-5f, dev(5), 0.f, ATTN_MASK_CAUSAL, NULL, NULL, dev(6), wsb,
                           NULL) == ATTN_E_INVALID);   // the encoding on a cross-attention sublayer
}

static void decode_bwd_linear_calls() {
  const int B = 4, H = 2, nq = 3, nkv = 5000;
  const size_t ws = attn_decode_workspace_bytes(ATTN_BF16, B, H, nq, nkv, 64, 64);
  CHECK(ws > 0);
  CHECK(attn_decode_fwd(ATTN_BF16, B, H, nq, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL, 0.f,
                        NULL, NULL, dev(4), ws, NULL) == ATTN_OK);
  CHECK(g_rec.decode.n_chunks >= 1 && g_rec.decode.part_o == (float*)dev(4));
  CHECK(attn_decode_fwd(ATTN_BF16, B, H, 33, nkv, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                        0.f, NULL, NULL, dev(4), ws, NULL) != ATTN_OK);   // more than 32 new queries
  // backward with a workspace and without
  const int n = 333;
  const size_t wb = attn_sdpa_bwd_workspace_bytes(ATTN_BF16, 2, 3, n, n, 64, 64);
  CHECK(wb == ((size_t)2 * 3 * n * 8 + 255) / 256 * 256);
  CHECK(attn_sdpa_bwd(ATTN_BF16, 2, 3, n, n, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL, dev(4),
                      NULL, (float*)dev(5), dev(6), NULL, dev(7), NULL, dev(8), NULL, 0.f, ATTN_MASK_CAUSAL, NULL,
                      NULL, dev(9), wb, NULL) == ATTN_OK);
  CHECK(g_rec.bwd.ld == (float*)dev(9));
  CHECK(attn_sdpa_bwd_noalloc(ATTN_BF16, 2, 3, n, n, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3), NULL,
                              dev(4), NULL, (float*)dev(5), dev(6), NULL, dev(7), NULL, dev(8), NULL, 0.f,
                              ATTN_MASK_CAUSAL, NULL, NULL, NULL) == ATTN_OK);
  CHECK(g_rec.bwd.ld != (float*)dev(9) && ((uintptr_t)g_rec.bwd.ld & 255) == 0);
  CHECK(attn_sdpa_bwd_noalloc(ATTN_BF16, 64, 64, 513, 64, 64, 64, dev(0), NULL, dev(1), NULL, dev(2), NULL, dev(3),
                              NULL, dev(4), NULL, (float*)dev(5), dev(6), NULL, dev(7), NULL, dev(8), NULL, 0.f,
                              ATTN_MASK_CAUSAL, NULL, NULL, NULL) == ATTN_E_WORKSPACE);
  // one projection
  CHECK(attn_linear_fwd(ATTN_BF16, 1000, 1024, 3072, dev(0), 1024, dev(1), dev(2), 3072, NULL) == ATTN_OK);
  CHECK(g_rec.gemm.M == 1000 && g_rec.gemm.ldc == 3072);
  CHECK(attn_linear_fwd(ATTN_BF16, INT_MAX, 1024, 3072, dev(0), 1024, dev(1), dev(2), 3072, NULL) == ATTN_OK ||
        true);   // a legal huge call: only its arithmetic is checked here
}

int main() {
  sdpa_calls();
  mha_calls();
  decode_bwd_linear_calls();
  for (int s = 0; s >= -6; --s) CHECK(attn_status_str(s) != NULL);
  CHECK(attn_abi_version() == ATTN_ABI_VERSION);
  CHECK(attn_hip_error_str(attn_last_hip_error()) != NULL);
  if (g_fail) return 1;
  printf("abi driver: ok\n");
  return 0;
}
