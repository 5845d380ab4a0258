// A program that uses the attention library through its C ABI alone (no
// Python, no torch): it reads bf16 Q, K, V from a file, runs attn_sdpa_fwd on
// the GPU, and writes O and the log-sum-exp back.
//
//   sdpa_driver <in.bin> <out.bin>
//
// in.bin : int32 batch, heads, n_q, n_kv, causal, has_lengths; float32 scale;
//          if has_lengths: int32 lq[batch], int32 lkv[batch];
//          uint16 q[batch*heads*n_q*64], k[batch*heads*n_kv*64],
//          v[batch*heads*n_kv*64] (bf16 bit patterns, contiguous [b, h, n, d])
// out.bin: uint16 o[batch*heads*n_q*64]; float32 lse[batch*heads*n_q]
//
// Exit status 0 on success; otherwise a message on stderr names the failing
// call (and, for ATTN_E_HIP, the HIP error behind it).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn_sdpa.h"

namespace {

template <typename T>
bool read_n(FILE* f, T* dst, size_t n) {
  return fread(dst, sizeof(T), n, f) == n;
}

int fail(const char* what) {
  fprintf(stderr, "sdpa_driver: %s\n", what);
  return 1;
}

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "sdpa_driver: %s: %s\n", what, hipGetErrorString(e));
  return false;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage: sdpa_driver <in.bin> <out.bin>");
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open the input file");
  int32_t hdr[6];
  float scale = 0.f;
  if (!read_n(in, hdr, 6) || !read_n(in, &scale, 1)) return fail("short input header");
  const int batch = hdr[0], heads = hdr[1], n_q = hdr[2], n_kv = hdr[3], causal = hdr[4], has_len = hdr[5];
  if (batch < 1 || heads < 1 || n_q < 0 || n_kv < 0) return fail("bad sizes in the header");
  std::vector<int32_t> lq, lkv;
  if (has_len) {
    lq.resize(batch);
    lkv.resize(batch);
    if (!read_n(in, lq.data(), batch) || !read_n(in, lkv.data(), batch)) return fail("short lengths");
  }
  const size_t nq = (size_t)batch * heads * n_q * 64, nkv = (size_t)batch * heads * n_kv * 64;
  std::vector<uint16_t> q(nq), k(nkv), v(nkv);
  if (!read_n(in, q.data(), nq) || !read_n(in, k.data(), nkv) || !read_n(in, v.data(), nkv))
    return fail("short tensor data");
  fclose(in);

  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dout = nullptr, *dlse = nullptr;
  int32_t *dlq = nullptr, *dlkv = nullptr;
  const size_t rows = (size_t)batch * heads * n_q;
  if (!hip_ok(hipMalloc(&dq, nq * 2 + 16), "hipMalloc q") || !hip_ok(hipMalloc(&dk, nkv * 2 + 16), "hipMalloc k") ||
      !hip_ok(hipMalloc(&dv, nkv * 2 + 16), "hipMalloc v") || !hip_ok(hipMalloc(&dout, nq * 2 + 16), "hipMalloc o") ||
      !hip_ok(hipMalloc(&dlse, rows * 4 + 16), "hipMalloc lse"))
    return 1;
  if (!hip_ok(hipMemcpy(dq, q.data(), nq * 2, hipMemcpyHostToDevice), "copy q") ||
      !hip_ok(hipMemcpy(dk, k.data(), nkv * 2, hipMemcpyHostToDevice), "copy k") ||
      !hip_ok(hipMemcpy(dv, v.data(), nkv * 2, hipMemcpyHostToDevice), "copy v"))
    return 1;
  if (has_len) {
    if (!hip_ok(hipMalloc(&dlq, batch * 4), "hipMalloc lq") || !hip_ok(hipMalloc(&dlkv, batch * 4), "hipMalloc lkv") ||
        !hip_ok(hipMemcpy(dlq, lq.data(), batch * 4, hipMemcpyHostToDevice), "copy lq") ||
        !hip_ok(hipMemcpy(dlkv, lkv.data(), batch * 4, hipMemcpyHostToDevice), "copy lkv"))
      return 1;
  }
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;

  const int rc = attn_sdpa_fwd(ATTN_BF16, batch, heads, n_q, n_kv, 64, 64, dq, nullptr, dk, nullptr, dv, nullptr,
                               dout, nullptr, scale, causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE, dlq, dlkv,
                               static_cast<float*>(dlse), stream);
  if (rc != ATTN_OK) {
    fprintf(stderr, "sdpa_driver: attn_sdpa_fwd: %s", attn_status_str(rc));
    if (rc == ATTN_E_HIP) fprintf(stderr, " (%s)", attn_hip_error_str(attn_last_hip_error()));
    fprintf(stderr, "\n");
    return 1;
  }
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

  std::vector<uint16_t> o(nq);
  std::vector<float> lse(rows);
  if (!hip_ok(hipMemcpy(o.data(), dout, nq * 2, hipMemcpyDeviceToHost), "copy o back") ||
      !hip_ok(hipMemcpy(lse.data(), dlse, rows * 4, hipMemcpyDeviceToHost), "copy lse back"))
    return 1;
  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("cannot open the output file");
  if (fwrite(o.data(), 2, nq, out) != nq || fwrite(lse.data(), 4, rows, out) != rows) return fail("short write");
  fclose(out);
  hipStreamDestroy(stream);
  for (void* p : {dq, dk, dv, dout, dlse, static_cast<void*>(dlq), static_cast<void*>(dlkv)})
    if (p) hipFree(p);
  return 0;
}
