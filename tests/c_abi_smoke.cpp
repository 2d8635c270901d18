// A C++ caller of the C ABI (include/moe_ragged_bf16.h) with no Python: it
// sizes and allocates a workspace, prepares a fwd launch, launches it twice,
// checks the result against a closed form and exercises the status codes, for
// an aligned shape and for one with a partial tile and a partial last stage.
//
// Closed form (API page, operations table, "fwd"): with W[e] row n equal to the
// unit vector of column (n + e) % K, Y[r][n] = X[r][(n + e(r)) % K] exactly (one
// product of a bf16 value by 1.0, summed with zeros), so every Y element must
// equal one X element bit for bit.  Exits 0 on success.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "moe_ragged_bf16.h"

#define CHECK_HIP(x)                                                      \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      return 2;                                                           \
    }                                                                     \
  } while (0)

#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "c_abi_smoke.cpp:%d: check failed: %s\n", __LINE__, #cond); \
      return 1;                                                           \
    }                                                                     \
  } while (0)

static uint16_t bf16_bits(float f) {  // exact for the small integers used here
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// One shape: prepare, launch twice, check the closed form.  Returns 0 on success.
static int run_case(const int N, const int K, int* kernels) {
  const int E = 3;
  const int sizes[E] = {5, 0, 300};
  const int64_t M = 305 + 2;  // two padding rows
  int32_t offs_h[E];
  for (int e = 0, s = 0; e < E; ++e) offs_h[e] = (s += sizes[e]);

  std::vector<uint16_t> x_h(M * K), w_h((size_t)E * N * K, 0), y_h(M * N);
  for (int64_t i = 0; i < M * K; ++i) x_h[i] = bf16_bits((float)((i * 7) % 61 - 30));
  for (int e = 0; e < E; ++e)
    for (int n = 0; n < N; ++n) w_h[((size_t)e * N + n) * K + (n + e) % K] = bf16_bits(1.0f);

  const size_t ws_bytes = grouped_det_gemm_fwd_workspace_bytes(M, N, K, E);
  EXPECT(ws_bytes != 0 && grouped_det_gemm_fwd_workspace_bytes(M, N + 1, K, E) == 0);

  void *x, *w, *y, *ws;
  int32_t* offs;
  CHECK_HIP(hipMalloc(&x, x_h.size() * 2));
  CHECK_HIP(hipMalloc(&w, w_h.size() * 2));
  CHECK_HIP(hipMalloc(&y, y_h.size() * 2));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc((void**)&offs, sizeof(offs_h)));
  CHECK_HIP(hipMemcpy(x, x_h.data(), x_h.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w, w_h.data(), w_h.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(offs, offs_h, sizeof(offs_h), hipMemcpyHostToDevice));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  // refusals come back as status codes and leave *launch NULL
  mdg_launch* l = (mdg_launch*)0x1;
  EXPECT(grouped_det_gemm_prepare_fwd(x, w, offs, y, M, N, K, E, ws, ws_bytes - 1, &l) == MDG_EWORKSPACE && !l);
  EXPECT(grouped_det_gemm_prepare_fwd(x, w, offs, x, M, N, K, E, ws, ws_bytes, &l) == MDG_EOVERLAP && !l);
  EXPECT(grouped_det_gemm_prepare_fwd(x, w, offs, y, M, 204, K, E, ws, ws_bytes, &l) == MDG_EUNSUPPORTED);

  int st = grouped_det_gemm_prepare_fwd(x, w, offs, y, M, N, K, E, ws, ws_bytes, &l);
  if (st != MDG_OK) {
    fprintf(stderr, "prepare: %s\n", mdg_status_string(st));
    return 1;
  }
  mdg_launch_info info;
  EXPECT(grouped_det_gemm_launch_info(l, &info) == MDG_OK && info.op == 0 && info.kernels >= 1);
  for (int rep = 0; rep < 2; ++rep) {
    CHECK_HIP(hipMemsetAsync(y, 0xFF, y_h.size() * 2, stream));  // every group row must be rewritten
    st = grouped_det_gemm_launch(l, stream);
    if (st != MDG_OK) {
      fprintf(stderr, "launch: %s\n", mdg_status_string(st));
      return 1;
    }
    CHECK_HIP(hipMemcpyAsync(y_h.data(), y, y_h.size() * 2, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    int64_t bad = 0;
    for (int e = 0, s = 0; e < E; s += sizes[e], ++e)
      for (int r = s; r < s + sizes[e]; ++r)
        for (int n = 0; n < N; ++n) bad += y_h[(size_t)r * N + n] != x_h[(size_t)r * K + (n + e) % K];
    for (int64_t r = 305; r < M; ++r)  // rows past the last group are left untouched
      for (int n = 0; n < N; ++n) bad += y_h[(size_t)r * N + n] != 0xFFFF;
    if (bad) {
      fprintf(stderr, "rep %d: %lld mismatches\n", rep, (long long)bad);
      return 1;
    }
  }
  grouped_det_gemm_launch_free(l);
  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(x);
  hipFree(w);
  hipFree(y);
  hipFree(ws);
  hipFree(offs);
  *kernels = info.kernels;
  return 0;
}

int main() {
  EXPECT(mdg_abi_version() == MDG_ABI_VERSION);
  // n = 256, k = 128: whole tiles and stages; n = 136, k = 200: a partial
  // 256-wide tile in n and a reduction that ends in a partial 32-deep stage
  const int shapes[2][2] = {{256, 128}, {136, 200}};
  int kernels[2];
  for (int c = 0; c < 2; ++c) {
    if (run_case(shapes[c][0], shapes[c][1], &kernels[c]) != 0) {
      fprintf(stderr, "case n=%d k=%d failed\n", shapes[c][0], shapes[c][1]);
      return 1;
    }
  }
  printf("c abi smoke ok: prepared fwd launched twice at n,k = 256,128 and 136,200 (%d and %d kernels), closed form exact\n",
         kernels[0], kernels[1]);
  return 0;
}
