// A C++ caller of the C ABI (include/moe_ragged_bf16.h) with no Python: it
// sizes and allocates workspaces, prepares a fwd launch and launches it twice,
// calls dgrad, wgrad (bf16 and fp32 out) and both accumulating wgrads one-shot,
// checks every result against a closed form and exercises the status codes,
// for an aligned shape and for one with a partial tile and a partial last stage.
//
// Closed forms (API page, operations table), all exact: the inputs are small
// integers and one-hot rows, so every product sum is an integer far below 2^8
// and exact in bf16; only the bf16 accumulate's sum (main_grad in quarters
// plus dW) may round, once, to nearest even.
//  * fwd: with W[e] row n the unit vector of column (n + e) % K,
//    Y[r][n] = X[r][(n + e) % K] bit for bit.
//  * dgrad, same W: dX[r][k] = sum of G[r][n] over n < N with (n + e) % K == k.
//  * wgrad, with a one-hot Xh (row r is the unit vector of column (3 r) % K):
//    dW[e][n][k] = sum of G[r][n] over the rows r of group e with (3 r) % K == k;
//    an empty group gives +0.0; the fused accumulates give main_grad + dW
//    (exact here) and turn a -0.0 of an empty expert into +0.0.
// Exits 0 on success.
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

// fp32 -> bf16, round to nearest, ties to even (finite values)
static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

// dgrad, wgrad and both accumulates, one-shot, against their closed forms.
static int run_backward(const int N, const int K, const int E, const int* sizes, const int64_t M,
                        const int32_t* offs, const void* w, const std::vector<int32_t>& offs_h,
                        hipStream_t stream) {
  std::vector<uint16_t> g_h(M * N), xh_h(M * K, 0), dx_h(M * K);
  for (int64_t r = 0; r < M; ++r)
    for (int n = 0; n < N; ++n) g_h[r * N + n] = bf16_bits((float)((r * 5 + n * 3) % 61 - 30));
  for (int64_t r = 0; r < M; ++r) xh_h[r * K + (3 * r) % K] = bf16_bits(1.0f);
  const size_t nk = (size_t)E * N * K;
  // expected dW in fp32 (integers)
  std::vector<float> dw_ref(nk, 0.0f);
  for (int e = 0, s = 0; e < E; s += sizes[e], ++e)
    for (int r = s; r < s + sizes[e]; ++r)
      for (int n = 0; n < N; ++n) {
        const uint32_t gb = (uint32_t)g_h[(size_t)r * N + n] << 16;
        float gv;
        memcpy(&gv, &gb, 4);
        dw_ref[((size_t)e * N + n) * K + (3 * r) % K] += gv;
      }
  std::vector<float> mg0(nk);
  for (size_t i = 0; i < nk; ++i) mg0[i] = 0.25f * (float)((int)(i % 13) - 6);
  mg0[(size_t)1 * N * K + 3] = -0.0f;  // expert 1 is empty: -0.0 + (+0.0) = +0.0

  void *g, *xh, *dx, *dw32, *dw16, *ws_d, *ws_w;
  const size_t wsd_bytes = grouped_det_gemm_dgrad_workspace_bytes(M, N, K, E);
  const size_t wsw_bytes = grouped_det_gemm_wgrad_workspace_bytes(M, N, K, E);
  EXPECT(wsd_bytes != 0 && wsw_bytes != 0);
  CHECK_HIP(hipMalloc(&g, g_h.size() * 2));
  CHECK_HIP(hipMalloc(&xh, xh_h.size() * 2));
  CHECK_HIP(hipMalloc(&dx, dx_h.size() * 2));
  CHECK_HIP(hipMalloc(&dw32, nk * 4));
  CHECK_HIP(hipMalloc(&dw16, nk * 2));
  CHECK_HIP(hipMalloc(&ws_d, wsd_bytes));
  CHECK_HIP(hipMalloc(&ws_w, wsw_bytes));
  CHECK_HIP(hipMemcpy(g, g_h.data(), g_h.size() * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(xh, xh_h.data(), xh_h.size() * 2, hipMemcpyHostToDevice));

  // dgrad
  CHECK_HIP(hipMemset(dx, 0xFF, dx_h.size() * 2));
  EXPECT(grouped_det_gemm_dgrad(g, w, offs, dx, M, N, K, E, ws_d, wsd_bytes - 1, stream) == MDG_EWORKSPACE);
  EXPECT(grouped_det_gemm_dgrad(g, w, offs, g, M, N, K, E, ws_d, wsd_bytes, stream) == MDG_EOVERLAP);
  EXPECT(grouped_det_gemm_dgrad(g, w, offs, dx, M, N, K, E, ws_d, wsd_bytes, stream) == MDG_OK);
  CHECK_HIP(hipMemcpyAsync(dx_h.data(), dx, dx_h.size() * 2, hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  int64_t bad = 0;
  const int last = offs_h[E - 1];
  for (int e = 0, s = 0; e < E; s += sizes[e], ++e)
    for (int r = s; r < s + sizes[e]; ++r)
      for (int k = 0; k < K; ++k) {
        float want = 0.0f;
        for (int n = 0; n < N; ++n)
          if ((n + e) % K == k) {
            const uint32_t gb = (uint32_t)g_h[(size_t)r * N + n] << 16;
            float gv;
            memcpy(&gv, &gb, 4);
            want += gv;
          }
        bad += dx_h[(size_t)r * K + k] != bf16_bits(want);
      }
  for (int64_t r = last; r < M; ++r)
    for (int k = 0; k < K; ++k) bad += dx_h[(size_t)r * K + k] != 0xFFFF;
  if (bad) {
    fprintf(stderr, "dgrad: %lld mismatches\n", (long long)bad);
    return 1;
  }

  // wgrad overwrite, fp32 and bf16
  std::vector<uint32_t> got32(nk);
  std::vector<uint16_t> got16(nk);
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw32, MDG_FP32, 0, M, N, K, E, ws_w, wsw_bytes - 1, stream) ==
         MDG_EWORKSPACE);
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw32, 7, 0, M, N, K, E, ws_w, wsw_bytes, stream) == MDG_EINVAL);
  CHECK_HIP(hipMemset(dw32, 0xFF, nk * 4));
  CHECK_HIP(hipMemset(dw16, 0xFF, nk * 2));
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw32, MDG_FP32, 0, M, N, K, E, ws_w, wsw_bytes, stream) == MDG_OK);
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw16, MDG_BF16, 0, M, N, K, E, ws_w, wsw_bytes, stream) == MDG_OK);
  CHECK_HIP(hipMemcpyAsync(got32.data(), dw32, nk * 4, hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipMemcpyAsync(got16.data(), dw16, nk * 2, hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  for (size_t i = 0; i < nk; ++i) {
    bad += got32[i] != f32_bits(dw_ref[i]);      // +0.0 where nothing is summed, empty experts included
    bad += got16[i] != bf16_bits(dw_ref[i]);
  }
  if (bad) {
    fprintf(stderr, "wgrad: %lld mismatches\n", (long long)bad);
    return 1;
  }

  // fused accumulates: fp32 main_grad and bf16 main_grad
  std::vector<uint16_t> mg0_16(nk);
  for (size_t i = 0; i < nk; ++i) mg0_16[i] = bf16_bits(mg0[i]);
  CHECK_HIP(hipMemcpy(dw32, mg0.data(), nk * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw16, mg0_16.data(), nk * 2, hipMemcpyHostToDevice));
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw32, MDG_FP32, 1, M, N, K, E, ws_w, wsw_bytes, stream) == MDG_OK);
  EXPECT(grouped_det_gemm_wgrad(g, xh, offs, dw16, MDG_BF16, 1, M, N, K, E, ws_w, wsw_bytes, stream) == MDG_OK);
  CHECK_HIP(hipMemcpyAsync(got32.data(), dw32, nk * 4, hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipMemcpyAsync(got16.data(), dw16, nk * 2, hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  for (size_t i = 0; i < nk; ++i) {
    const float want = mg0[i] + dw_ref[i];   // exact: quarters and small integers
    bad += got32[i] != f32_bits(want);
    bad += got16[i] != bf16_rne(want);       // the bf16 sum rounds once
  }
  if (bad) {
    fprintf(stderr, "wgrad accumulate: %lld mismatches\n", (long long)bad);
    return 1;
  }
  EXPECT(got32[(size_t)1 * N * K + 3] == 0u && got16[(size_t)1 * N * K + 3] == 0u);  // +0.0
  hipFree(g);
  hipFree(xh);
  hipFree(dx);
  hipFree(dw32);
  hipFree(dw16);
  hipFree(ws_d);
  hipFree(ws_w);
  return 0;
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
    fprintf(stderr, "prepare: %s\n", grouped_det_gemm_status_string(st));
    return 1;
  }
  mdg_launch_info info;
  EXPECT(grouped_det_gemm_launch_info(l, &info) == MDG_OK && info.op == 0 && info.kernels >= 1);
  for (int rep = 0; rep < 2; ++rep) {
    CHECK_HIP(hipMemsetAsync(y, 0xFF, y_h.size() * 2, stream));  // every group row must be rewritten
    st = grouped_det_gemm_launch(l, stream);
    if (st != MDG_OK) {
      fprintf(stderr, "launch: %s\n", grouped_det_gemm_status_string(st));
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
  if (run_backward(N, K, E, sizes, M, offs, w, std::vector<int32_t>(offs_h, offs_h + E), stream) != 0) return 1;
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
  EXPECT(grouped_det_gemm_abi_version() == MDG_ABI_VERSION);
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
  printf("c abi smoke ok: prepared fwd launched twice, one-shot dgrad, wgrad bf16/fp32 and both fused accumulates "
         "at n,k = 256,128 and 136,200 (fwd: %d and %d kernels), closed forms exact\n",
         kernels[0], kernels[1]);
  return 0;
}
