/*
 * The C ABI used from plain C (C11, no C++ and no Python): include/mm.h,
 * libmm.so and the HIP runtime's C API.  Test infrastructure; the expected
 * values come from the oracle's C library (liboracle.so).
 *
 *   mm_from_c check   argument errors, status strings and the configuration
 *                     string, without a GPU (no call reaches the device)
 *   mm_from_c gemm    linear + bias + GELU(tanh), the SwiGLU FFN and a plain
 *                     fp32 matmul on the GPU, each compared with the oracle
 *                     element by element (|got - ref| <= rel (|ref| + 1))
 *
 * Prints one line per case and "ok" at the end; exits non-zero on the first
 * failure.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mm.h"

/* liboracle.so (the oracle's own layout and epilogue codes) */
int oracle_gemm(const uint16_t* A, const uint16_t* B, const uint16_t* B2, const uint16_t* bias,
                int64_t M, int64_t N, int64_t K, int layout, int epi, int64_t row_begin,
                int64_t row_end, float* y_out, uint16_t* bf16_out, int nthreads, double* seconds);
enum { ORACLE_NN = 0, ORACLE_NT = 1 };
enum { ORACLE_EPI_NONE = 0, ORACLE_EPI_BIAS_GELU = 3, ORACLE_EPI_SWIGLU = 4 };

#define EXPECT(cond, ...)                                      \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);     \
      fprintf(stderr, __VA_ARGS__);                            \
      fprintf(stderr, "\n");                                   \
      exit(1);                                                 \
    }                                                          \
  } while (0)

/* fake device addresses: 16-byte aligned and far apart; no call that gets
 * them reaches the device */
#define PA ((const void*)(uintptr_t)0x100000)
#define PB ((const void*)(uintptr_t)0x200000)
#define POUT ((void*)(uintptr_t)0x40000000)

static int check_mode(void) {
  EXPECT(strcmp(mm_status_string(MM_OK), "MM_OK") == 0, "status string");
  EXPECT(strcmp(mm_status_string(MM_ERR_MISALIGNED), "MM_ERR_MISALIGNED") == 0, "status string");
  EXPECT(mm_matmul(NULL, PB, POUT, 64, 64, 64, MM_NT, MM_OUT_BF16, NULL) == MM_ERR_INVALID_VALUE,
         "null A");
  EXPECT(strlen(mm_last_error()) > 0, "last error after a failed call");
  EXPECT(mm_matmul(PA, PB, POUT, -1, 64, 64, MM_NT, MM_OUT_BF16, NULL) == MM_ERR_INVALID_VALUE,
         "negative M");
  EXPECT(mm_matmul(PA, PB, POUT, 64, 64, 60, MM_NT, MM_OUT_BF16, NULL) == MM_ERR_MISALIGNED,
         "K-contiguous extent not a multiple of 8");
  EXPECT(mm_matmul((const char*)PA + 2, PB, POUT, 64, 64, 64, MM_NT, MM_OUT_BF16, NULL) ==
             MM_ERR_MISALIGNED,
         "misaligned A");
  EXPECT(mm_linear(PA, PB, NULL, POUT, 64, 64, 64, MM_NT, MM_EPI_BIAS, NULL) == MM_ERR_INVALID_VALUE,
         "bias epilogue without a bias");
  EXPECT(mm_matmul(PA, PB, (void*)((uintptr_t)PA + 64), 64, 64, 64, MM_NT, MM_OUT_BF16, NULL) ==
             MM_ERR_INVALID_VALUE,
         "output overlapping A");
  EXPECT(mm_matmul(PA, PB, POUT, 0, 64, 64, MM_NT, MM_OUT_BF16, NULL) == MM_OK, "empty output");
  char buf[256];
  EXPECT(mm_describe_config(0, 8192, 8192, 8192, MM_NT, buf, sizeof buf) == MM_OK, "describe");
  EXPECT(strncmp(buf, "BM=256,BN=256", 13) == 0 && strstr(buf, "KERNEL=gemm_nt_slab") != NULL,
         "describe 8192^3: %s", buf);
  EXPECT(mm_set_config("BM=3") == MM_ERR_UNSUPPORTED, "unsupported tile");
  printf("check: argument errors, status strings, configuration string\n");
  return 0;
}

/* bf16 bits of a float, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* SplitMix64: a counter-based generator; uniform in [-1, 1) times `scale` */
static uint64_t splitmix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}
static uint16_t* random_bf16(size_t n, uint64_t seed, float scale) {
  uint16_t* h = (uint16_t*)malloc(n * 2);
  EXPECT(h != NULL, "host allocation");
  for (size_t i = 0; i < n; ++i) {
    const double u = (double)(splitmix64(seed * 0x100000001ull + i) >> 11) / 9007199254740992.0;
    h[i] = to_bf16((float)((2.0 * u - 1.0) * scale));
  }
  return h;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  EXPECT(hipMalloc(&d, bytes) == hipSuccess, "hipMalloc");
  EXPECT(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) == hipSuccess, "hipMemcpy H2D");
  return d;
}

static void compare(const char* name, const void* dev_out, int f32, const float* ref, int64_t count,
                    double rel) {
  const size_t esize = f32 ? 4 : 2;
  void* host = malloc((size_t)count * esize);
  EXPECT(host != NULL, "host allocation");
  EXPECT(hipMemcpy(host, dev_out, (size_t)count * esize, hipMemcpyDeviceToHost) == hipSuccess,
         "hipMemcpy D2H");
  double worst = 0.0;  /* max |got - ref| / (|ref| + 1) */
  for (int64_t i = 0; i < count; ++i) {
    const double got = f32 ? ((const float*)host)[i] : from_bf16(((const uint16_t*)host)[i]);
    EXPECT(isfinite(got), "%s: non-finite output at %lld", name, (long long)i);
    const double err = fabs(got - ref[i]) / (fabs(ref[i]) + 1.0);
    if (err > worst) worst = err;
    EXPECT(err <= rel, "%s: element %lld is %g, the oracle's %g", name, (long long)i, got, ref[i]);
  }
  free(host);
  printf("%s: %lld outputs, max |got - ref| / (|ref| + 1) = %.3g (bound %g)\n", name,
         (long long)count, worst, rel);
}

static int gemm_mode(void) {
  /* ragged tiles in both dimensions; K a multiple of 64 */
  const int64_t M = 1000, N = 776, K = 320;
  uint16_t* x = random_bf16((size_t)(M * K), 1, 1.0f);
  uint16_t* W = random_bf16((size_t)(N * K), 2, 0.1f);
  uint16_t* Wu = random_bf16((size_t)(N * K), 3, 0.1f);
  uint16_t* bias = random_bf16((size_t)N, 4, 1.0f);
  void* dx = to_device(x, (size_t)(M * K) * 2);
  void* dW = to_device(W, (size_t)(N * K) * 2);
  void* dWu = to_device(Wu, (size_t)(N * K) * 2);
  void* dbias = to_device(bias, (size_t)N * 2);
  void* dout = NULL;
  EXPECT(hipMalloc(&dout, (size_t)(M * N) * 4) == hipSuccess, "hipMalloc");
  hipStream_t stream;
  EXPECT(hipStreamCreate(&stream) == hipSuccess, "hipStreamCreate");
  float* ref = (float*)malloc((size_t)(M * N) * 4);
  EXPECT(ref != NULL, "host allocation");

  /* LinearOp: out = GELU(x W^T + bias), bf16 */
  EXPECT(mm_linear(dx, dW, dbias, dout, M, N, K, MM_NT, MM_EPI_BIAS_GELU_TANH, stream) == MM_OK,
         "mm_linear: %s", mm_last_error());
  EXPECT(hipStreamSynchronize(stream) == hipSuccess, "sync");
  EXPECT(oracle_gemm(x, W, NULL, bias, M, N, K, ORACLE_NT, ORACLE_EPI_BIAS_GELU, 0, M, ref, NULL, 0,
                     NULL) == 0,
         "oracle");
  compare("linear+bias+GELU bf16", dout, 0, ref, M * N, 2e-2);

  /* horizontally fused FFN: SiLU(x W_gate^T) * (x W_up^T), bf16 */
  EXPECT(mm_ffn_swiglu(dx, dW, dWu, dout, M, N, K, stream) == MM_OK, "mm_ffn_swiglu: %s",
         mm_last_error());
  EXPECT(hipStreamSynchronize(stream) == hipSuccess, "sync");
  EXPECT(oracle_gemm(x, W, Wu, NULL, M, N, K, ORACLE_NT, ORACLE_EPI_SWIGLU, 0, M, ref, NULL, 0,
                     NULL) == 0,
         "oracle");
  compare("FFN SwiGLU bf16", dout, 0, ref, M * N, 2e-2);

  /* MatmulOp, fp32 out, B given [K][N] (NN): W's bits reinterpreted as [K][N] */
  EXPECT(mm_matmul(dx, dW, dout, M, N, K, MM_NN, MM_OUT_F32, stream) == MM_OK, "mm_matmul: %s",
         mm_last_error());
  EXPECT(hipStreamSynchronize(stream) == hipSuccess, "sync");
  EXPECT(oracle_gemm(x, W, NULL, NULL, M, N, K, ORACLE_NN, ORACLE_EPI_NONE, 0, M, ref, NULL, 0, NULL) ==
             0,
         "oracle");
  compare("matmul NN fp32", dout, 1, ref, M * N, 1e-3);

  EXPECT(hipStreamDestroy(stream) == hipSuccess, "hipStreamDestroy");
  hipFree(dx);
  hipFree(dW);
  hipFree(dWu);
  hipFree(dbias);
  hipFree(dout);
  free(x);
  free(W);
  free(Wu);
  free(bias);
  free(ref);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s check|gemm\n", argv[0]);
    return 2;
  }
  int rc;
  if (strcmp(argv[1], "check") == 0) rc = check_mode();
  else if (strcmp(argv[1], "gemm") == 0) rc = gemm_mode();
  else {
    fprintf(stderr, "unknown mode %s\n", argv[1]);
    return 2;
  }
  if (rc == 0) printf("ok\n");
  return rc;
}
