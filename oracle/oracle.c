/*
 * oracle.c -- plain, slow CPU reference of the bf16 GEMM hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this file; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or helper with the GPU kernels.
 *
 * What it computes (the operation these pages are about):
 *   - MatmulOp form   out = A . B                (issue "Automate performant
 *     Hopper matmul", section "Persistent matmul": MatmulOp / LinearOp nodes)
 *   - LinearOp form   out = epi(x . W^T + bias)  (same passage; the bias and
 *     activation are the forward epilogue fusion of PR "Implement persistent
 *     matmul scheduling", description: MLPBenchmarkTest.FwdEpilogueFusion)
 *   - Llama-FFN horizontal fusion out = SiLU(x . Wg^T) * (x . Wu^T)
 *     (PR "Translate MmaOp patterns properly on Hopper", commit list:
 *     "Fix llama ffn horizontal fusion", "Fixes the horizontal fusion tests")
 *   The contraction itself is the broadcast-multiply-sum the PR "Implement
 *   persistent matmul scheduling" describes for its _BroadcastInputs tests
 *   (fusedMultiplySum): out[i][j] = sum over k of A[i][k] * B[k][j].
 *
 * Precision (the reading adopted where the pages are silent): inputs are the
 * bf16 bit patterns the GPU receives, widened exactly to fp32; every output
 * element has ONE fp32 accumulator that starts at +0 and adds the products in
 * ascending k.  A bf16 x bf16 product has at most 16 significant bits, so it
 * is exact in fp32 and fused or separate multiply-add give the same bits.
 * The epilogue adds the bias in fp32, evaluates the activation in double from
 * that fp32 value, rounds once to fp32 (y) and, for bf16 outputs, rounds y
 * to bf16 with round-to-nearest-even.
 *
 * Two evaluation orders are provided and must agree bit for bit:
 *   oracle_gemm         row range, i-k-j loop (one accumulator per output,
 *                       k ascending) over operands widened to fp32;
 *   oracle_gemm_points  the literal per-element k loop, read straight from
 *                       the bf16 storage, for sampled (i, j) at any size.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage layouts.  Letters are op(A), op(B) in row-major terms:
 *   NN: A stored [M][K],  B stored [K][N]
 *   NT: A stored [M][K],  B stored [N][K]   (B = Bs^T; the LinearOp weight)
 *   TN: A stored [K][M],  B stored [K][N]   (A = As^T)
 *   TT: A stored [K][M],  B stored [N][K]                                  */
enum { OR_NN = 0, OR_NT = 1, OR_TN = 2, OR_TT = 3 };

/* Epilogues: none, +bias, GELU(tanh), GELU(tanh)(.+bias), and the two
 * gated forms of the horizontal fusion (SiLU(g)*u, and g*u). */
enum {
  OR_EPI_NONE = 0,
  OR_EPI_BIAS = 1,
  OR_EPI_GELU = 2,
  OR_EPI_BIAS_GELU = 3,
  OR_EPI_SWIGLU = 4,
  OR_EPI_GLU_IDENTITY = 5
};

static float bf16_bits_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round-to-nearest-even fp32 -> bf16 on the bit pattern.  NaN stays NaN
 * (quiet bit set, sign kept); overflow past the largest bf16 gives inf. */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* tanh-approximated GELU, evaluated in double from an fp32 argument. */
static double gelu_tanh_d(double t) {
  const double c = sqrt(2.0 / 3.14159265358979323846);
  return 0.5 * t * (1.0 + tanh(c * (t + 0.044715 * t * t * t)));
}

static double silu_d(double g) { return g / (1.0 + exp(-g)); }

static int layout_ok(int layout) { return layout >= OR_NN && layout <= OR_TT; }
static int a_transposed(int layout) { return layout == OR_TN || layout == OR_TT; }
static int b_transposed(int layout) { return layout == OR_NT || layout == OR_TT; }

/* Element (i, k) of op(A) and (k, j) of op(B), read from storage. */
static uint16_t a_elem(const uint16_t* A, int64_t M, int64_t K, int layout, int64_t i, int64_t k) {
  return a_transposed(layout) ? A[k * M + i] : A[i * K + k];
}
static uint16_t b_elem(const uint16_t* B, int64_t N, int64_t K, int layout, int64_t k, int64_t j) {
  return b_transposed(layout) ? B[j * K + k] : B[k * N + j];
}

/* The epilogue on one fp32 accumulator (and its gated partner u). */
static float epilogue(int epi, float acc, float u, const uint16_t* bias, int64_t j) {
  float t = acc;
  switch (epi) {
    case OR_EPI_NONE:
      return acc;
    case OR_EPI_BIAS:
      return acc + bf16_bits_to_f32(bias[j]);
    case OR_EPI_GELU:
      return (float)gelu_tanh_d((double)t);
    case OR_EPI_BIAS_GELU:
      t = acc + bf16_bits_to_f32(bias[j]);
      return (float)gelu_tanh_d((double)t);
    case OR_EPI_SWIGLU:
      return (float)(silu_d((double)acc) * (double)u);
    case OR_EPI_GLU_IDENTITY:
      return (float)((double)acc * (double)u);
  }
  return acc;
}

static int check_args(const uint16_t* A, const uint16_t* B, const uint16_t* B2,
                      const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                      int layout, int epi) {
  if (!A || !B || M < 0 || N < 0 || K < 0 || !layout_ok(layout)) return 1;
  if (epi < OR_EPI_NONE || epi > OR_EPI_GLU_IDENTITY) return 1;
  if ((epi == OR_EPI_BIAS || epi == OR_EPI_BIAS_GELU) && !bias) return 1;
  if ((epi == OR_EPI_SWIGLU || epi == OR_EPI_GLU_IDENTITY) && !B2) return 1;
  return 0;
}

static double now_s(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* Widen op(B) (or op(A)) to a dense fp32 [K][N] (or [M][K]) array. */
static float* widen_b(const uint16_t* B, int64_t N, int64_t K, int layout) {
  float* Bf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1) * (size_t)(N > 0 ? N : 1));
  if (!Bf) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j) Bf[k * N + j] = bf16_bits_to_f32(b_elem(B, N, K, layout, k, j));
  return Bf;
}

/*
 * Full rows [row_begin, row_end) of the output.
 *   y_out    fp32 result y after the epilogue, (row_end-row_begin) x N, may be NULL
 *   bf16_out RNE(y) bit patterns, same shape, may be NULL
 *   nthreads OpenMP threads (<= 0: library default)
 *   seconds  if non-NULL, receives the wall time of the contraction+epilogue
 *            loop nest alone (widening to fp32 is excluded)
 * Returns 0 on success, 1 on bad arguments, 2 when out of memory.
 */
int oracle_gemm(const uint16_t* A, const uint16_t* B, const uint16_t* B2, const uint16_t* bias,
                int64_t M, int64_t N, int64_t K, int layout, int epi, int64_t row_begin,
                int64_t row_end, float* y_out, uint16_t* bf16_out, int nthreads,
                double* seconds) {
  if (check_args(A, B, B2, bias, M, N, K, layout, epi)) return 1;
  if (row_begin < 0 || row_end > M || row_begin > row_end) return 1;
  const int gated = (epi == OR_EPI_SWIGLU || epi == OR_EPI_GLU_IDENTITY);
  int b2_layout = layout;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  float* Bf = widen_b(B, N, K, layout);
  float* B2f = gated ? widen_b(B2, N, K, b2_layout) : NULL;
  const int64_t R = row_end - row_begin;
  float* Af = (float*)malloc(sizeof(float) * (size_t)(R > 0 ? R : 1) * (size_t)(K > 0 ? K : 1));
  if (!Bf || !Af || (gated && !B2f)) {
    free(Bf);
    free(B2f);
    free(Af);
    return 2;
  }
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) Af[r * K + k] = bf16_bits_to_f32(a_elem(A, M, K, layout, row_begin + r, k));

  const double t0 = now_s();
  int oom = 0;
#pragma omp parallel
  {
    float* acc = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    float* acc2 = gated ? (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1)) : NULL;
    if (!acc || (gated && !acc2)) {
#pragma omp atomic write
      oom = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < R; ++r) {
        /* one accumulator per output element, products added in ascending k */
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0f;
        if (gated)
          for (int64_t j = 0; j < N; ++j) acc2[j] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
          const float a = Af[r * K + k];
          const float* brow = Bf + k * N;
          for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * brow[j];
          if (gated) {
            const float* b2row = B2f + k * N;
            for (int64_t j = 0; j < N; ++j) acc2[j] = acc2[j] + a * b2row[j];
          }
        }
        for (int64_t j = 0; j < N; ++j) {
          const float y = epilogue(epi, acc[j], gated ? acc2[j] : 0.0f, bias, j);
          if (y_out) y_out[r * N + j] = y;
          if (bf16_out) bf16_out[r * N + j] = f32_to_bf16_rne(y);
        }
      }
    }
    free(acc);
    free(acc2);
  }
  const double t1 = now_s();
  if (seconds) *seconds = t1 - t0;
  free(Af);
  free(Bf);
  free(B2f);
  return oom ? 2 : 0;
}

/*
 * Sampled outputs: element p is (rows[p], cols[p]), computed by the literal
 * triple loop straight from the bf16 storage (no widening pass, no blocking).
 * Same result bits as oracle_gemm.  Returns 0, or 1 on bad arguments.
 */
int oracle_gemm_points(const uint16_t* A, const uint16_t* B, const uint16_t* B2,
                       const uint16_t* bias, int64_t M, int64_t N, int64_t K, int layout,
                       int epi, const int64_t* rows, const int64_t* cols, int64_t npoints,
                       float* y_out, uint16_t* bf16_out, int nthreads) {
  if (check_args(A, B, B2, bias, M, N, K, layout, epi)) return 1;
  if (npoints < 0 || (npoints > 0 && (!rows || !cols))) return 1;
  for (int64_t p = 0; p < npoints; ++p)
    if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return 1;
  const int gated = (epi == OR_EPI_SWIGLU || epi == OR_EPI_GLU_IDENTITY);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t p = 0; p < npoints; ++p) {
    const int64_t i = rows[p], j = cols[p];
    float acc = 0.0f, acc2 = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const float a = bf16_bits_to_f32(a_elem(A, M, K, layout, i, k));
      acc = acc + a * bf16_bits_to_f32(b_elem(B, N, K, layout, k, j));
      if (gated) acc2 = acc2 + a * bf16_bits_to_f32(b_elem(B2, N, K, layout, k, j));
    }
    const float y = epilogue(epi, acc, acc2, bias, j);
    if (y_out) y_out[p] = y;
    if (bf16_out) bf16_out[p] = f32_to_bf16_rne(y);
  }
  return 0;
}

/* The epilogue's building blocks on their own, for checking them against
 * closed forms and independent libraries. */
void oracle_round_bf16(const float* x, uint16_t* out, int64_t n) {
  for (int64_t p = 0; p < n; ++p) out[p] = f32_to_bf16_rne(x[p]);
}

void oracle_gelu_tanh(const float* t, float* y, int64_t n) {
  for (int64_t p = 0; p < n; ++p) y[p] = (float)gelu_tanh_d((double)t[p]);
}

void oracle_silu_mul(const float* g, const float* u, float* y, int64_t n) {
  for (int64_t p = 0; p < n; ++p) y[p] = (float)(silu_d((double)g[p]) * (double)u[p]);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
