// Skinny products: at most 16 rows of activations against a large weight
// (the decode step of a served model at small batch: x [M][K], M <= 16,
// W [N][K]).
//
// Such a product is bound by reading W once from HBM; its MFMA work is small.
// The 256-row tiles of the slab kernel would spend almost all of their MFMAs
// on rows past M, so here a workgroup takes 16 of W's rows (16 output
// columns) and streams them once: its four waves split the k range into four
// parts, each wave loads its weight and activation fragments straight from
// global memory into registers, a few 32-k steps ahead, and the parts meet in
// LDS in a fixed order.  With a workspace the k range is also split over S
// workgroups per column block: each writes its fp32 sums to slice s of the
// workspace and skinny_reduce adds the slices in k order.  Results: fp32 sums
// of the bf16 products, the epilogue on the sum, one rounding -- the
// contraction and epilogue of the other kernels.
//
// Measured against the slab kernel's split path (256 x 128 tiles, rows past
// M computed and dropped), with a workspace: 16 x 14336 x 4096 35.6 -> 30.0
// us, 16 x 8192 x 8192 34.2 -> 33.4 us, 8 x 8192 x 8192 34.2 -> 28.3 us.  A
// 64-row form of the same design (four waves each re-reading the activation
// fragments for their own column block) was slower than the slab path (80
// against 35 us at 64 x 8192 x 8192), and non-temporal weight loads cost a
// third (each load reads 64-byte halves of 16 lines; the other halves then
// miss).
#pragma once

#include "gemm_kernel.hpp"

namespace mmk {

struct SkinnyParams {
  const uint16_t* A;     // x [M][K]
  const uint16_t* B;     // W [N][K]
  const uint16_t* bias;  // [N] or null
  void* out;             // [M][N], bf16 or fp32
  float* part;           // [S][M][N] fp32 partial sums (S > 1), else null
  int M, N, K;
  int kc;      // k per workgroup slice (a multiple of 32); the last may be shorter
  int slices;  // S
  int epi;
  int out_f32;
};

constexpr int kSkinnyMaxM = 16;
constexpr int kSkinnyDepth = 4;  // 32-k steps of loads in flight per wave

// epilogue of one output: + bias, activation, one rounding
__device__ __forceinline__ void skinny_store(const SkinnyParams& p, int m, int n, float v) {
  if (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU) v += __builtin_bit_cast(float, (uint32_t)p.bias[n] << 16);
  if (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU) v = gelu_tanh(v);
  if (p.out_f32)
    reinterpret_cast<float*>(p.out)[(int64_t)m * p.N + n] = v;
  else
    reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.N + n] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

__global__ void __launch_bounds__(256) gemm_skinny(SkinnyParams p) {
  constexpr int D = kSkinnyDepth;
  __shared__ f32x4 red[3 * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the k part
  const int lx = lane & 15, lk = lane >> 4;
  const int nblocks = (p.N + 15) / 16;
  const int s = __builtin_amdgcn_readfirstlane((int)blockIdx.x / nblocks);
  const int nb = (int)blockIdx.x - s * nblocks;
  const int M = p.M, N = p.N, K = p.K;

  // the workgroup's slice [kbeg, kend) of K, cut into four parts of whole
  // 32-k steps, one per wave
  const int kbeg = s * p.kc;
  const int kend = min(K, kbeg + p.kc);
  const int steps = (kend - kbeg + 31) / 32;
  const int per = (steps + 3) / 4;
  const int j0 = wave * per, j1 = min(steps, j0 + per);
  const int n = nb * 16 + lx;  // the weight row (output column) this lane loads
  const bool n_ok = n < N, m_ok = lx < M;
  const uint16_t* wrow = p.B + (int64_t)(n_ok ? n : 0) * K;
  const uint16_t* xrow = p.A + (int64_t)(m_ok ? lx : 0) * K;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 wq[D], xq[D];
  // fragments of step j: weight row n and activation row lx, 8 k from
  // kbeg + 32 j + 8 lk; zeros past the part, K, N or M (masked lanes keep an
  // address inside the operands: k = 0 of row 0)
  auto load = [&](int j, int slot) __attribute__((always_inline)) {
    const int k = kbeg + 32 * j + 8 * lk;
    const bool k_ok = j < j1 && k < kend;
    const int kk = k_ok ? k : 0;
    wq[slot] = (k_ok && n_ok) ? *reinterpret_cast<const u32x4*>(wrow + kk) : zero4();
    xq[slot] = (k_ok && m_ok) ? *reinterpret_cast<const u32x4*>(xrow + kk) : zero4();
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(j0 + d, d);
  for (int j = j0; j < j1; j += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xq[d]), __builtin_bit_cast(bf16x8, wq[d]),
                                                    acc, 0, 0, 0);
      load(j + d + D, d);
    }
  }

  // the k parts meet in LDS: parts 1..3 store, part 0 adds them in order
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave > 0 || !n_ok) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const f32x4 v = red[q * 64 + lane];
    acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
  }
  // lane (lx, lk) holds rows 4 lk + i, i = 0..3, of column n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * lk + i;
    if (m >= M) continue;
    if (p.slices > 1)
      p.part[((int64_t)s * M + m) * N + n] = acc[i];
    else
      skinny_store(p, m, n, acc[i]);
  }
}

// Second launch of a split skinny product: each output is the sum of its S
// slices in k order, then the epilogue and one rounding.
__global__ void __launch_bounds__(256) skinny_reduce(SkinnyParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t mn = (int64_t)p.M * p.N;
  if (i >= mn) return;
  float v = p.part[i];
  for (int s = 1; s < p.slices; ++s) v += p.part[(int64_t)s * mn + i];
  skinny_store(p, (int)(i / p.N), (int)(i % p.N), v);
}

}  // namespace mmk
