// Small products: 64 x 64 output tiles whose whole K (at most 256) sits in
// LDS at once.
//
// A problem of a few tiles with a short K (the 256^3 matmul: sixteen 64 x 64
// tiles, K = 256) leaves each workgroup almost no arithmetic; what it waits
// for is memory latency.  The two-stage kernel (gemm_persistent) waits for
// one global round trip per 64-k step, four at K = 256.  Here a workgroup
// issues every load of its tile at once (operands stored K-contiguous go
// straight into LDS; the others pass through registers and are transposed
// into the same layout), waits once, and then runs all of its MFMAs from
// LDS: one round trip per tile.  The MFMA fragments, their lane layout and
// the epilogue are those of gemm_persistent.
#pragma once

#include "gemm_kernel.hpp"

namespace mmk {

constexpr int kSmallKMax = 256;  // K elements held in LDS per tile

// LDS rows of the small kernel hold all of K: 512 bytes, 32 chunks of 8 k.
// Chunk c of row r sits at physical chunk c ^ s(r), s(r) = (r & 15) ^ (bit 4
// of r moved to bit 2): the 16 consecutive rows of an activation fragment
// read and the comb of a weight fragment read (rows 8a + b, a, b < 4) all
// land on distinct 16-byte positions.
__device__ __forceinline__ uint32_t small_off(int row, int chunk) {
  const int s = (row & 15) ^ ((row >> 2) & 4);
  return (uint32_t)(row * (kSmallKMax * 2) + ((chunk ^ s) << 4));
}

template <bool A_KC, bool B_KC>
__global__ void __launch_bounds__(256) gemm_small(GemmParams p) {
  constexpr int BM = 64, BN = 64, ROWB = kSmallKMax * 2;
  constexpr int FM = 2, FN = 2;  // 32 x 32 per wave, 2 x 2 waves
  __shared__ __attribute__((aligned(1024))) char smem[(BM + BN) * ROWB];  // 64 KiB
  char* const As = smem;
  char* const Bs = smem + BM * ROWB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int G = gridDim.x;
  const int units = p.num_tiles * p.batch;
  const int M = p.M, N = p.N, K = p.K;
  const int KS = (K + 31) / 32;  // MFMA k-steps of 32 (K <= kSmallKMax)

  // fragment addressing (gemm_persistent's): activation fragment fm is rows
  // wrow_a + 16 fm + lx; weight fragment fn is the comb 32 (fn >> 1) +
  // 8 (lx >> 2) + 4 (fn & 1) + (lx & 3) from wrow_b; k-chunk 4 s + lk
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * 32;
  const int wrow_b = wave_n * 32;

  for (int u = blockIdx.x; u < units; u += G) {
    const BatchView v = batch_view(p, u);
    int tm, tn;
    tile_coords(v.tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    if (u != (int)blockIdx.x) __syncthreads();  // the previous tile's reads are done

    // ---- every load of the tile at once
    // K-contiguous operand, rows [r0, r0 + 64) of a [R][K] matrix: wave
    // instruction j fills LDS bytes 1024 j .. (rows 2j and 2j + 1); lane L
    // writes physical chunk L % 32 of row 2j + L / 32, fetching the logical
    // chunk that maps there.  Chunks at k >= K read 16 zero bytes; rows past
    // R repeat row R - 1 (their outputs are never stored).
    auto load_kc = [&](const uint16_t* base, int r0, int R, char* dst) {
      // (a loop rather than unrolled: unrolled, the eight LDS destinations and
      // addresses held at once overflowed the scalar registers)
#pragma unroll 1
      for (int q = 0; q < 8; ++q) {
        const int j = q * 4 + wave;
        const int row = 2 * j + (lane >> 5);
        const int s = (row & 15) ^ ((row >> 2) & 4);
        const int c = (lane & 31) ^ s;
        const int k = 8 * c;
        const int rg = r0 + row < R ? r0 + row : R - 1;
        const uint16_t* g = k < K ? base + (int64_t)rg * K + k : reinterpret_cast<const uint16_t*>(g_zero_chunk);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g),
                                         (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, 0, 0);
      }
    };
    // M- or N-contiguous operand, columns [r0, r0 + 64) of a [K][R] matrix:
    // thread t loads the 8 x 8 block of k-rows 8 (t / 8) .. + 7 and columns
    // r0 + 8 (t % 8) .. + 7 (eight 16-byte reads; R is a multiple of 8), zero
    // past K or R; stored transposed below.
    auto load_mn = [&](const uint16_t* base, int r0, int R, u32x4 (&blk)[8]) {
      const int kb = tid >> 3, cb = tid & 7;
      const int col = r0 + 8 * cb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 8 * kb + i;
        blk[i] = (col < R && k < K) ? *reinterpret_cast<const u32x4*>(base + (int64_t)k * R + col) : zero4();
      }
    };
    // block -> 8 LDS rows (columns 8 cb + j) of 8 k each (chunk kb)
    auto store_mn = [&](const u32x4 (&blk)[8], char* dst) {
      const int kb = tid >> 3, cb = tid & 7;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int word = j >> 1;
        const bool hi = j & 1;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = blk[2 * e][word];
          const uint32_t b = blk[2 * e + 1][word];
          w[e] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<u32x4*>(dst + small_off(8 * cb + j, kb)) = w;
      }
    };
    u32x4 blk_a[8], blk_b[8];
    if constexpr (A_KC) load_kc(v.A, m0, M, As);
    else load_mn(v.A, m0, M, blk_a);
    if constexpr (B_KC) load_kc(v.B, n0, N, Bs);
    else load_mn(v.B, n0, N, blk_b);
    __builtin_amdgcn_s_waitcnt(0);  // one round trip
    if constexpr (!A_KC) store_mn(blk_a, As);
    if constexpr (!B_KC) store_mn(blk_b, Bs);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- MFMAs over all of K from LDS (chunks past K are zero)
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < KS; ++s) {
      bf16x8 xb[FN], ya[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int rb = wrow_b + 32 * (fn >> 1) + 8 * (lx >> 2) + 4 * (fn & 1) + (lx & 3);
        xb[fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + small_off(rb, 4 * s + lk)));
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int ra = wrow_a + 16 * fm + lx;
        ya[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + small_off(ra, 4 * s + lk)));
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[fn], ya[fm], acc[fm][fn], 0, 0, 0);
    }

    // ---- epilogue: a lane holds 8 consecutive columns of fragment pair 0
    const bool has_bias = (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU);
    const bool gelu = (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU);
    const int n = n0 + wrow_b + 8 * lk;
    float bv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      bv[j] = (has_bias && n + j < N) ? __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16) : 0.f;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = m0 + wrow_a + 16 * fm + lx;
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = acc[fm][j >> 2][j & 3] + bv[j];
      if (m >= M) continue;
      if (p.out_pre) store_row8(p.out_pre, p.out_f32, p.out_vec, m, N, n, y);
      if (gelu) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = gelu_tanh(y[j]);
      }
      store_row8(v.out, p.out_f32, p.out_vec, m, N, n, y);
    }
  }
}

}  // namespace mmk
