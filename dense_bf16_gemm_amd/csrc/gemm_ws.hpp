// gemm_ws.hpp -- wave-specialized producer/consumer variant of the slab
// kernel (K-contiguous operands, 256 x 128 tiles, eight waves).
//
// The pages' default for Hopper matmuls is warp specialization: some warps
// only issue the loads into shared memory, the others only run the MMAs
// (issue "Automate performant Hopper matmul", sections "K loop efficiency"
// and "Syncing persistent matmuls").  Here, on gfx950:
//   * waves 4..7 (producers, one per SIMD) issue every global->LDS copy
//     (buffer_load ... lds, whole 128-byte lines, the slab kernel's row
//     swizzle) and wait for them; they hold no accumulators and read no LDS;
//   * waves 0..3 (consumers) only read fragments from LDS and issue MFMAs;
//     each owns a 128 x 64 block of the 256 x 128 tile (128 fp32
//     accumulators: two waves per SIMD must fit in its 512 registers per
//     lane, which is why the tile is half the slab kernel's);
//   * an LDS ring of 3 stages of one 64-k super-step (A 256 rows + weight
//     128 rows of 128 bytes = 48 KiB); one workgroup barrier per super-step
//     hands stage s+1 to the consumers and stage s-1 back to the producers.
// Barrier B(s+1) sits inside super-step s, after the consumers' first two
// MFMA rows of its second k-step: by then they have read every fragment of
// stage s into registers.  Between B(s) and B(s+1) the producers issue the
// copies of super-step s+2 into stage (s+2) % 3 = (s-1) % 3 and wait until
// those of s+1 have landed.  Both roles pass the same number of barriers
// (one before the loop, one per super-step).
// Measured against the cooperative slab kernel; selected only by the
// configuration override (PIPE=4 with BN=128).
#pragma once

#include "gemm_nt_slab.hpp"

namespace mmk {

constexpr int kWsStages = 3;

__global__ void __launch_bounds__(512) gemm_ws(GemmParams p) {
  constexpr int BM = 256, BN = 128;  // tile: activation rows, weight rows (output columns)
  constexpr int WTM = 128, WTN = 64;  // consumer block
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_BYTES = BM * kSlabRowB;
  constexpr int STAGE = A_BYTES + BN * kSlabRowB;  // 48 KiB
  constexpr int CA = BM / 8 / 4, CB = BN / 8 / 4;  // copies per producer per super-step
  constexpr int CPP = CA + CB;
  constexpr int kRsrcWord3 = 0x00020000;
  __shared__ __attribute__((aligned(1024))) char smem[kWsStages * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x;
  const int wg = __builtin_amdgcn_readfirstlane(remap_workgroup(blockIdx.x, G, p.xcd_remap));
  if (wg >= p.num_tiles) return;
  const int my_tiles = __builtin_amdgcn_readfirstlane((p.num_tiles - wg + G - 1) / G);
  const int KS = p.k_tiles;  // super-steps of 64 per tile (>= 2)
  const int S = my_tiles * KS;
  const int M = p.M, N = p.N, K = p.K;
  const uint32_t row_bytes = (uint32_t)K * 2u;

  if (wave >= 4) {
    // ---------------------------------------------------------- producers
    const int pw = wave - 4;
    // lane L of copy j fills stage row 8j + L/8, physical chunk L%8, from
    // logical chunk (L%8) ^ lds_swz(row); j = 4c + pw, so bit 4 of the row
    // is bit 1 of pw
    const int crow = lane >> 3;
    const int cchunk = (lane & 7) ^ lds_swz(crow + 8 * (pw & 2));
    const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
    auto issue = [&](int s) __attribute__((always_inline)) {
      const int ti = __builtin_amdgcn_readfirstlane(s / KS);
      const int ks = s - ti * KS;
      int tm, tn;
      tile_coords(wg + ti * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
      tm = __builtin_amdgcn_readfirstlane(tm);
      tn = __builtin_amdgcn_readfirstlane(tn);
      const int m0 = tm * BM, n0 = tn * BN;
      const uint32_t mrows = (uint32_t)((M - m0) < BM ? (M - m0) : BM);
      const uint32_t nrows = (uint32_t)((N - n0) < BN ? (N - n0) : BN);
      const uint32_t kbytes = (uint32_t)ks * (uint32_t)kSlabRowB;
      const uint64_t abase = reinterpret_cast<uint64_t>(p.A + (int64_t)m0 * K) + kbytes;
      const uint64_t bbase = reinterpret_cast<uint64_t>(p.B + (int64_t)n0 * K) + kbytes;
      const int stage = s % kWsStages;
      // (readfirstlane returns a signed int: each half goes through uint32_t
      // so that the low word is not sign-extended into the high one)
      const uint32_t a_lo = __builtin_amdgcn_readfirstlane((uint32_t)abase);
      const uint32_t a_hi = __builtin_amdgcn_readfirstlane((uint32_t)(abase >> 32));
      const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)bbase);
      const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(bbase >> 32));
      const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(((uint64_t)a_hi << 32) | a_lo), (short)0,
          (int)__builtin_amdgcn_readfirstlane(mrows * row_bytes - kbytes), kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void*>(((uint64_t)b_hi << 32) | b_lo), (short)0,
          (int)__builtin_amdgcn_readfirstlane(nrows * row_bytes - kbytes), kRsrcWord3);
#pragma unroll
      for (int c = 0; c < CA; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(smem + stage * STAGE + (4 * c + pw) * 1024), 16,
            lane_base + (uint32_t)(8 * (4 * c + pw)) * row_bytes, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < CB; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(smem + stage * STAGE + A_BYTES + (4 * c + pw) * 1024),
            16, lane_base + (uint32_t)(8 * (4 * c + pw)) * row_bytes, 0, 0, 0);
    };
    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPP));  // super-step 0 landed
    __builtin_amdgcn_s_barrier();                       // B(0)
    for (int s = 0; s < S; ++s) {
      if (s + 2 < S) {
        issue(s + 2);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPP));  // s+1 landed, s+2 in flight
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      }
      __builtin_amdgcn_s_barrier();  // B(s+1)
    }
    return;
  }

  // ------------------------------------------------------------ consumers
  const int wave_m = wave & 1, wave_n = wave >> 1;
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
  // fragment offsets as in gemm_nt_slab: activation rows wrow_a + 16 fm + lx;
  // the comb of weight rows wrow_b + 32 (fn >> 1) + 8 (lx >> 2) + 4 (fn & 1)
  // + (lx & 3), so that a lane owns 8 consecutive output columns of a pair
  const uint32_t a_x0 = (uint32_t)((wrow_a + lx) * kSlabRowB + ((lk ^ (lx & 7)) << 4));
  const uint32_t b_x0 = (uint32_t)(A_BYTES + (wrow_b + 8 * (lx >> 2) + (lx & 3)) * kSlabRowB +
                                   ((lk ^ (lx & 3) ^ (((lx >> 3) & 1) << 2)) << 4));
  bf16x8 fa[FM];
  bf16x8 fb[2][FN];
  f32x4 acc[FM][FN];
  auto read_a = [&](int fm, int h, uint32_t base) __attribute__((always_inline)) {
    const uint32_t off = (((h ^ fm) & 1) ? (base ^ 64u) : base) + (uint32_t)(16 * fm * kSlabRowB);
    fa[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + off));
  };
  auto read_b = [&](int set, int fn, int h, uint32_t base) __attribute__((always_inline)) {
    const uint32_t off = (((h ^ fn) & 1) ? (base ^ 64u) : base) +
                         (uint32_t)((4 * (fn & 1) + 32 * (fn >> 1)) * kSlabRowB);
    fb[set][fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + off));
  };
  auto mfma_row = [&](int r, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      acc[r][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[set][fn], fa[r], acc[r][fn], 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // epilogue of tile i of this workgroup, straight from the accumulators
  const bool has_bias = (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU);
  const bool act_on = (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU);
  auto epilogue = [&](int ti) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(wg + ti * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m_base = tm * BM + wrow_a + lx;
    constexpr int PAIRS = FN / 2;
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int n = tn * BN + wrow_b + 32 * pr + 8 * lk;
      float bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bv[j] = (has_bias && n + j < N) ? __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16) : 0.f;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int m = m_base + 16 * fm;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = acc[fm][2 * pr + (j >> 2)][j & 3] + bv[j];
        if (m >= M) continue;
        if (act_on) gelu_tanh8(v);
        store_row8(p.out, p.out_f32, p.out_vec, m, N, n, v);
      }
    }
  };

  auto stage_base = [](int s) __attribute__((always_inline)) {
    return (uint32_t)((s % kWsStages) * STAGE);
  };
  __builtin_amdgcn_s_barrier();  // B(0)
#pragma unroll
  for (int f = 0; f < FM; ++f) read_a(f, 0, a_x0);
#pragma unroll
  for (int f = 0; f < FN; ++f) read_b(0, f, 0, b_x0);
  int ti = 0, ks = 0;
  for (int s = 0; s < S; ++s) {
    const uint32_t st = stage_base(s), nst = stage_base(s + 1);
    // k-step 2s: half 0 in registers; half 1 of stage s into fa and fb[1]
#pragma unroll
    for (int r = 0; r < FM; ++r) {
      mfma_row(r, 0);
      read_a(r, 1, st + a_x0);
      if (r < FN) read_b(1, r, 1, st + b_x0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // k-step 2s+1: rows 0 and 1, then the barrier (every fragment of stage s
    // is in registers once the LDS reads have returned)
    mfma_row(0, 1);
    mfma_row(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();  // B(s+1)
    __builtin_amdgcn_sched_barrier(0);
    read_a(0, 0, nst + a_x0);
    read_a(1, 0, nst + a_x0);
#pragma unroll
    for (int r = 2; r < FM; ++r) {
      mfma_row(r, 1);
      read_a(r, 0, nst + a_x0);
      if (r - 2 < FN) read_b(0, r - 2, 0, nst + b_x0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (++ks == KS) {
      epilogue(ti);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      ks = 0;
      ++ti;
    }
  }
}

}  // namespace mmk
