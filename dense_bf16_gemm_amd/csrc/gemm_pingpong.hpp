// gemm_pingpong.hpp -- K-contiguous ("NT") GEMM with a two-group ping-pong
// schedule: 8 waves per workgroup, two per SIMD, one 256 x 256 output tile.
//
// The pages plan a ping-pong persistent matmul in which two consumer groups
// take turns on the matrix units (issue "Automate performant Hopper matmul",
// section "Persistent matmul" and the roadmap).  On gfx950 the groups are the
// two waves that share each SIMD:
//   * group 0 = waves 0..3, group 1 = waves 4..7; wave (g, i) owns rows
//     128*(i & 1) and columns 64*(2g + (i >> 1)) of the tile (128 x 64, 32
//     fp32 accumulator blocks in VGPRs);
//   * every k-step has two phases separated by a workgroup barrier.  In
//     phase A group 0 issues its 32 MFMAs while group 1 reads its operand
//     fragments from LDS and issues its share of the global->LDS copies; in
//     phase B the roles swap.  A wave in its MFMA phase issues nothing but
//     MFMAs (at raised priority), so a copy that stalls at issue never holds
//     back the matrix pipe of its SIMD;
//   * the LDS ring, copies, swizzle and epilogue are those of gemm_nt_pipe: 5
//     stages of k32 (64-byte rows, 32 KiB each), buffer_load ... lds copies
//     that read zeros past M/N/K, the ring position running across tiles.
// Phase timeline of k-step t (stage s holds k-step s % 5):
//   A(t): G0 MFMA(t)                | G1 reads frags(t), copies k-step t+4
//   B(t): G0 reads frags(t+1),      | G1 MFMA(t)
//         copies k-step t+5
// Stage t is last read in A(t), so its copies for k-step t+5 start in B(t).
// Before each barrier every wave waits until its own copies of the k-steps
// up to t+1 have landed (vmcnt), so the barrier publishes them.
#pragma once

#include "gemm_nt_pipe.hpp"

namespace mmk {

template <bool FFN>
__global__ void __launch_bounds__(512)
gemm_pingpong(GemmParams p) {
  constexpr int BM = 256, BN = 256;  // LDS tile rows of A and of the weight tile
  constexpr int WTM = 128, WTN = 64;
  constexpr int FM = WTM / 16, FN = WTN / 16;  // 8 x 4 fragments of 16 x 16
  constexpr int OUT_BN = FFN ? BN / 2 : BN;
  constexpr int A_BYTES = BM * kPipeRowB;
  constexpr int STAGE_BYTES = (BM + BN) * kPipeRowB;
  constexpr int S = kPipeStages;           // 5
  constexpr int CPW = 2;                   // 1 KiB copies per wave per operand per k-step
  constexpr int COPIES = 2 * CPW;          // per wave per k-step
  static_assert(BM / 16 == 8 * CPW && BN / 16 == 8 * CPW, "copy split");
  static_assert(!FFN || FN % 4 == 0, "FFN wave tile holds gate and up pairs");

  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wi = wave & 3;
  const int wave_m = wi & 1;
  const int wave_n = 2 * grp + (wi >> 1);
  const int G = gridDim.x;
  const int wg = remap_workgroup(blockIdx.x, G, p.xcd_remap);
  if (wg >= p.num_tiles) return;
  const int my_tiles = (p.num_tiles - wg + G - 1) / G;
  const int KT = p.k_tiles;  // k-steps of 32 per tile
  const int M = p.M, N = p.N, K = p.K;
  const int64_t ld = K;

  // ---- copies (as gemm_nt_pipe): lane L of a 1 KiB copy fills LDS row
  // 16j + L/4, physical chunk L%4, from logical chunk (L%4) ^ swz(row)
  const int crow = lane >> 2;
  const int cchunk = (lane & 3) ^ pipe_swz(crow);
  const uint32_t row_bytes = (uint32_t)ld * 2u;
  const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
  constexpr int kRsrcWord3 = 0x00020000;

  // Per-tile copy state of this wave's load cursor, kept as plain integers;
  // the buffer resources are rebuilt from wave-uniform (readfirstlane)
  // copies at each use, so they always live in scalar registers.
  uint64_t a_base = 0, b0_base = 0, b1_base = 0;
  uint32_t a_rec = 0, b_rec = 0;
  int ld_alt = 0;
  auto enter_tile = [&](int tile_i) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(wg + tile_i * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BM;
    const int mrows = (M - m0) < BM ? (M - m0) : BM;
    a_base = reinterpret_cast<uint64_t>(p.A + (int64_t)m0 * ld);
    a_rec = (uint32_t)mrows * row_bytes;
    const int n0 = tn * OUT_BN;
    const int nrows = (N - n0) < OUT_BN ? (N - n0) : OUT_BN;
    b_rec = (uint32_t)nrows * row_bytes;
    b0_base = reinterpret_cast<uint64_t>(p.B + (int64_t)n0 * ld);
    b1_base = FFN ? reinterpret_cast<uint64_t>(p.B2 + (int64_t)n0 * ld) : b0_base;
    ld_alt = p.k_alt && (tile_i & 1);
  };
  auto rsrc = [&](uint64_t base, uint32_t rec) __attribute__((always_inline)) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    void* ptr = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, (int)__builtin_amdgcn_readfirstlane(rec),
                                             kRsrcWord3);
  };

  // This wave's copies of one k-step: A copies j = wave, wave + 8 and weight
  // copies j = wave, wave + 8 (16 rows each).
  auto issue_copies = [&](int kt, int stage) __attribute__((always_inline)) {
    const int k0 = (ld_alt ? (KT - 1 - kt) : kt) * kPipeBK;
    const uint32_t koff = lane_base + 2u * (uint32_t)k0 +
                          ((k0 + 8 * cchunk) < K ? 0u : 0x80000000u);
    char* st = smem + stage * STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = rsrc(a_base, a_rec);
    const __amdgpu_buffer_rsrc_t rb0 = rsrc(b0_base, b_rec);
    const __amdgpu_buffer_rsrc_t rb1 = FFN ? rsrc(b1_base, b_rec) : rb0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int j = wave + 8 * c;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(st + j * 1024), 16,
          koff + (uint32_t)(16 * j) * row_bytes, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int j = wave + 8 * c;
      const int r0 = 16 * j;
      int prow = r0;
      bool up = false;
      if constexpr (FFN) {
        // each wave column's 64 weight rows: 32 gate rows, then the 32 up rows
        const int wb = r0 / WTN, within = r0 % WTN;
        up = within >= WTN / 2;
        prow = wb * (WTN / 2) + (up ? within - WTN / 2 : within);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          up ? rb1 : rb0, (__attribute__((address_space(3))) void*)(st + A_BYTES + j * 1024), 16,
          koff + (uint32_t)prow * row_bytes, 0, 0, 0);
    }
  };

  // Load cursor (k-step whose copies this wave issues next), as in gemm_nt_pipe.
  int ld_tile = 0, ld_kt = 0, ld_stage = 0;
  enter_tile(0);
  auto issue_next = [&]() __attribute__((always_inline)) {
    issue_copies(ld_kt, ld_stage);
    ld_stage = (ld_stage + 1 == S) ? 0 : ld_stage + 1;
    if (ld_tile < my_tiles) {
      if (++ld_kt == KT) {
        ld_kt = 0;
        ++ld_tile;
        if (ld_tile < my_tiles) enter_tile(ld_tile);
        else ld_kt = KT - 1;  // past the end: re-copy the last k-step (never read)
      }
    }
  };

  // ---- fragments
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
  const uint32_t a_off = (uint32_t)((wrow_a + lx) * kPipeRowB + ((lk ^ pipe_swz(lx)) << 4));
  const int rbb = 8 * (lx >> 2) + (lx & 3);
  const uint32_t b_off =
      (uint32_t)(A_BYTES + (wrow_b + rbb) * kPipeRowB + ((lk ^ pipe_swz(rbb)) << 4));

  bf16x8 fa[FM], fb[FN];
  f32x4 acc[FM][FN];

  auto read_frags = [&](int stage) __attribute__((always_inline)) {
    const char* st = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      fb[fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              st + b_off + (32 * (fn >> 1) + 4 * (fn & 1)) * kPipeRowB));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      fa[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              st + a_off + 16 * fm * kPipeRowB));
  };

  auto mfmas = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // the barrier between phases; before it, this wave's copies older than the
  // newest three k-steps have landed and its fragment reads are done
  auto phase_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * COPIES));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: k-steps 0..3 copied (stages 0..3); group 0 reads frags(0)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue_next();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * COPIES));
  __builtin_amdgcn_s_barrier();
  // Group 0 reads frags(0) and copies k-step 4 before its loop (it copies
  // k-step t+5 in B(t)); group 1 copies k-step t+4 in A(t).

  // ---- epilogue of this wave's 128 x 64 block (as gemm_nt_pipe)
  auto epilogue = [&](int tile_i) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(wg + tile_i * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m_base = tm * BM + wrow_a + lx;
    const int g8 = 8 * lk;
    constexpr int PAIRS = FFN ? FN / 4 : FN / 2;
    const bool has_bias = (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU);
    const bool gelu = (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU);
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int n = FFN ? tn * OUT_BN + wave_n * (WTN / 2) + 32 * pr + g8
                        : tn * OUT_BN + wrow_b + 32 * pr + g8;
      float bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float b = 0.f;
        if (has_bias && n + j < N) b = __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16);
        bv[j] = b;
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int m = m_base + 16 * fm;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = acc[fm][2 * pr + (j >> 2)][j & 3];
          float y;
          if constexpr (FFN) {
            const float u = acc[fm][FN / 2 + 2 * pr + (j >> 2)][j & 3];
            y = (p.epi == EPI_SWIGLU) ? silu(a) * u : a * u;
          } else {
            const float t = a + bv[j];
            y = gelu ? gelu_tanh(t) : t;
          }
          v[j] = y;
        }
        if (m >= M) continue;
        if (p.out_f32) {
          float* o = reinterpret_cast<float*>(p.out) + (int64_t)m * N + n;
          if (p.out_vec && n + 8 <= N) {
            reinterpret_cast<f32x4*>(o)[0] = f32x4{v[0], v[1], v[2], v[3]};
            reinterpret_cast<f32x4*>(o)[1] = f32x4{v[4], v[5], v[6], v[7]};
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (n + j < N) o[j] = v[j];
          }
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (int64_t)m * N + n;
          if (p.out_vec && n + 8 <= N) {
            u32x4 w;
            w[0] = pack_bf16x2(v[0], v[1]);
            w[1] = pack_bf16x2(v[2], v[3]);
            w[2] = pack_bf16x2(v[4], v[5]);
            w[3] = pack_bf16x2(v[6], v[7]);
            *reinterpret_cast<u32x4*>(o) = w;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (n + j < N) o[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[j]));
          }
        }
      }
    }
  };

  // The tile loop, one straight-line copy per group (the roles never merge,
  // so the accumulators keep their registers); both copies execute the same
  // barriers.
  auto run = [&](auto group) __attribute__((always_inline)) {
    constexpr int GRP = decltype(group)::value;
    if constexpr (GRP == 0) {
      read_frags(0);
      issue_next();
    }
    int rd_stage = 0;  // stage of k-step t
    for (int tile_i = 0; tile_i < my_tiles; ++tile_i) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kt = 0; kt < KT; ++kt) {
        const int next_stage = (rd_stage + 1 == S) ? 0 : rd_stage + 1;
        if constexpr (GRP == 0) {
          mfmas();                  // A(t)
          phase_end();
          read_frags(next_stage);   // B(t)
          issue_next();
          phase_end();
        } else {
          read_frags(rd_stage);     // A(t)
          issue_next();
          phase_end();
          mfmas();                  // B(t)
          phase_end();
        }
        rd_stage = next_stage;
      }
      epilogue(tile_i);
    }
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
}

}  // namespace mmk
