// gemm_nt_pipe.hpp -- the K-contiguous ("NT": A [M][K], B [N][K]) fast path.
//
// Same persistent schedule, epilogue and result as gemm_persistent (see
// gemm_kernel.hpp), with a deeper software pipeline built for one wave per
// SIMD feeding the matrix cores without stalls:
//   * a ring of 4 LDS stages of 32 k each (rows of 64 bytes).  The copies for
//     k-step i+4 are issued at the top of k-step i into the stage that held
//     k-step i, so global loads have three k-steps of MFMA work to land (the
//     prefetch depth the pages ask for: issue "Automate performant Hopper
//     matmul", section "K loop efficiency": prefetch_gap > 1);
//   * MFMA operand fragments are read from LDS one k-step ahead into a
//     second register set, interleaved with the current k-step's MFMAs, so
//     no MFMA waits on an LDS read;
//   * one wait + barrier per k-step: it publishes the stage the next
//     fragments come from and frees the stage the next copies go to (the
//     write-after-read hazard of section "Syncing issues");
//   * the ring position is a running k-step counter over all tiles of the
//     workgroup, so nothing restarts at a tile boundary and the next tile's
//     first stages are loading while this tile's epilogue runs (sections
//     "Syncing persistent matmuls" and "Syncing issues").
// The step at which a wave issues copies past its last k-step re-copies that
// last k-step (always in bounds), so every k-step issues the same number of
// copies and the wait count is a constant.
#pragma once

#include "gemm_kernel.hpp"

namespace mmk {

constexpr int kPipeBK = 32;      // k per stage
constexpr int kPipeRowB = 64;    // LDS bytes per row of a stage
constexpr int kPipeStages = 5;

// Swizzle of 64-byte rows: chunk ^ (bit 3 of row) << 1, measured conflict
// free (SQ_LDS_BANK_CONFLICT) for 16 consecutive rows and for the 4x4-row
// comb of the permuted weight fragments.
__host__ __device__ __forceinline__ int pipe_swz(int row) { return (row >> 2) & 2; }

// s_waitcnt immediate for gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4
// (left at its maximum), lgkmcnt 11:8 (0).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

template <int BM, int BN, int WGM, int WGN, bool FFN>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_nt_pipe(GemmParams p) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int OUT_BN = FFN ? BN / 2 : BN;
  constexpr int A_BYTES = BM * kPipeRowB;
  constexpr int STAGE_BYTES = (BM + BN) * kPipeRowB;
  constexpr int LA = BM / 16 / NW;  // 1 KiB copies of A per wave per k-step
  constexpr int LB = BN / 16 / NW;
  constexpr int LOADS = LA + LB;
  static_assert(LA >= 1 && LB >= 1 && (BM / 16) % NW == 0 && (BN / 16) % NW == 0, "copy split");
  static_assert(FN % 2 == 0 && (!FFN || FN % 4 == 0), "fragment pairs");
  static_assert(WTN % 32 == 0 && WTM % 16 == 0, "wave tile");
  static_assert((kPipeStages - 1) * LOADS <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[kPipeStages * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wave_m = wave / WGN;
  const int wave_n = wave % WGN;
  const int G = gridDim.x;
  const int wg = remap_workgroup(blockIdx.x, G, p.xcd_remap);
  if (wg >= p.num_tiles) return;
  const int my_tiles = (p.num_tiles - wg + G - 1) / G;
  const int KT = p.k_tiles;  // k-steps of 32 per tile, even
  const int M = p.M, N = p.N, K = p.K;
  const int64_t ld = K;  // both operands are [rows][K]

  // ---- copies: buffer_load ... lds, one 1 KiB copy = 16 LDS rows.  Lane L
  // writes LDS row 16j + L/4, physical chunk L%4, and so fetches logical
  // chunk (L%4) ^ swz(row); bit 3 of that row is bit 3 of L/4, so the chunk
  // is the same for every j.  Each operand's rows of the current tile are one
  // buffer resource whose size ends at the last valid row: copies of rows
  // past M (or N) and of chunks past K (pushed out of range by setting the
  // offset's top bit) read as zero, with no clamping and no branches.  The
  // host only picks this kernel when a tile's rows span < 2^31 bytes.
  const int crow = lane >> 2;
  const int cchunk = (lane & 3) ^ pipe_swz(crow);
  const uint32_t row_bytes = (uint32_t)ld * 2u;
  const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
  constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family

  // Per-tile copy state of the load cursor, set when the cursor enters a
  // tile: buffer resources of the tile's A rows and weight rows, and the K
  // direction.  Each k-step then costs a handful of instructions per copy.
  __amdgpu_buffer_rsrc_t ra, rb0, rb1;
  int ld_alt = 0;
  auto enter_tile = [&](int tile_i) {
    int tm, tn;
    tile_coords(wg + tile_i * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BM;
    const int mrows = (M - m0) < BM ? (M - m0) : BM;
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.A + (int64_t)m0 * ld), (short)0,
                                           (int)((uint32_t)mrows * row_bytes), kRsrcWord3);
    const int n0 = tn * OUT_BN;
    const int nrows = (N - n0) < OUT_BN ? (N - n0) : OUT_BN;
    const int nrec = (int)((uint32_t)nrows * row_bytes);
    rb0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.B + (int64_t)n0 * ld), (short)0,
                                            nrec, kRsrcWord3);
    rb1 = rb0;
    if constexpr (FFN)
      rb1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.B2 + (int64_t)n0 * ld),
                                              (short)0, nrec, kRsrcWord3);
    ld_alt = p.k_alt && (tile_i & 1);
  };

  // Lane offset of the copies of k-step kt of the cursor's tile: chunks past
  // K are pushed out of range (top bit) and read as zero.
  auto copy_koff = [&](int kt) {
    const int k0 = (ld_alt ? (KT - 1 - kt) : kt) * kPipeBK;
    return lane_base + 2u * (uint32_t)k0 + ((k0 + 8 * cchunk) < K ? 0u : 0x80000000u);
  };

  // Issues copy q (of LOADS) of one k-step into the stage at byte offset
  // stage_off: copies 0..LA-1 fill A rows, the rest weight rows.
  auto issue_copy = [&](int q, uint32_t koff, int stage_off) {
    if (q < LA) {
      const int j = q * NW + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(smem + stage_off + j * 1024), 16,
          koff + (uint32_t)(16 * j) * row_bytes, 0, 0, 0);
    } else {
      const int j = (q - LA) * NW + wave;
      const int r0 = 16 * j;  // first B-tile row of this copy
      int prow = r0;          // its row within the weight panel
      bool up = false;
      if constexpr (FFN) {
        // each wave's B rows: WTN/2 gate rows then the up rows of the same columns
        const int wb = r0 / WTN, within = r0 % WTN;
        up = within >= WTN / 2;
        prow = wb * (WTN / 2) + (up ? within - WTN / 2 : within);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          up ? rb1 : rb0, (__attribute__((address_space(3))) void*)(smem + stage_off + A_BYTES + j * 1024),
          16, koff + (uint32_t)prow * row_bytes, 0, 0, 0);
    }
  };

  // ---- fragment addresses (bit 3 of every fragment row is a lane constant)
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
  const uint32_t a_off = (uint32_t)((wrow_a + lx) * kPipeRowB + ((lk ^ pipe_swz(lx)) << 4));
  const int rb = 8 * (lx >> 2) + (lx & 3);
  const uint32_t b_off =
      (uint32_t)(A_BYTES + (wrow_b + rb) * kPipeRowB + ((lk ^ pipe_swz(rb)) << 4));

  bf16x8 fa[2][FM], fb[2][FN];
  f32x4 acc[FM][FN];

  // Fragment f of a k-step: f < FN is weight fragment f, else A fragment f-FN.
  auto read_frag = [&](const char* stage, int f, bf16x8* a, bf16x8* b) {
    if (f < FN)
      b[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                            stage + b_off + (32 * (f >> 1) + 4 * (f & 1)) * kPipeRowB));
    else
      a[f - FN] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                 stage + a_off + 16 * (f - FN) * kPipeRowB));
  };
  auto read_frags = [&](const char* stage, bf16x8* a, bf16x8* b) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      b[fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                             stage + b_off + (32 * (fn >> 1) + 4 * (fn & 1)) * kPipeRowB));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      a[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                             stage + a_off + 16 * fm * kPipeRowB));
  };

  // ---- load cursor: (ld_tile, ld_kt) is the k-step whose copies are issued
  // next; past the last k-step it keeps re-copying that k-step (in bounds,
  // never read).  ld_stage is its ring slot.
  int ld_tile = 0, ld_kt = 0, ld_stage = 0;
  enter_tile(0);
  // Advances the cursor; entering a new tile rebuilds the per-tile state.
  // Kept out of the scheduling region of the MFMAs (it may branch).
  auto advance_cursor = [&]() {
    ld_stage = (ld_stage + 1 == kPipeStages) ? 0 : ld_stage + 1;
    if (ld_tile < my_tiles) {
      if (++ld_kt == KT) {
        ld_kt = 0;
        ++ld_tile;
        if (ld_tile < my_tiles) enter_tile(ld_tile);
        else ld_kt = KT - 1;  // stay on the last k-step
      }
    }
  };
  auto issue_next = [&]() {
    const uint32_t koff = copy_koff(ld_kt);
#pragma unroll
    for (int q = 0; q < LOADS; ++q) issue_copy(q, koff, ld_stage * STAGE_BYTES);
  };

  // ---- prologue: k-steps 0..3 in flight; wait for k-step 0 and read its
  // fragments.  Invariant at the top of k-step it: copies of k-steps it+1,
  // it+2, it+3 are outstanding and the fragments of k-step it are in
  // registers.
#pragma unroll
  for (int s = 0; s < kPipeStages; ++s) {
    issue_next();
    advance_cursor();
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((kPipeStages - 1) * LOADS));
  __builtin_amdgcn_s_barrier();
  read_frags(smem, fa[0], fb[0]);

  // One k-step: P = parity of the running counter (register set in use).
  // rd_stage: the ring slot holding the k-step after the current one
  int rd_stage = 1;
  auto kstep = [&](auto par) {
    constexpr int P = decltype(par)::value;
    // own copies of k-step it+1 done, own fragment reads done; then all
    // waves: k-step it+1 is visible and stage it % 4 (whose data every wave
    // already holds in registers) is free for the copies of k-step it+4
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((kPipeStages - 2) * LOADS));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // LOADS chunks of {one copy, a share of the next fragments, a share of
    // the MFMAs}, fenced from each other: the copies and reads are spread
    // evenly over the MFMAs.  Bunched copies overfill the vector-memory
    // address queue, and a wave stalled on a copy cannot issue the MFMAs
    // behind it.
    constexpr int NMFMA = FM * FN;
    constexpr int NDS = FM + FN;
    const uint32_t koff = copy_koff(ld_kt);
    const char* rd = smem + rd_stage * STAGE_BYTES;
#pragma unroll
    for (int c = 0; c < LOADS; ++c) {
      issue_copy(c, koff, ld_stage * STAGE_BYTES);
#pragma unroll
      for (int f = (c * NDS) / LOADS; f < ((c + 1) * NDS) / LOADS; ++f) read_frag(rd, f, fa[P ^ 1], fb[P ^ 1]);
#pragma unroll
      for (int i = (c * NMFMA) / LOADS; i < ((c + 1) * NMFMA) / LOADS; ++i) {
        const int fm = i / FN, fn = i % FN;
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[P][fn], fa[P][fm], acc[fm][fn], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int tile_i = 0; tile_i < my_tiles; ++tile_i) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // k-steps in pairs so each register set has a fixed role (the host makes
    // KT even: a padding k-step past K reads zeros)
    for (int kt = 0; kt < KT; kt += 2) {
      kstep(std::integral_constant<int, 0>{});
      advance_cursor();
      rd_stage = (rd_stage + 1 == kPipeStages) ? 0 : rd_stage + 1;
      kstep(std::integral_constant<int, 1>{});
      advance_cursor();
      rd_stage = (rd_stage + 1 == kPipeStages) ? 0 : rd_stage + 1;
    }
    // ---- epilogue (same arithmetic and store pattern as gemm_persistent)
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
  }
}

}  // namespace mmk
