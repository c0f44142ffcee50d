// gemm_pp.hpp -- ping-pong persistent GEMM: two wave groups own alternate
// output tiles, and each group's epilogue runs while the other group's MFMAs
// run (K-contiguous operands, 256 x 128 tiles, eight waves).
//
// The pages plan a ping-pong persistent matmul (issue "Automate performant
// Hopper matmul", section "Persistent matmul", and its roadmap): two
// consumer groups alternate on output tiles so that one group's epilogue
// overlaps the other group's main loop.  Here, on gfx950:
//   * waves 0..3 are group 0, waves 4..7 group 1, one wave of each group per
//     SIMD; a group's four waves hold a 256 x 128 tile as 2 x 2 blocks of
//     128 x 64 (128 fp32 accumulators per lane: two waves per SIMD share its
//     512 registers per lane, so a group's tile is half the slab kernel's);
//   * the workgroup's persistent tiles 0, 1, 2, ... belong to groups 0, 1,
//     0, ...; while one group (the consumer) runs a tile's K loop, reading
//     fragments from LDS and issuing MFMAs only, the other (the producer)
//     issues every global->LDS copy of the ring (whole 128-byte lines, the
//     slab kernel's row swizzle) and, between those copies and the shared
//     barriers, writes the epilogue of its own previous tile, one row block
//     of its accumulators per super-step; when the consumer's tile ends the
//     groups swap roles;
//   * an LDS ring of 3 stages of one 64-k super-step (A 256 rows + weight 128
//     rows of 128 bytes = 48 KiB); barrier B(s+1) sits inside super-step s,
//     after the consumer's first two MFMA rows of its second k-step (by then
//     every fragment of stage s is in its registers), and hands stage s+1 to
//     the consumer and stage s-1 back to the producer, which copies super-step
//     s+2 into it.  Both groups pass the same barriers: one before the loop
//     and one per super-step.
// Each wave waits before a barrier for every copy it issued for a stage the
// barrier publishes: the producer leaves only the copies of s+2 in flight
// (vmcnt(12): twelve loads younger than the last copy of s+1, so the count
// is safe whatever order stores retire in), and a consumer drains all of its
// memory operations (at a role swap it still owns the copies of s+1 it
// issued as the producer).  Selected by the configuration override
// (PIPE=5 with BN=128); measured against the cooperative slab kernel.
#pragma once

#include "gemm_nt_slab.hpp"

namespace mmk {

constexpr int kPpStages = 3;

// f(integral_constant<int, C>) for C = I .. N-1, in order.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__global__ void __launch_bounds__(512) gemm_pp(GemmParams p) {
  constexpr int BM = 256, BN = 128;   // tile: activation rows, weight rows (output columns)
  constexpr int WTM = 128, WTN = 64;  // a wave's block of its group's tile
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int PAIRS = FN / 2;
  constexpr int A_BYTES = BM * kSlabRowB;
  constexpr int STAGE = A_BYTES + BN * kSlabRowB;  // 48 KiB
  constexpr int CA = BM / 8 / 4, CB = BN / 8 / 4;  // copies per producer wave per super-step
  constexpr int CPP = CA + CB;
  constexpr int kRsrcWord3 = 0x00020000;
  __shared__ __attribute__((aligned(1024))) char smem[kPpStages * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // group 0: waves 0..3, group 1: waves 4..7
  const int gw = wave & 3;    // wave within its group
  const int G = gridDim.x;
  const int wg = __builtin_amdgcn_readfirstlane(remap_workgroup(blockIdx.x, G, p.xcd_remap));
  if (wg >= p.num_tiles) return;
  const int my_tiles = __builtin_amdgcn_readfirstlane((p.num_tiles - wg + G - 1) / G);
  const int KS = p.k_tiles;  // super-steps of 64 per tile (>= 2)
  const int S = my_tiles * KS;
  const int M = p.M, N = p.N, K = p.K;
  const uint32_t row_bytes = (uint32_t)K * 2u;

  // ---- producer role: copies of one super-step (as gemm_ws's producers).
  // Lane L of copy j fills stage row 8j + L/8, physical chunk L%8, from
  // logical chunk (L%8) ^ lds_swz(row); j = 4c + gw, so bit 4 of the row is
  // bit 1 of gw.
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ lds_swz(crow + 8 * (gw & 2));
  const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
  // Super-steps past the last one (s >= S) are issued with records of 0
  // bytes: nothing is fetched, zeros land in a stage no wave reads again, and
  // every producer step issues the same twelve copies (with a conditional
  // issue the compiler would wait for all of them before the epilogue's first
  // use of the bias, the youngest loads on the other path).
  auto issue = [&](int s) __attribute__((always_inline)) {
    const bool real = s < S;
    const int ti = real ? __builtin_amdgcn_readfirstlane(s / KS) : 0;
    const int ks = real ? s - ti * KS : 0;
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
    const int stage = s % kPpStages;
    // (readfirstlane returns a signed int: each half goes through uint32_t so
    // that the low word is not sign-extended into the high one)
    const uint32_t a_lo = __builtin_amdgcn_readfirstlane((uint32_t)abase);
    const uint32_t a_hi = __builtin_amdgcn_readfirstlane((uint32_t)(abase >> 32));
    const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)bbase);
    const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(bbase >> 32));
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)a_hi << 32) | a_lo), (short)0,
        (int)__builtin_amdgcn_readfirstlane(real ? mrows * row_bytes - kbytes : 0u), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)b_hi << 32) | b_lo), (short)0,
        (int)__builtin_amdgcn_readfirstlane(real ? nrows * row_bytes - kbytes : 0u), kRsrcWord3);
#pragma unroll
    for (int c = 0; c < CA; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(smem + stage * STAGE + (4 * c + gw) * 1024), 16,
          lane_base + (uint32_t)(8 * (4 * c + gw)) * row_bytes, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < CB; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(smem + stage * STAGE + A_BYTES + (4 * c + gw) * 1024),
          16, lane_base + (uint32_t)(8 * (4 * c + gw)) * row_bytes, 0, 0, 0);
  };

  // ---- consumer role: fragments and MFMAs (as gemm_ws's consumers):
  // activation rows wrow_a + 16 fm + lx; the comb of weight rows wrow_b +
  // 32 (fn >> 1) + 8 (lx >> 2) + 4 (fn & 1) + (lx & 3), so that a lane owns
  // 8 consecutive output columns of a fragment pair
  const int wave_m = gw & 1, wave_n = gw >> 1;
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
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
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto stage_base = [](int s) __attribute__((always_inline)) {
    return (uint32_t)((s % kPpStages) * STAGE);
  };
  auto read_half0 = [&](int s) __attribute__((always_inline)) {
    const uint32_t st = stage_base(s);
#pragma unroll
    for (int f = 0; f < FM; ++f) read_a(f, 0, st + a_x0);
#pragma unroll
    for (int f = 0; f < FN; ++f) read_b(0, f, 0, st + b_x0);
  };

  // ---- epilogue of the group's previous tile, row blocks [r0, r1) of the
  // accumulators: bias, GELU, one rounding, 16-byte stores of 8 consecutive
  // columns per lane (non-temporal: output lines are written once, never read
  // back); tiles on the edges of the output take a masked path.
  const bool has_bias = (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU);
  const bool act_on = (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU);
  const bool bias_vec = (reinterpret_cast<uintptr_t>(p.bias) & 15) == 0;
  u32x4 bw[PAIRS];  // the pending tile's bias vectors (interior tiles)
  int pend = -1;     // the group's tile whose epilogue is pending, -1: none
  int pm0 = 0, pn0 = 0;
  bool pfast = false;  // pending tile lies inside the output, rows 16-byte aligned
  auto begin_epilogue = [&](int ti) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(wg + ti * G, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    pend = ti;
    pm0 = __builtin_amdgcn_readfirstlane(tm * BM);
    pn0 = __builtin_amdgcn_readfirstlane(tn * BN);
    pfast = p.out_vec && pm0 + BM <= M && pn0 + BN <= N;
    if (pfast && has_bias && bias_vec) {
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr)
        bw[pr] = *reinterpret_cast<const u32x4*>(p.bias + pn0 + wrow_b + 32 * pr + 8 * lk);
    }
  };
  // (row blocks [R0, R1) as compile-time constants: with a run-time range the
  // compiler evaluated all eight blocks at once and spilled)
  auto epilogue_rows = [&](auto r0c, auto r1c) __attribute__((always_inline)) {
    constexpr int r0 = decltype(r0c)::value, r1 = decltype(r1c)::value;
    float bv[PAIRS][8];
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int n = pn0 + wrow_b + 32 * pr + 8 * lk;
      if (pfast && has_bias && bias_vec) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[pr][2 * j] = __builtin_bit_cast(float, bw[pr][j] << 16);
          bv[pr][2 * j + 1] = __builtin_bit_cast(float, bw[pr][j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          bv[pr][j] = (has_bias && n + j < N) ? __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16) : 0.f;
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm < r0 || fm >= r1) continue;
      const int m = pm0 + wrow_a + lx + 16 * fm;
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        const int n = pn0 + wrow_b + 32 * pr + 8 * lk;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = acc[fm][2 * pr + (j >> 2)][j & 3] + bv[pr][j];
        if (act_on) gelu_tanh8(v);
        if (pfast) {
          if (p.out_f32) {
            float* o = reinterpret_cast<float*>(p.out) + (int64_t)m * N + n;
            __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(o));
            __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(o) + 1);
          } else {
            u32x4 w;
            w[0] = pack_bf16x2(v[0], v[1]);
            w[1] = pack_bf16x2(v[2], v[3]);
            w[2] = pack_bf16x2(v[4], v[5]);
            w[3] = pack_bf16x2(v[6], v[7]);
            __builtin_nontemporal_store(
                w, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)m * N + n));
          }
        } else if (m < M) {
          store_row8(p.out, p.out_f32, p.out_vec, m, N, n, v);
        }
      }
    }
  };
  // The epilogue runs one row block per super-step of the other group's tile
  // when that tile has at least FM super-steps, else all of it in the first
  // one (a tile runs KS >= 2 super-steps).
  using I0 = std::integral_constant<int, 0>;
  using IFM = std::integral_constant<int, FM>;

  // ---- prologue: group 1 (the producer of tile 0) copies super-steps 0 and
  // 1; group 0 reads the first fragments after B(0)
  if (grp == 1) {
    issue(0);
    issue(1);  // (S >= KS >= 2)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPP));  // super-step 0 landed
  }
  __builtin_amdgcn_s_barrier();  // B(0)
  if (grp == 0) read_half0(0);

  // Tiles in order; within a tile both groups step through its KS
  // super-steps, one in each role (separate loops, so that the fragments are
  // dead while a group produces and its epilogue can use their registers).
  for (int ti = 0; ti < my_tiles; ++ti) {
    const int s0 = ti * KS;
    if ((ti & 1) == grp) {
      // ------------------------------------------------------ consumer
      // (zeroed here, not at the role swap: zeroed in the producer branch,
      // the accumulators met the pending tile's at the loop merge and the
      // compiler kept both sets, spilling 274 registers)
      zero_acc();
      for (int ks = 0; ks < KS; ++ks) {
        const int s = s0 + ks;
        const bool more = ks + 1 < KS;  // the next super-step is this tile's too
        const uint32_t st = stage_base(s), nst = stage_base(s + 1);
        // k-step 2s: half 0 in registers; half 1 of stage s into fa and fb[1]
#pragma unroll
        for (int r = 0; r < FM; ++r) {
          mfma_row(r, 0);
          read_a(r, 1, st + a_x0);
          if (r < FN) read_b(1, r, 1, st + b_x0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // k-step 2s+1: rows 0 and 1, then the barrier; the first super-step
        // after a role swap still owns copies of stage s+1 (issued as the
        // producer)
        mfma_row(0, 1);
        mfma_row(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();  // B(s+1)
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          read_a(0, 0, nst + a_x0);
          read_a(1, 0, nst + a_x0);
        }
#pragma unroll
        for (int r = 2; r < FM; ++r) {
          mfma_row(r, 1);
          if (more) {
            read_a(r, 0, nst + a_x0);
            if (r - 2 < FN) read_b(0, r - 2, 0, nst + b_x0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the tile is done: its epilogue runs during the other group's next
      // tile (or after the loop, for the workgroup's last tile)
      begin_epilogue(ti);
    } else {
      // ------------------------------------------------------ producer
      // copies of s+1 landed; only those of s+2 may stay in flight
      auto produce = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPP));
        __builtin_amdgcn_s_barrier();  // B(s+1)
      };
      int ks = 0;
      static_for<0, FM>([&](auto c) __attribute__((always_inline)) {
        constexpr int C = decltype(c)::value;
        if (ks < KS) {
          issue(s0 + ks + 2);
          if (pend >= 0) {
            if (KS >= FM)
              epilogue_rows(c, std::integral_constant<int, C + 1>{});
            else if (C == 0)
              epilogue_rows(I0{}, IFM{});
          }
          produce();
          ++ks;
        }
      });
      for (; ks < KS; ++ks) {
        issue(s0 + ks + 2);
        produce();
      }
      pend = -1;
      // role swap: the next tile is this group's.  (Read unconditionally:
      // after the workgroup's last tile the stage holds stale data that no
      // MFMA uses; with the read under a condition the fragments stayed live
      // through the producer loop and its epilogue spilled.)
      read_half0(s0 + KS);
    }
  }
  // the workgroup's last tile: its consumer writes it without overlap; no
  // wave leaves with copies in flight
  if (pend >= 0) epilogue_rows(I0{}, IFM{});
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

}  // namespace mmk
