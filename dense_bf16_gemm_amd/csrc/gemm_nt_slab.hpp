// gemm_nt_slab.hpp -- K-contiguous ("NT") GEMM whose global->LDS copies move
// whole 128-byte lines.
//
// Same schedule, MFMA loop and epilogue as gemm_nt_pipe, with the LDS ring
// reorganised so that each copy instruction reads 8 rows x 128 bytes (64 k)
// instead of 16 rows x 64 bytes: a line then travels from L2 once instead of
// twice, which halves the requests the vector L1 has to keep in flight (its
// pending-request stalls were the main cost of the copies).
//   * The ring is 5 units of 32 KiB.  A unit holds one operand's 256 rows of
//     one 64-k "super-step" (rows of 128 bytes, XOR-swizzled as lds_swz);
//     the A and the weight slab of super-step S take consecutive units.
//   * The MFMA loop still runs k-steps of 32 (two per super-step), with the
//     operand fragments read one k-step ahead into a second register set.
//   * The slabs of super-step S are last read during k-step 2S (which reads
//     the fragments of k-step 2S+1), so after the barrier at the top of
//     k-step 2S+1 both units are free.  The copies of super-step S+2 go out
//     as: A slab during k-step 2S, weight slab during k-step 2S+1.  Each
//     slab has 2 to 3 k-steps to land; one barrier per super-step publishes
//     the next super-step's slabs and frees the previous one's.
#pragma once

#include "gemm_nt_pipe.hpp"

namespace mmk {

constexpr int kSlabK = 64;       // k per super-step
constexpr int kSlabRowB = 128;   // LDS bytes per row of a unit
constexpr int kSlabUnits = 5;

template <int BM, int BN, int WGM, int WGN, bool FFN>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_nt_slab(GemmParams p) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int OUT_BN = FFN ? BN / 2 : BN;
  constexpr int UNIT = 256 * kSlabRowB;  // 32 KiB
  static_assert(BM == 256 && BN == 256, "a unit holds 256 rows");
  constexpr int CPS = 256 / 8 / NW;  // 1 KiB copies per wave per slab
  static_assert(CPS * NW * 8 == 256, "copy split");
  static_assert(FN % 2 == 0 && (!FFN || FN % 4 == 0), "fragment pairs");
  static_assert(WTN % 32 == 0 && WTM % 32 == 0, "wave tile");

  __shared__ __attribute__((aligned(1024))) char smem[kSlabUnits * UNIT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / WGN;
  const int wave_n = wave % WGN;
  const int G = gridDim.x;
  const int wg = remap_workgroup(blockIdx.x, G, p.xcd_remap);
  if (wg >= p.num_tiles) return;
  const int my_tiles = (p.num_tiles - wg + G - 1) / G;
  const int KS = p.k_tiles;  // super-steps of 64 per tile
  const int M = p.M, N = p.N, K = p.K;
  const int64_t ld = K;

  // ---- copies: lane L of a 1 KiB copy fills unit row 8j + L/8, physical
  // chunk L%8, from logical chunk (L%8) ^ lds_swz(row).  Bits 0..2 of that
  // row are L/8 and bit 4 is bit 1 of j; a wave's copies j = i*NW + wave
  // all share bit 1 of j when NW is a multiple of 4, so the chunk is fixed.
  static_assert(NW % 4 == 0, "copy chunk constant per wave");
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ lds_swz(crow + 8 * (wave & ~1));
  const uint32_t row_bytes = (uint32_t)ld * 2u;
  const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
  constexpr int kRsrcWord3 = 0x00020000;

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
  auto koff_of = [&](int ks) __attribute__((always_inline)) {
    const int k0 = (ld_alt ? (KS - 1 - ks) : ks) * kSlabK;
    return lane_base + 2u * (uint32_t)k0 + ((k0 + 8 * cchunk) < K ? 0u : 0x80000000u);
  };
  // copy c (0..CPS-1) of this wave for the A slab / the weight slab
  auto copy_a = [&](int c, uint32_t koff, int unit) __attribute__((always_inline)) {
    const int j = c * NW + wave;
    // (typed explicitly: deducing the builtin's type leaves the host stub uninstantiated)
    const __amdgpu_buffer_rsrc_t r = rsrc(a_base, a_rec);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + j * 1024),
        16, koff + (uint32_t)(8 * j) * row_bytes, 0, 0, 0);
  };
  auto copy_b = [&](int c, uint32_t koff, int unit) __attribute__((always_inline)) {
    const int j = c * NW + wave;
    const int r0 = 8 * j;
    int prow = r0;
    bool up = false;
    if constexpr (FFN) {
      // each wave column's WTN weight rows: WTN/2 gate rows, then the up rows
      const int wb = r0 / WTN, within = r0 % WTN;
      up = within >= WTN / 2;
      prow = wb * (WTN / 2) + (up ? within - WTN / 2 : within);
    }
    const __amdgpu_buffer_rsrc_t r = rsrc(up ? b1_base : b0_base, b_rec);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r,
        (__attribute__((address_space(3))) void*)(smem + unit * UNIT + j * 1024), 16,
        koff + (uint32_t)prow * row_bytes, 0, 0, 0);
  };

  // ---- load cursor: super-step (ld_tile, ld_ks) whose slabs are copied next
  int ld_tile = 0, ld_ks = 0, ld_unit = 0;  // ld_unit: unit of its A slab
  enter_tile(0);
  auto advance_cursor = [&]() __attribute__((always_inline)) {
    ld_unit = (ld_unit + 2) % kSlabUnits;
    if (ld_tile < my_tiles) {
      if (++ld_ks == KS) {
        ld_ks = 0;
        ++ld_tile;
        if (ld_tile < my_tiles) enter_tile(ld_tile);
        else ld_ks = KS - 1;  // past the end: re-copy the last super-step (never read)
      }
    }
  };
  auto next_unit = [](int u) { return u + 1 == kSlabUnits ? 0 : u + 1; };

  // ---- fragments: 128-byte rows, k-step half h uses chunks 4h..4h+3
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
  // Swizzled chunk of k-step half h: (4h + lk) ^ lds_swz(row).  For A rows
  // wrow_a + 16q + lx, lds_swz = (lx & 7) ^ 4q; for the comb rows of the
  // weight fragments wrow_b + 8(lx>>2) + 4q + (lx&3), lds_swz = (lx & 3) ^
  // 4(q ^ bit 3 of lx).  Either way the chunk is a lane constant XOR 4(h^q),
  // so two offsets per operand cover every (h, q).
  const uint32_t a_x0 = (uint32_t)((wrow_a + lx) * kSlabRowB + ((lk ^ (lx & 7)) << 4));
  const uint32_t b_x0 = (uint32_t)((wrow_b + 8 * (lx >> 2) + (lx & 3)) * kSlabRowB +
                                   ((lk ^ (lx & 3) ^ (((lx >> 3) & 1) << 2)) << 4));

  bf16x8 fa[2][FM], fb[2][FN];
  f32x4 acc[FM][FN];

  // fragments of k-step half h from the slabs in units ua (A) and ub (weight)
  auto read_frag = [&](int f, int h, int ua, int ub, bf16x8* a, bf16x8* b)
      __attribute__((always_inline)) {
    if (f < FN) {
      const char* base = smem + ub * UNIT;
      const int q = f & 1;
      const uint32_t off = ((h ^ q) ? (b_x0 ^ 64u) : b_x0) + (uint32_t)((4 * q + 32 * (f >> 1)) * kSlabRowB);
      b[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
    } else {
      const int fm = f - FN;
      const char* base = smem + ua * UNIT;
      const int q = fm & 1;
      const uint32_t off = ((h ^ q) ? (a_x0 ^ 64u) : a_x0) + (uint32_t)(16 * fm * kSlabRowB);
      a[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
    }
  };

  // ---- prologue: slabs of super-steps 0 and 1 in flight; fragments of
  // k-step 0 in register set 0.  (Each wave: CPS copies per slab.)
  {
    for (int s = 0; s < 2; ++s) {
      const uint32_t koff = koff_of(ld_ks);
      const int ua = ld_unit, ub = next_unit(ld_unit);
#pragma unroll
      for (int c = 0; c < CPS; ++c) copy_a(c, koff, ua);
#pragma unroll
      for (int c = 0; c < CPS; ++c) copy_b(c, koff, ub);
      advance_cursor();
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * CPS));
  __builtin_amdgcn_s_barrier();
  int cur_unit = 0;  // unit of the A slab of the current super-step
#pragma unroll
  for (int f = 0; f < FM + FN; ++f) read_frag(f, 0, 0, 1, fa[0], fb[0]);

  constexpr int NMFMA = FM * FN;
  constexpr int NDS = FM + FN;
  // One k-step: MFMAs on register set P, fragments of the next k-step
  // (half nh of the slabs in units nua/nub) into set P^1, and the CPS copies
  // of one slab (A if copy_is_a) interleaved CPS-way.
  auto kstep = [&](auto par, int nh, int nua, int nub, bool copy_is_a, uint32_t koff, int cunit)
      __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      if (copy_is_a) copy_a(c, koff, cunit);
      else copy_b(c, koff, cunit);
#pragma unroll
      for (int f = (c * NDS) / CPS; f < ((c + 1) * NDS) / CPS; ++f)
        read_frag(f, nh, nua, nub, fa[P ^ 1], fb[P ^ 1]);
#pragma unroll
      for (int i = (c * NMFMA) / CPS; i < ((c + 1) * NMFMA) / CPS; ++i) {
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
    for (int ks = 0; ks < KS; ++ks) {
      // super-step S = this one; its slabs are in units cur_unit, cur_unit+1
      const int ua = cur_unit, ub = next_unit(cur_unit);
      const int nua = next_unit(ub), nub = next_unit(nua);  // super-step S+1
      const uint32_t koff = koff_of(ld_ks);                  // super-step S+2
      const int cua = ld_unit, cub = next_unit(ld_unit);
      // k-step 2S: fragments of 2S+1 (same slabs, half 1); copy A slab of S+2
      kstep(std::integral_constant<int, 0>{}, 1, ua, ub, true, koff, cua);
      // top of k-step 2S+1: own copies of S+1 landed (the A slab of S+2 may
      // still fly); then publish S+1 and free the units of S
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPS));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // k-step 2S+1: fragments of 2S+2 (S+1, half 0); copy weight slab of S+2
      kstep(std::integral_constant<int, 1>{}, 0, nua, nub, false, koff, cub);
      advance_cursor();
      cur_unit = nua;
    }

    // ---- epilogue (as gemm_nt_pipe)
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
