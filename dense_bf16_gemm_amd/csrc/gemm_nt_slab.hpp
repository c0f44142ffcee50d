// gemm_nt_slab.hpp -- GEMM whose global->LDS copies move whole lines, for
// 256 x 256 tiles on four waves.  K-contiguous operands ("NT") are copied as
// rows of 128 bytes (64 k); an operand stored [K][N] or [K][M] (the BKN and
// AMK instances: the NN, TN and TT layouts) as k-rows of 512 bytes, read
// back with the LDS transpose read (see lds_read_tr16 and the BKN/AMK notes
// in the kernel).
//
// Same persistent schedule, tile order and result as gemm_nt_pipe, with
// three changes aimed at keeping one wave per SIMD issuing MFMAs:
//   * Copies.  Each copy instruction reads 8 rows x 128 bytes (64 k) instead
//     of 16 rows x 64 bytes, so every cache line travels from L2 once and the
//     vector L1 keeps half as many requests in flight.  The LDS ring is 5
//     units of 32 KiB; a unit holds one operand's 256 rows of one 64-k
//     "super-step" (XOR-swizzled rows of 128 bytes), and the A and weight
//     slabs of a super-step sit in consecutive units.  The slabs of
//     super-step q+2 are copied during super-step q (A during its first
//     k-step, the weight slab during its second), and one wait + barrier per
//     super-step publishes q+1 and frees q (the write-after-read hazard of
//     issue "Automate performant Hopper matmul", section "Syncing issues";
//     prefetch distance > 1 as its section "K loop efficiency" asks).
//   * Registers.  The MFMAs of a k-step run row by row (8 output-row blocks
//     of 16 x 128); the activation fragment of row r is dead after row r and
//     is refilled at once with the next k-step's fragment, while the weight
//     fragments are double-buffered.  24 live fragments instead of 32 leave
//     the accumulators in place (no AGPR shuffles, no spills).
//   * The K loop of a tile has no tile bookkeeping: the load cursor moves to
//     the next tile once, before the last two super-steps, whose copies fetch
//     that tile's first slabs (so they land while this tile's epilogue runs:
//     section "Syncing persistent matmuls").
// The host uses this kernel only when K is a multiple of the 64-k super-step
// and spans at least two of them (ragged K runs gemm_nt_pipe, or for the
// other layouts gemm_persistent).
#pragma once

#include "gemm_nt_pipe.hpp"

namespace mmk {

constexpr int kSlabK = 64;       // k per super-step
constexpr int kSlabRowB = 128;   // LDS bytes per row of a unit
constexpr int kSlabUnits = 5;

// GELU(tanh) as t / (1 + 2^(t (c1 + c2 t^2))) with c1 = -2 sqrt(2/pi) log2(e)
// and c2 = 0.044715 c1: the same function as 0.5 t (1 + tanh z), rewritten
// so that one exp2 and one reciprocal remain.
__device__ __forceinline__ float gelu_tanh_fast(float t) {
  constexpr float c1 = -2.3022081983f;   // -2 * 0.7978845608 * 1.4426950409
  constexpr float c2 = -0.1029432396f;   // c1 * 0.044715
  const float e = __builtin_amdgcn_exp2f(t * __builtin_fmaf(c2, t * t, c1));
  return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// The same GELU on eight independent values, one operation across all eight
// at a time, so that the exp2 and reciprocal latencies overlap.
__device__ __forceinline__ void gelu_tanh8(float (&v)[8]) {
  constexpr float c1 = -2.3022081983f;
  constexpr float c2 = -0.1029432396f;
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = v[j] * v[j];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = __builtin_fmaf(c2, e[j], c1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = v[j] * e[j];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(e[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = 1.0f + e[j];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_rcpf(e[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * e[j];
}

// The scalar bookkeeping at the head of a k-step (ring units, descriptor
// bases, LDS destinations: a dependent chain of ~25 instructions) would idle
// the matrix core if it ran in front of the first MFMA, since one wave issues
// at most one instruction per four cycles and an MFMA takes sixteen.  These
// scheduling groups spread it, with the row's copy and fragment reads, over
// the three free issue slots after each of the row's eight MFMAs.
// 0x008: MFMA, 0x006: scalar or vector ALU, 0x020: memory read (the copy),
// 0x100: LDS read.
// MPR: MFMAs per row (8 for a 128-column wave block, 6 for 96 columns, 4 for
// 64).
template <int MPR>
__device__ __forceinline__ void spread_first_row_a() {
  if constexpr (MPR == 4) {
    // (four MFMAs for the same scalar chain: it overflows the free slots)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 6, 0);
    }
  } else if constexpr (MPR == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 4, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
    }
  } else {
    static_assert(MPR == 6, "rows of 8, 6 or 4 MFMAs");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 4, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 5, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
}
// Rows of 4 MFMAs leave too few slots for a k-step head in one row.  With
// them the first k-step's head spans rows 0..2 (12 MFMAs: the scalar chain
// over the first eight, then the three copies and six fragment reads) and
// the second k-step's its first two rows (8 MFMAs: the weight descriptors
// over the first three, then three copies and five fragment reads).
__device__ __forceinline__ void spread_first_rows_a4() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x006, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}
__device__ __forceinline__ void spread_rows_b4() {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
}
// Rows of 8 MFMAs: the first k-step's head spans two rows (16 MFMAs).
__device__ __forceinline__ void spread_first_rows_a8() {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}
// Rows of 6 MFMAs: both heads span two rows (12 MFMAs).
__device__ __forceinline__ void spread_first_rows_a6() {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}
__device__ __forceinline__ void spread_rows_b6() {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
  }
}
template <int MPR>
__device__ __forceinline__ void spread_first_row_b() {
  if constexpr (MPR == 4) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 5, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
    return;
  }
  constexpr int lead = MPR == 8 ? 3 : 2;
#pragma unroll
  for (int i = 0; i < lead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x006, 3, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (MPR == 8) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);
}

// Last row of a super-step: 2, 2 and 1 scalar instructions after its first
// three MFMAs, the row's LDS read after the fourth (after the third, with
// three MFMAs per half row).
template <int MPR>
__device__ __forceinline__ void spread_loop_latch() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);
  if constexpr (MPR == 8) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS transpose read of 16-bit elements (gfx950).  Within each group of 16
// lanes, lane 4r + q supplies the address of 4 consecutive elements (row r,
// column block q of a 4 x 16 block) and lane i receives column i of the 4
// rows: element e is row e's element i.  The restrict parameter gives the
// read alias information: without it the compiler treats the intrinsic as
// possibly reading what any direct-to-LDS copy in flight writes and waits
// for all of them (vmcnt 0) before it, as it does not for plain LDS loads;
// the copies and these reads are ordered by the kernel's own waits and
// barriers.
__device__ __forceinline__ s16x4 lds_read_tr16(__attribute__((address_space(3))) char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// SiLU as g / (1 + 2^(-g log2 e)).
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950409f));
}

template <int BM, int BN, int WGM, int WGN, bool FFN, bool SPLITK = false, bool PRE = false,
          bool BKN = false, bool AMK = false, bool BSTAGE = false, bool RAGGED = false>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_nt_slab(GemmParams p) {
  // BKN: the weight operand is stored [K][N] (the MatmulOp form's B as
  // given, N contiguous).  Its slab of a super-step is 64 k-rows of 256
  // columns (512 bytes), copied as stored, and the fragments are read with
  // the LDS transpose read, which hands each lane 4 consecutive k of one
  // column: two of them make the 8 k of an MFMA operand.
  static_assert(!(BKN && (FFN || PRE)), "[K][N] weights in the single-weight form only");
  // AMK: the activation operand is stored [K][M] (M contiguous), handled the
  // same way: 64 k-rows of 256 rows' values per slab, transpose reads.
  static_assert(!(AMK && (FFN || PRE)), "[K][M] activations in the single-weight form only");
  // BSTAGE: the instance whose K loop also brings each tile's bias into LDS
  // (see copy_bias); built for the K-contiguous linear form with bias.
  static_assert(!(BSTAGE && (FFN || SPLITK || PRE || BKN || AMK)), "bias staging: plain linear form only");
  static_assert(!(SPLITK && FFN), "split-K is built for the single-weight forms");
  // RAGGED: K is not a multiple of 64 (it is one of 8, the alignment of
  // K-contiguous rows).  The tile's last super-step is a partial one.  A
  // K-contiguous operand's copies push the lanes whose 16-byte chunk lies past
  // K out of the buffer range, so those chunks arrive as zeros (see
  // tail_bits); an operand stored [K][N] or [K][M] needs nothing: its k-rows
  // past K lie past the end of the matrix, outside the record, and read as
  // zeros too.
  static_assert(!(RAGGED && (PRE || BSTAGE || (FFN && (BKN || AMK)))), "ragged K: single-output forms");
  // PRE: the instance that also stores the pre-activation (p.out_pre).  It is
  // a separate instance because any extra epilogue path in the default one
  // changes the register allocation of its K loop.
  static_assert(!(PRE && (FFN || SPLITK)), "pre-activation output of the linear GELU form only");
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int OUT_BN = FFN ? BN / 2 : BN;
  constexpr int UNIT = 256 * kSlabRowB;  // 32 KiB
  // BN = 192 or 128 (a 128 x 96 or 128 x 64 block per wave): K-contiguous
  // single-weight products whose 256 x 256 tiles would leave much of the grid
  // idle (split or not); the weight slab then fills 3/4 or 1/2 of its unit
  static_assert(BM == 256 &&
                    (BN == 256 || ((BN == 192 || BN == 128) && !BKN && !AMK && !FFN && !PRE && !BSTAGE)) &&
                    NW == 4,
                "a unit holds 256 rows; four waves");
  static_assert(FM == 8 && (FN == 8 || FN == 6 || FN == 4), "row schedule assumes 8 x 8, 8 x 6 or 8 x 4 fragments per wave");
  constexpr int CPS = BM / 8 / NW;     // 1 KiB activation copies per wave per slab
  constexpr int CPS_B = BN / 8 / NW;   // weight copies (as many, or 6 / 4 for BN = 192 / 128)
  static_assert(CPS == FM, "one activation copy per MFMA row");

  __shared__ __attribute__((aligned(1024))) char smem[kSlabUnits * UNIT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / WGN;
  const int wave_n = wave % WGN;
  const int G = gridDim.x;
  // (integer division runs on the vector unit; readfirstlane hands the
  // wave-uniform results back to scalar registers, so that all descriptor
  // and offset arithmetic below stays scalar)
  const int wg = __builtin_amdgcn_readfirstlane(remap_workgroup(blockIdx.x, G, p.xcd_remap));
  const int KS = p.k_tiles;  // super-steps of 64 per tile (>= 2; the last partial when RAGGED)
  // work units: tiles (of every batch entry), or (stream-K) the one or two
  // pieces of this workgroup's chunk range [ci0, ci1)
  // (sk_items == 0: chunk-major split-K, workgroup c runs chunk c / tiles of
  // tile c % tiles, one unit)
  const int SKN = SPLITK ? p.sk_chunks : 1;
  const bool sk_cmaj = SPLITK && p.sk_items == 0;
  const int ci0 = SPLITK ? (sk_cmaj ? wg : wg * p.sk_items) : 0;
  const int ci1 = SPLITK ? (sk_cmaj ? wg + 1 : min(ci0 + p.sk_items, p.num_tiles * SKN)) : 0;
  const int units = SPLITK ? 0 : p.num_tiles * p.batch;
  if (SPLITK ? ci1 > p.num_tiles * SKN || ci0 >= ci1 : wg >= units) return;
  const int my_tiles = __builtin_amdgcn_readfirstlane(
      SPLITK ? (sk_cmaj ? 1 : (ci1 - 1) / SKN - ci0 / SKN + 1) : (units - wg + G - 1) / G);
  const int M = p.M, N = p.N, K = p.K;
  const int64_t ld = K;

  // ---- copies: lane L of a 1 KiB copy fills unit row 8j + L/8, physical
  // chunk L%8, from logical chunk (L%8) ^ lds_swz(row).  Bits 0..2 of that
  // row are L/8 and bit 4 is bit 1 of j = 4c + wave, i.e. bit 1 of the wave,
  // so the logical chunk of a lane is the same for all its copies.
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ lds_swz(crow + 8 * (wave & 2));
  const uint32_t row_bytes = (uint32_t)ld * 2u;
  const uint32_t lane_base = (uint32_t)crow * row_bytes + 16u * (uint32_t)cchunk;
  // RAGGED: the copies of a tile's partial last super-step OR tail_bits into
  // their lane offsets; it is lane_oob there (bit 31 for a lane whose chunk,
  // 8 cchunk values of k past the super-step's first, lies past K: the offset
  // then exceeds the record, below 2^31, and the chunk reads as zeros) and 0
  // in every other super-step
  const uint32_t lane_oob = RAGGED && 8 * cchunk >= (K & 63) ? 0x80000000u : 0u;
  uint32_t tail_bits = 0u;
  constexpr int kRsrcWord3 = 0x00020000;
  // [K][N] weight slab: copy c of this wave fills unit rows 2j, 2j + 1 (k),
  // j = 4c + wave, 512 bytes each; lane L fills row 2j + L/32, physical
  // 16-byte chunk L%32, from logical chunk (L%32) ^ (4 (row & 3)).  Row & 3
  // is 2 (wave & 1) + L/32 for every copy, so the logical chunk is a lane
  // constant.
  const uint32_t rowb_kn = (uint32_t)N * 2u;
  const int kn_row = lane >> 5;
  const int kn_chunk = (lane & 31) ^ (((2 * (wave & 1) + kn_row) & 3) << 2);
  const uint32_t lane_kn = (uint32_t)kn_row * rowb_kn + 16u * (uint32_t)kn_chunk;
  // [K][M] activation slab: the same copy pattern with rows of M values;
  // lane L fetches logical chunk (L%32) ^ 2 s(row), s(row) = (row & 3) |
  // 4 (bit 3 of row).  Bit 3 of row 2j + L/32 is bit 0 of the copy index c
  // (j = 4c + wave), so there are two lane constants, for even and odd c.
  const uint32_t rowb_km = (uint32_t)M * 2u;
  const int km_s_lo = (2 * (wave & 1) + kn_row) & 3;
  const uint32_t lane_km0 = (uint32_t)kn_row * rowb_km + 16u * (uint32_t)((lane & 31) ^ (2 * km_s_lo));
  const uint32_t lane_km1 = (uint32_t)kn_row * rowb_km + 16u * (uint32_t)((lane & 31) ^ (2 * (km_s_lo | 4)));

  // Descriptors of the tile the copies currently fetch (cur) and of the
  // workgroup's next tile (nxt; the current one again after the last tile,
  // whose re-fetched slabs are never read).
  struct TileDesc {
    uint64_t a_base, b0_base, b1_base;
    uint32_t a_rec, b_rec;
    uint64_t b_rem;  // [K][N] weights: bytes from b0_base to the end of B
    uint64_t a_rem;  // [K][M] activations: bytes from a_base to the end of A
    int alt;
    int kbeg;  // first super-step of a split-K slice (0 otherwise)
  };
  // output tile, batch entry, and first and count of super-steps of this
  // workgroup's unit i
  auto unit_of = [&](int i, int* tile, int* slice, int* kbeg, int* nks) __attribute__((always_inline)) {
    const int u = wg + i * G;
    *tile = u;
    *slice = 0;
    *kbeg = 0;
    *nks = KS;
    if constexpr (SPLITK) {
      // piece i: the chunks of [ci0, ci1) that fall in one tile
      int t, a;
      if (sk_cmaj) {
        a = __builtin_amdgcn_readfirstlane(wg / p.num_tiles);
        t = wg - a * p.num_tiles;
      } else {
        t = __builtin_amdgcn_readfirstlane(ci0 / SKN + i);
        a = (i == 0 ? ci0 : t * SKN) - t * SKN;
      }
      const int b = sk_cmaj ? a + 1 : min(ci1, (t + 1) * SKN) - t * SKN;
      *tile = t;
      *kbeg = __builtin_amdgcn_readfirstlane(a * KS / SKN);
      *nks = __builtin_amdgcn_readfirstlane(b * KS / SKN) - *kbeg;
    } else {
      if (p.batch > 1) {  // slice = batch entry
        *slice = __builtin_amdgcn_readfirstlane(u / p.num_tiles);
        *tile = u - *slice * p.num_tiles;
      }
    }
  };
  auto tile_desc = [&](int tile_i) __attribute__((always_inline)) {
    int tm, tn;
    int tile, slice, kbeg, nks;
    unit_of(tile_i, &tile, &slice, &kbeg, &nks);
    tile_coords(tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    tm = __builtin_amdgcn_readfirstlane(tm);
    tn = __builtin_amdgcn_readfirstlane(tn);
    const int m0 = tm * BM;
    const int mrows = (M - m0) < BM ? (M - m0) : BM;
    const int n0 = tn * OUT_BN;
    const int nrows = (N - n0) < OUT_BN ? (N - n0) : OUT_BN;
    TileDesc d;
    // batch entry (never with split-K): operand bases move by the strides
    const int64_t ea = SPLITK ? 0 : (int64_t)slice * p.stride_a;
    const int64_t eb = SPLITK ? 0 : (int64_t)slice * p.stride_b;
    d.a_base = reinterpret_cast<uint64_t>(p.A + ea + (AMK ? (int64_t)m0 : (int64_t)m0 * ld));
    d.a_rem = AMK ? ((uint64_t)K * (uint64_t)M - (uint64_t)m0) * 2u : 0;
    d.a_rec = (uint32_t)mrows * row_bytes;
    d.b_rec = (uint32_t)nrows * row_bytes;
    d.b0_base = reinterpret_cast<uint64_t>(p.B + eb + (BKN ? (int64_t)n0 : (int64_t)n0 * ld));
    d.b1_base = FFN ? reinterpret_cast<uint64_t>(p.B2 + eb + (int64_t)n0 * ld) : d.b0_base;
    // columns past N read the next row's values (or zeros past the end of
    // B): they only reach output columns past N, which are never stored
    d.b_rem = BKN ? ((uint64_t)K * (uint64_t)N - (uint64_t)n0) * 2u : 0;
    d.alt = SPLITK ? 0 : (p.k_alt && (tile_i & 1));
    d.kbeg = kbeg;
    return d;
  };
  TileDesc cur = tile_desc(0);
  // Buffer descriptors are rebuilt from wave-uniform values at each use so
  // that they stay in scalar registers.
  auto rsrc = [&](uint64_t base, uint32_t rec) __attribute__((always_inline)) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    void* ptr = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, (int)__builtin_amdgcn_readfirstlane(rec),
                                             kRsrcWord3);
  };
  // Copy c of this wave fills unit rows 8j .. 8j+7, j = 4c + wave.  Each
  // lane's vector offset is a constant (voff_*: its row and chunk); the k
  // position of the super-step moves the descriptor's base instead, with the
  // record count shrunk by the same amount, so rows past the tile's last row
  // still fail the range check and read as zeros.  No vector instruction is
  // spent on addressing in the K loop.
  // weight row of copy c's first row, and whether it is an up-weight row
  auto wrow_of = [&](int c, bool* up) __attribute__((always_inline)) -> int {
    const int r0 = 8 * (c * NW + wave);
    *up = false;
    if constexpr (FFN) {
      // each wave column's WTN weight rows: WTN/2 gate rows, then the up rows.
      // The NW waves' rows of copy c lie in one half of a wave column, so
      // the half (and with it the operand) follows from c alone.
      static_assert((WTN / 2) % (8 * NW) == 0, "a copy's rows stay in one half");
      const int c0 = 8 * c * NW;  // first row of copy c over all waves
      *up = (c0 % WTN) >= WTN / 2;
      return (c0 / WTN) * (WTN / 2) + (c0 % WTN) - (*up ? WTN / 2 : 0) + 8 * wave;
    }
    return r0;
  };
  // first k of super-step ks of the fetched tile
  auto k0_of = [&](int ks) __attribute__((always_inline)) {
    if constexpr (SPLITK) return (cur.kbeg + ks) * kSlabK;
    const int alt = __builtin_amdgcn_readfirstlane(cur.alt);
    return (alt ? (KS - 1 - ks) : ks) * kSlabK;
  };
  // Copy c of this wave for the A slab / the weight slab of the super-step at
  // k byte offset kbytes into unit `unit`.
  // (The lane offsets are loop-invariant and stay in registers.  They are
  // written out inline: passing them through a helper or an array leaves the
  // host stub of the kernel uninstantiated, as does deducing the descriptor
  // type.)
  auto copy_a = [&](int c, uint32_t kbytes, int unit) __attribute__((always_inline)) {
    if constexpr (AMK) {
      // rows past M read the next k-row's values (or zeros past the end of
      // A): they only reach output rows past M, which are never stored
      const uint64_t kb = (uint64_t)(kbytes >> 1) * rowb_km;
      const uint64_t rem = cur.a_rem - kb;
      const uint32_t rec = rem > 0xffffffffull ? 0xffffffffu : (uint32_t)rem;
      const __amdgpu_buffer_rsrc_t r = rsrc(cur.a_base + kb, rec);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + (c * NW + wave) * 1024), 16,
          ((c & 1) ? lane_km1 : lane_km0) + (uint32_t)(2 * (c * NW + wave)) * rowb_km, 0, 0, 0);
      return;
    }
    const __amdgpu_buffer_rsrc_t r = rsrc(cur.a_base + kbytes, cur.a_rec - kbytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + (c * NW + wave) * 1024), 16,
        (lane_base + (uint32_t)(8 * (c * NW + wave)) * row_bytes) | tail_bits, 0, 0, 0);
  };
  auto copy_b = [&](int c, uint32_t kbytes, int unit) __attribute__((always_inline)) {
    if constexpr (BKN) {
      // the super-step's k rows: the base moves by k0 rows of N columns
      const uint64_t kb = (uint64_t)(kbytes >> 1) * rowb_kn;
      const uint64_t rem = cur.b_rem - kb;
      const uint32_t rec = rem > 0xffffffffull ? 0xffffffffu : (uint32_t)rem;
      const __amdgpu_buffer_rsrc_t r = rsrc(cur.b0_base + kb, rec);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + (c * NW + wave) * 1024), 16,
          lane_kn + (uint32_t)(2 * (c * NW + wave)) * rowb_kn, 0, 0, 0);
      return;
    }
    bool up;
    const int prow = wrow_of(c, &up);
    const __amdgpu_buffer_rsrc_t r = rsrc((up ? cur.b1_base : cur.b0_base) + kbytes, cur.b_rec - kbytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + (c * NW + wave) * 1024), 16,
        (lane_base + (uint32_t)prow * row_bytes) | tail_bits, 0, 0, 0);
  };
  auto next_unit = [](int u) __attribute__((always_inline)) {
    return u + 1 == kSlabUnits ? 0 : u + 1;
  };

  // ---- fragments: 128-byte rows; k-step half h uses logical chunks 4h..4h+3.
  // For A rows wrow_a + 16 fm + lx the swizzle is (lx & 7) ^ 4 (fm & 1); for
  // the comb rows of the weight fragments wrow_b + 32 (fn >> 1) + 8 (lx >> 2)
  // + 4 (fn & 1) + (lx & 3) it is (lx & 3) ^ 4 ((fn & 1) ^ bit 3 of lx).
  // Either way the chunk is a lane constant XOR 4 (h ^ (f & 1)), which flips
  // bit 6 of the byte offset.
  const int lx = lane & 15;
  const int lk = lane >> 4;
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;
  const uint32_t a_x0 = AMK
      // [K][M] slab: lane (lk, lx) of a transpose read supplies k-row
      // 8 lk + 4 hk + lx / 4 (+ 32 h) and rows wrow_a + 16 fm + 4 (lx & 3) ..
      // + 3: 16-byte chunk 16 wave_m + 2 fm + (lx & 3) / 2, half (lx & 1), at
      // chunk ^ 2 s, s = (lx >> 2) | 4 (lk & 1): bits 5..7 of the offset hold
      // fm ^ s, so this is the offset for fm = 0 and the others XOR 32 fm in
      ? (uint32_t)((8 * lk + (lx >> 2)) * 512 + 256 * wave_m + 16 * ((lx & 3) >> 1) + 8 * (lx & 1) +
                   32 * ((lx >> 2) | ((lk & 1) << 2)))
      : (uint32_t)((wrow_a + lx) * kSlabRowB + ((lk ^ (lx & 7)) << 4));
  const uint32_t b_x0 = BKN
      // [K][N] slab: lane (lk, lx) of a transpose read supplies k-row
      // 8 lk + 4 hk + lx / 4 (+ 32 h) and the 4 columns from wrow_b +
      // 8 (lx & 3) + 4 (fn & 1) + 32 (fn >> 1) (the comb); their 16-byte chunk
      // 16 wave_n + (lx & 3) + 4 (fn >> 1) sits at chunk ^ 4 (row & 3), i.e.
      // bits 6..7 of the offset hold (fn >> 1) ^ (lx >> 2): this is the offset
      // for fn >> 1 = 0, the others XOR 64 (fn >> 1) into it.
      ? (uint32_t)((8 * lk + (lx >> 2)) * 512 + 256 * wave_n + 16 * (lx & 3) + 64 * (lx >> 2))
      : (uint32_t)((wrow_b + 8 * (lx >> 2) + (lx & 3)) * kSlabRowB +
                   ((lk ^ (lx & 3) ^ (((lx >> 3) & 1) << 2)) << 4));

  bf16x8 fa[FM];     // activation fragments, refilled row by row
  bf16x8 fb[2][FN];  // weight fragments, double-buffered
  f32x4 acc[FM][FN];

  auto read_a = [&](int fm, int h, uint32_t ubase) __attribute__((always_inline)) {
    if constexpr (AMK) {
      typedef __attribute__((address_space(3))) char lds_char;
      const uint32_t off = (ubase ^ (uint32_t)(32 * fm)) + (uint32_t)(32 * h * 512);
      const s16x4 lo = lds_read_tr16((lds_char*)smem + off);
      const s16x4 hi = lds_read_tr16((lds_char*)smem + off + 4 * 512);
      fa[fm] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      return;
    }
    const uint32_t off = (((h ^ fm) & 1) ? (ubase ^ 64u) : ubase) + (uint32_t)(16 * fm * kSlabRowB);
    fa[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + off));
  };
  auto read_b = [&](int set, int fn, int h, uint32_t ubase) __attribute__((always_inline)) {
    if constexpr (BKN) {
      // two transpose reads: k 8 lk + 0..3 and 8 lk + 4..7 of the lane's column
      typedef __attribute__((address_space(3))) char lds_char;
      const uint32_t off = (ubase ^ (uint32_t)(64 * (fn >> 1))) + (uint32_t)(32 * h * 512 + 8 * (fn & 1));
      const s16x4 lo = lds_read_tr16((lds_char*)smem + off);
      const s16x4 hi = lds_read_tr16((lds_char*)smem + off + 4 * 512);
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      fb[set][fn] = __builtin_bit_cast(bf16x8, v);
      return;
    }
    const uint32_t off = (((h ^ fn) & 1) ? (ubase ^ 64u) : ubase) +
                         (uint32_t)((4 * (fn & 1) + 32 * (fn >> 1)) * kSlabRowB);
    fb[set][fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + off));
  };
  // half of the MFMAs of output-row block r with weight set `set`
  auto mfma_half = [&](int r, int set, int half) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FN / 2; ++i) {
      const int fn = half * (FN / 2) + i;
      acc[r][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[set][fn], fa[r], acc[r][fn], 0, 0, 0);
    }
  };

  const bool has_bias = (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU);
  const bool bias_vec = (reinterpret_cast<uintptr_t>(p.bias) & 15) == 0;

  // ---- ring: super-step q (counted over all tiles of this workgroup) has
  // its A slab in unit (2q) % 5 and its weight slab in unit (2q + 1) % 5.
  int cur_unit = 0;  // A unit of the current super-step
  {
    // prologue: slabs of super-steps 0 and 1 of the first tile (KS >= 2)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k0 = k0_of(s);
      const uint32_t kbytes = 2u * (uint32_t)k0;
      if constexpr (RAGGED) tail_bits = k0 + kSlabK > K ? lane_oob : 0u;  // a reversed tile starts with it
#pragma unroll
      for (int c = 0; c < CPS; ++c) copy_a(c, kbytes, 2 * s);
#pragma unroll
      for (int c = 0; c < CPS_B; ++c) copy_b(c, kbytes, 2 * s + 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPS + CPS_B));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < FM; ++f) read_a(f, 0, a_x0);
#pragma unroll
    for (int f = 0; f < FN; ++f) read_b(0, f, 0, b_x0 + (uint32_t)UNIT);
  }
  // An LDS wait before each tile's K loop (free: the reads are long done by
  // then) lets the compiler's wait placement inside the loop follow the loop's
  // own read order instead of merging it with the prologue's or epilogue's.
  constexpr int kLgkmDrained = waitcnt_vm_lgkm0(63);

  // One super-step q: k-steps 2q (half 0, weight set 0) and 2q+1 (half 1,
  // weight set 1).  Fragments of the next k-step are read as soon as their
  // registers are free; the copies of super-step q+2 (first k k0_fetch in
  // the fetched tile) go out one per MFMA row.  k-step 2q+1 runs its rows in the order 4..7, 0..3, so the
  // fragment read last in a k-step is needed four rows into the next one
  // and no k-step starts by waiting on LDS.
  uint32_t a_cur = a_x0, b_cur = b_x0 + (uint32_t)UNIT;  // units of super-step q
  // BSTAGE: epilogue inputs prefetched under the K loop (issue "Automate
  // performant Hopper matmul", section "Epilogue inputs").  The registers have
  // no room for them during the K loop (holding a tile's bias vectors across
  // it spilled 221 registers), but LDS has, at one moment of every
  // super-step: after its mid-step barrier no wave reads q's weight unit again
  // until the next super-step copies into it.  So in the k-step after that
  // barrier, among its weight copies, each wave copies its 128 columns of the
  // tile's bias (256 bytes) straight from global memory into two of its own
  // 1 KiB blocks of that unit.  The next super-step's first two activation
  // copies of the same wave overwrite those blocks (a wave's later copies land
  // later); the copy of a tile's last super-step survives into the epilogue,
  // which reads the bias back from LDS after a wait that leaves the weight
  // copies issued after it (the next tile's) in flight.  Every super-step
  // does it, with a record of 0 bytes (nothing fetched) when the tile's bias
  // is not staged, so the loop has no branch for it (a branch, or a peeled
  // last super-step, changed the loop's register allocation).  A copy is one
  // 16-byte load per lane at the copies' lane offsets: lanes 0..7 (row 0)
  // fetch the 8 chunks of a 128-byte half, permuted by the row swizzle; the
  // other lanes' offsets lie past the 128-byte record and fill the rest of
  // the block with zeros.
  int bias_n0 = -1;  // first column of this tile if its bias goes through LDS, else -1
  auto copy_bias = [&](int unit) __attribute__((always_inline)) {
    const uint64_t bb = reinterpret_cast<uint64_t>(p.bias) + 2u * (uint32_t)(bias_n0 + wrow_b);
    const uint32_t rec = bias_n0 >= 0 ? 128u : 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const __amdgpu_buffer_rsrc_t r = rsrc(bb + 128u * h, rec);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(smem + unit * UNIT + (h * NW + wave) * 1024), 16,
          lane_base, 0, 0, 0);
    }
  };
  auto super_step = [&](int k0_fetch) __attribute__((always_inline)) {
    const uint32_t kbytes = 2u * (uint32_t)k0_fetch;
    if constexpr (RAGGED) tail_bits = k0_fetch + kSlabK > K ? lane_oob : 0u;
    const int ua = cur_unit, ub = next_unit(ua);
    const int nua = next_unit(ub), nub = next_unit(nua);  // super-step q+1
    const int cua = next_unit(nub);                        // A slab of q+2
    const int cub = ua;                                    // weight slab of q+2
    const uint32_t a_nxt = a_x0 + (uint32_t)(nua * UNIT), b_nxt = b_x0 + (uint32_t)(nub * UNIT);
#ifdef MM_DEBUG_FULL_SYNC
    // Race-check build: every copy landed and every LDS read done, in every
    // wave, before the super-step starts; its results must equal the normal
    // build's bit for bit.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#endif

    // k-step 2q: MFMAs on half 0; half 1 of q (same units) into fa and fb[1]
    // (the first kHeadRows rows form the head's scheduling region)
    constexpr int kHeadRows = FN == 4 ? 3 : 2;
#pragma unroll
    for (int r = 0; r < FM; ++r) {
      mfma_half(r, 0, 0);
      copy_a(r, kbytes, cua);
      if (r < FN / 2) {
        read_b(1, 2 * r, 1, b_cur);
        read_b(1, 2 * r + 1, 1, b_cur);
      }
      const bool head = r < kHeadRows, head_end = r == kHeadRows - 1;
      if (head) {
        mfma_half(r, 0, 1);
        if (head_end) {
          if constexpr (FN == 4) spread_first_rows_a4();
          else if constexpr (FN == 6) spread_first_rows_a6();
          else spread_first_rows_a8();
        }
      } else {
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(r, 0, 1);
      }
      if (!head || head_end) __builtin_amdgcn_sched_barrier(0);
      read_a(r, 1, a_cur);
      if (!head || head_end) __builtin_amdgcn_sched_barrier(0);
    }

    // k-step 2q+1, first row (4): its fragments are already in registers
    mfma_half(4, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_half(4, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    // This wave's copies of q+1 have landed (only the A slab of q+2 may still
    // be in flight) and its reads of q's units are done; after the barrier
    // q+1 is visible to all waves and q's units may be overwritten.
#ifdef MM_DEBUG_FULL_SYNC
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // the A slab of q+2 too
#else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPS));
#endif
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_a(4, 0, a_nxt);
    // rows 5, 6, 7, 0, 1, 2, 3: half 0 of q+1 into fa and fb[0]; the weight
    // slab of q+2 (rows p = 1 .. kHeadRowsB form the head's region)
    constexpr int kHeadRowsB = FN == 4 || FN == 6 ? 2 : 1;
#pragma unroll
    for (int p = 1; p < FM; ++p) {
      const int r = (p + 4) & 7;
      mfma_half(r, 1, 0);
      if (p == 1) copy_b(0, kbytes, cub);
      if (p < CPS_B) copy_b(p, kbytes, cub);
      if constexpr (BSTAGE)
        if (p == 2) copy_bias(ub);  // five weight copies follow it
      if (p <= FN / 2) {
        read_b(0, 2 * (p - 1), 0, b_nxt);
        read_b(0, 2 * (p - 1) + 1, 0, b_nxt);
      }
      const bool head = p <= kHeadRowsB, head_end = p == kHeadRowsB;
      if (head) {
        mfma_half(r, 1, 1);
        if (head_end) {
          if constexpr (FN == 4) spread_rows_b4();
          else if constexpr (FN == 6) spread_rows_b6();
          else spread_first_row_b<FN>();
        }
      } else {
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(r, 1, 1);
      }
      if (p == FM - 1) {
        // last row: the loop's own scalar bookkeeping (counter, compare,
        // carried unit) goes between its MFMAs instead of after them
        read_a(r, 0, a_nxt);
        spread_loop_latch<FN>();
      } else if (!head || head_end) {
        __builtin_amdgcn_sched_barrier(0);
        read_a(r, 0, a_nxt);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        read_a(r, 0, a_nxt);
      }
    }
    cur_unit = nua;
    a_cur = a_nxt;
    b_cur = b_nxt;
  };

  // ---- epilogue straight from the accumulators.  A lane holds 8
  // consecutive columns of a fragment pair; the two pairs that make up one
  // 128-byte output line are stored back to back.  F32 / ACT / CHECKED are
  // compile-time in the fast paths (interior tiles with aligned rows) and
  // run-time in the one checked path for edge tiles.
  const bool act_on = FFN ? (p.epi == EPI_SWIGLU) : (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU);
  constexpr int PAIRS = FFN ? FN / 4 : FN / 2;
  void* obase = p.out;  // output of the current batch entry
  // 8 consecutive outputs of row m from column n on: one 16-byte (bf16) or
  // two 16-byte (fp32) stores when `vec`, else element by element up to N.
  // The vector stores are non-temporal: output lines are written once and
  // never read back, so they should neither displace operand panels from L2
  // nor wait there as dirty lines for the write-back at the end of the
  // kernel (8192^3 linear + bias + GELU: 693.7 -> 684.1 us per launch, the
  // slowest workgroup's lag behind the median one about halved).
  auto store8 = [&](void* base, int m, int n, const float (&v)[8], auto f32, bool vec)
      __attribute__((always_inline)) {
    if (f32) {
      float* o = reinterpret_cast<float*>(base) + (int64_t)m * N + n;
      if (vec) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(o));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(o) + 1);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n + j < N) o[j] = v[j];
      }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(base) + (int64_t)m * N + n;
      if (vec) {
        u32x4 w;
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
        w[2] = pack_bf16x2(v[4], v[5]);
        w[3] = pack_bf16x2(v[6], v[7]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n + j < N) o[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[j]));
      }
    }
  };
  auto epilogue = [&](int m0, int n0, auto f32, auto act, auto checked, auto pre) __attribute__((always_inline)) {
    const int m_base = m0 + wrow_a + lx;
    int ncol[PAIRS];
    float bv[PAIRS][8];
    // A tile whose columns all lie inside N with a 16-byte aligned bias (the
    // same for the whole wave) loads all of its bias vectors before the first
    // wait; other tiles check each lane's columns.
    const bool bias_fast = !FFN && has_bias && bias_vec && n0 + OUT_BN <= N;
    if (BSTAGE && bias_n0 >= 0) {
      // the bias staged in LDS by the last super-step (copy_bias): logical
      // 16-byte chunk 4 pr + lk of the wave's 256 bytes sits in block pr / 2,
      // at physical chunk ((4 pr + lk) & 7) ^ s, s the row-0 swizzle of the
      // copies; five weight copies were issued after it
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(CPS_B - 3));
      const int bunit = cur_unit == 0 ? kSlabUnits - 1 : cur_unit - 1;
      const int bsw = lds_swz(8 * (wave & 2));
      u32x4 w[PAIRS];
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        ncol[pr] = n0 + wrow_b + 32 * pr + 8 * lk;
        w[pr] = *reinterpret_cast<const u32x4*>(smem + bunit * UNIT + ((pr >> 1) * NW + wave) * 1024 +
                                                 16 * (((4 * pr + lk) & 7) ^ bsw));
      }
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[pr][2 * j] = __builtin_bit_cast(float, w[pr][j] << 16);
          bv[pr][2 * j + 1] = __builtin_bit_cast(float, w[pr][j] & 0xffff0000u);
        }
    } else if (bias_fast) {
      u32x4 w[PAIRS];
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        ncol[pr] = n0 + wrow_b + 32 * pr + 8 * lk;
        w[pr] = *reinterpret_cast<const u32x4*>(p.bias + ncol[pr]);
      }
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[pr][2 * j] = __builtin_bit_cast(float, w[pr][j] << 16);
          bv[pr][2 * j + 1] = __builtin_bit_cast(float, w[pr][j] & 0xffff0000u);
        }
    } else
#pragma unroll
    for (int pr = 0; pr < PAIRS; ++pr) {
      const int n = FFN ? n0 + wave_n * (WTN / 2) + 32 * pr + 8 * lk : n0 + wrow_b + 32 * pr + 8 * lk;
      ncol[pr] = n;
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[pr][j] = 0.f;
      if constexpr (!FFN) {
        if (has_bias && bias_vec && n + 8 <= N) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(p.bias + n);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bv[pr][2 * j] = __builtin_bit_cast(float, w[j] << 16);
            bv[pr][2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
          }
        } else if (has_bias) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (n + j < N) bv[pr][j] = __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16);
        }
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = m_base + 16 * fm;
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        const int n = ncol[pr];
        float v[8];
        if constexpr (FFN) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = acc[fm][2 * pr + (j >> 2)][j & 3];
            const float u = acc[fm][FN / 2 + 2 * pr + (j >> 2)][j & 3];
            v[j] = (act ? silu_fast(a) : a) * u;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = acc[fm][2 * pr + (j >> 2)][j & 3] + bv[pr][j];
        }
        if (checked && m >= M) continue;
        const bool vec = !checked || (p.out_vec && n + 8 <= N);
        if constexpr (!FFN) {
          // second output: the pre-activation (bias added, before GELU)
          if (pre) store8(p.out_pre, m, n, v, f32, vec);
          if (act) gelu_tanh8(v);
        }
        store8(obase, m, n, v, f32, vec);
      }
    }
  };

  // Split-K / stream-K end of a work unit: the piece's raw fp32 sums go to
  // its own 256 x 256 row-major workspace slot (every element of the tile,
  // rows and columns past M and N included: they hold zeros).  The pieces
  // meet in splitk_reduce, launched after this kernel on the same stream, so
  // no workgroup waits for another and no cross-XCD cache maintenance is
  // needed inside the kernel.
  auto epilogue_part = [&](float* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int pr = 0; pr < PAIRS; ++pr) {
        const int ml = wrow_a + lx + 16 * fm;      // tile-local row
        const int nl = wrow_b + 32 * pr + 8 * lk;  // tile-local first column
        // (the accumulators are read at their point of use, behind a
        // scheduling barrier, through one vector add each: stored straight
        // from the accumulator registers, or read any earlier, they make the
        // compiler rotate the K loop's accumulators through temporaries.
        // Adding +0 turns a -0 sum into +0, which no later addition can tell
        // apart.)
        __builtin_amdgcn_sched_barrier(0);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = acc[fm][2 * pr + (j >> 2)][j & 3] + 0.0f;
        float* o = slot + ml * 256 + nl;
        reinterpret_cast<f32x4*>(o)[0] = f32x4{v[0], v[1], v[2], v[3]};
        reinterpret_cast<f32x4*>(o)[1] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  };

  for (int tile_i = 0; tile_i < my_tiles; ++tile_i) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The copies of super-step ks fetch this unit's super-step ks + 2, and
    // from ks = nks - 2 on the next unit's super-steps 0 and 1.
    const TileDesc nxt = tile_desc(tile_i + 1 < my_tiles ? tile_i + 1 : tile_i);
    int h_tile, h_slice, h_kbeg, nks;
    unit_of(tile_i, &h_tile, &h_slice, &h_kbeg, &nks);
    int tm, tn;
    if constexpr (BSTAGE) {
      // a tile whose columns all lie inside N, with a 16-byte aligned bias
      // (the same for the whole wave), stages its bias through LDS; other
      // tiles load it in the epilogue
      tile_coords(h_tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
      bias_n0 = (has_bias && bias_vec && (tn + 1) * OUT_BN <= N) ? tn * OUT_BN : -1;
    }
    __builtin_amdgcn_s_waitcnt(kLgkmDrained);
    for (int ks = 0; ks < nks; ++ks) {
      int lks = ks + 2;
      if (lks >= nks) {
        lks -= nks;
        cur = nxt;
      }
      super_step(k0_of(lks));
    }
    if constexpr (SPLITK) {
      // slot of this piece: chunk-major, the workgroup's one chunk; stream-K,
      // piece tile_i (0 or 1) of the workgroup's range
      constexpr int64_t kSlot = 256 * 256;
      const int slot = sk_cmaj ? wg : 2 * wg + tile_i;
      epilogue_part(p.sk_part + (int64_t)slot * kSlot);
      continue;
    }

    if constexpr (!BSTAGE) tile_coords(h_tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * OUT_BN;
    obase = static_cast<char*>(p.out) + (int64_t)h_slice * p.stride_out * (p.out_f32 ? 4 : 2);
    using T = std::true_type;
    using F = std::false_type;
    if constexpr (PRE) {  // bf16, GELU: unmasked on interior tiles
      if (p.out_vec && m0 + BM <= M && n0 + OUT_BN <= N) epilogue(m0, n0, F{}, T{}, F{}, T{});
      else epilogue(m0, n0, F{}, T{}, T{}, T{});
    } else if (p.out_vec && m0 + BM <= M && n0 + OUT_BN <= N) {
      if (FFN || !p.out_f32) {
        if (act_on) epilogue(m0, n0, F{}, T{}, F{}, F{});
        else epilogue(m0, n0, F{}, F{}, F{}, F{});
      } else {
        if (act_on) epilogue(m0, n0, T{}, T{}, F{}, F{});
        else epilogue(m0, n0, T{}, F{}, F{}, F{});
      }
    } else {
      epilogue(m0, n0, p.out_f32 != 0, act_on, T{}, F{});
    }
  }
}

// Second launch of a split-K product: out = the epilogue of the sum of the
// pieces' partial tiles (added in k order): + bias[n] and/or GELU, rounded
// once to the output type.  Block b covers rows
// 8 (b % 32) .. + 8 of tile b / 32.  Chunk-major: the pieces of tile t are the
// slots j T + t, j = 0 .. n - 1.  Stream-K: chunk range [w q, (w + 1) q) of
// workgroup w covers the tail of one tile and/or the head of the next; its
// piece i lives in slot 2 w + i, and the workgroups covering tile t are
// t n / q .. ((t + 1) n - 1) / q.
__global__ void __launch_bounds__(256) splitk_reduce(SkReduceParams p) {
  const int t = blockIdx.x >> 5;
  const int r0 = (blockIdx.x & 31) << 3;
  int tm, tn;
  tile_coords(t, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
  int s0, s1, sstep;  // workgroups (stream-K) or slots (chunk-major) s0, s0 + sstep, .., s1
  if (p.items == 0) {
    s0 = t;
    s1 = t + (p.chunks - 1) * p.num_tiles;
    sstep = p.num_tiles;
  } else {
    s0 = (t * p.chunks) / p.items;
    s1 = ((t + 1) * p.chunks - 1) / p.items;
    sstep = 1;
  }
  auto slot_of = [&](int w) { return p.items == 0 ? w : 2 * w + (t - (w * p.items) / p.chunks); };
  const bool add_bias = p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU;
  const bool gelu = p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU;
  if (!p.out_vec) {
    // rows not 16-byte aligned: thread = one column of the 8 rows, so that
    // each load and each store of a wave covers consecutive elements
    const int c = threadIdx.x;
    const int n = tn * p.tile_n + c;
    if (c >= p.tile_n || n >= p.N) return;
    float v[8];
    for (int w = s0; w <= s1; w += sstep) {
      const float* src = p.part + (int64_t)slot_of(w) * (256 * 256) + r0 * 256 + c;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = src[j * 256];
        v[j] = w == s0 ? x : v[j] + x;
      }
    }
    const float bn = add_bias ? __builtin_bit_cast(float, (uint32_t)p.bias[n] << 16) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] += bn;
      if (gelu) v[j] = gelu_tanh(v[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = tm * 256 + r0 + j;
      if (m >= p.M) break;
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[(int64_t)m * p.N + n] = v[j];
      else
        reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.N + n] =
            __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[j]));
    }
    return;
  }
  // aligned rows: thread = 8 consecutive columns of one row, 16-byte accesses
  const int r = r0 + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) << 3;
  const int m = tm * 256 + r, n = tn * p.tile_n + c;
  if (c >= p.tile_n || m >= p.M || n >= p.N) return;
  float v[8];
  for (int w = s0; w <= s1; w += sstep) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.part + (int64_t)slot_of(w) * (256 * 256) + r * 256 + c);
    const f32x4 x0 = src[0], x1 = src[1];
    if (w == s0) {
      v[0] = x0[0]; v[1] = x0[1]; v[2] = x0[2]; v[3] = x0[3];
      v[4] = x1[0]; v[5] = x1[1]; v[6] = x1[2]; v[7] = x1[3];
    } else {
      v[0] += x0[0]; v[1] += x0[1]; v[2] += x0[2]; v[3] += x0[3];
      v[4] += x1[0]; v[5] += x1[1]; v[6] += x1[2]; v[7] += x1[3];
    }
  }
  const bool vec = n + 8 <= p.N;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (add_bias && n + j < p.N) v[j] += __builtin_bit_cast(float, (uint32_t)p.bias[n + j] << 16);
    if (gelu) v[j] = gelu_tanh(v[j]);
  }
  if (p.out_f32) {
    float* o = reinterpret_cast<float*>(p.out) + (int64_t)m * p.N + n;
    if (vec) {
      __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(o));
      __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(o) + 1);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (n + j < p.N) o[j] = v[j];
    }
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (int64_t)m * p.N + n;
    if (vec) {
      u32x4 w;
      w[0] = pack_bf16x2(v[0], v[1]);
      w[1] = pack_bf16x2(v[2], v[3]);
      w[2] = pack_bf16x2(v[4], v[5]);
      w[3] = pack_bf16x2(v[6], v[7]);
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (n + j < p.N) o[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[j]));
    }
  }
}

}  // namespace mmk
