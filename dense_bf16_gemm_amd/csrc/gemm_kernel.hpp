// gemm_kernel.hpp -- persistent bf16 MFMA GEMM for gfx950 (CDNA4).
//
// One template covers the MatmulOp and LinearOp forms in every operand
// layout, the fused epilogues and the two-weight FFN (horizontal fusion).
//
// Structure of one workgroup (4 waves of 64 lanes by default):
//   * Persistent loop (issue "Automate performant Hopper matmul", section
//     "Persistent matmul": cooperative persistent strategy).  The grid holds
//     one wave of resident workgroups; workgroup w takes tiles w, w+G, ...
//   * Tile order (same issue, section "Operand load efficiency/L2 locality/
//     grid swizzling"): the workgroup id is first remapped so that the ids
//     the hardware places on one XCD (round-robin over the 8 XCDs) become
//     consecutive, then tiles are walked in bands of G tile-rows, column by
//     column inside a band (a Z-like order), with a short last band instead
//     of padding, so a large band height adds no extra waves.
//   * K direction alternates from one persistent tile to the next when the
//     K loop is long (same section: turning around in the K loop finds the
//     most recently used K panels still in cache).
//   * The K loop and the tile loop are one flattened loop over (tile, k-step)
//     pairs: the prefetch of the next k-step runs across tile boundaries, so
//     the LDS ring position is a running counter that never resets at a new
//     tile (same issue, section "Syncing persistent matmuls"), and the next
//     tile's first loads are in flight while this tile's epilogue runs
//     (section "Syncing issues": overlap stores with the next tile's MMAs).
//   * global -> VGPR -> LDS double buffer, one barrier per k-step; LDS rows
//     of 64 bf16 (128 B) with 16-byte chunks XOR-swizzled by the row so that
//     both the writes and the MFMA fragment reads are bank-conflict free
//     (section "Epilogue inputs": avoid bank conflicts).  Operands whose
//     contiguous dimension is M or N are transposed in registers (8x8 bf16
//     blocks) on their way into the same k-contiguous LDS layout, so the
//     stored transpose is read in place and never materialised (PR
//     "Translate MmaOp patterns properly on Hopper", description: skip
//     metadata ops / intermediates).
//   * v_mfma_f32_16x16x32_bf16 with fp32 accumulators; the weight tile feeds
//     the MFMA's first operand so each lane ends with runs of output columns,
//     and fragment rows are permuted so a lane owns 8 consecutive columns.
//   * Epilogue straight from the accumulators: bias, GELU(tanh), SiLU-gate,
//     one rounding (RNE) to bf16 or fp32 stores, ragged edges masked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mmk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Epilogue codes (kernel-internal; the C ABI maps onto them).
enum : int {
  EPI_NONE = 0,
  EPI_BIAS = 1,
  EPI_GELU = 2,
  EPI_BIAS_GELU = 3,
  EPI_SWIGLU = 4,
  EPI_GLU_ID = 5
};

constexpr int kBK = 64;          // K elements per k-step
constexpr int kRowBytes = 128;   // one LDS row = 64 bf16
constexpr int kNumXcd = 8;       // MI355X: 8 accelerator dies, round-robin dispatch

struct GemmParams {
  const uint16_t* A;     // stored [M][K] (A_KC) or [K][M]
  const uint16_t* B;     // stored [N][K] (B_KC) or [K][N]; gate weight for the FFN
  const uint16_t* B2;    // FFN up weight [N][K], else unused
  const uint16_t* bias;  // [N] or null
  void* out;             // [M][N] bf16 or fp32
  void* out_pre;         // null, or a second [M][N] output of the same type that
                         // receives the pre-activation of a GELU epilogue
  int M, N, K;
  int epi;
  int out_f32;
  int out_vec;           // 16-byte vector stores are aligned for every row
  int tiles_m, tiles_n, num_tiles, k_tiles;
  int group_m;           // band height of the grouped tile order, in tiles
  int xcd_remap;
  int k_alt;             // alternate K direction per persistent tile
  // Split-K / stream-K (gemm_nt_slab with SPLITK): each tile's K loop is cut
  // into sk_chunks chunks (chunk j: super-steps [j*KS/n, (j+1)*KS/n)).
  // sk_items == 0 (chunk-major): workgroup c runs chunk c / num_tiles of tile
  // c % num_tiles, so that workgroups running at once cover neighbouring
  // tiles at the same k (they share operand panels in L2).  sk_items = q > 0
  // (stream-K): the num_tiles * n chunks, tile-major, are dealt to the
  // workgroups in contiguous ranges of q (< n) chunks; a range covers the
  // tail of one tile and/or the head of the next.  Every piece writes its
  // raw fp32 partial tile into its own workspace slot; splitk_reduce adds
  // them in k order afterwards.
  // Batched form: `batch` independent products; operand / output bases of
  // entry b are b * stride elements past entry 0 (a stride of 0 broadcasts).
  // The persistent loop walks batch * num_tiles units, unit u being tile
  // u % num_tiles of entry u / num_tiles.
  int batch;             // >= 1
  int64_t stride_a, stride_b, stride_out;
  int sk_chunks;         // n (1 = off)
  int sk_items;          // chunks per workgroup range (0: chunk-major, one each)
  float* sk_part;        // partial tiles of 256*256 floats: slot wg (chunk-major)
                         // or 2 wg + piece (stream-K)
};

// The split-K reduction's arguments (the same tiles, order and dealing as
// the GemmParams of the launch before it).
struct SkReduceParams {
  const float* part;
  void* out;
  int M, N;
  int tiles_m, tiles_n, num_tiles, group_m;
  int chunks;  // n
  int items;   // q, 0 = chunk-major
  int out_f32, out_vec;
  int tile_n;  // output columns per tile (256, or 192); slots stay 256 columns wide
  const uint16_t* bias;  // [N], read when epi adds a bias
  int epi;               // EPI_NONE / EPI_BIAS / EPI_GELU / EPI_BIAS_GELU, on the summed value
};

// A product with K = 0 (empty_k_fill): every sum over k is empty.
struct EmptyKParams {
  const uint16_t* bias;  // read only when epi adds a bias
  void* out;
  void* out_pre;        // the pre-activation output, or null
  int64_t M, N, batch;
  int64_t stride_out;   // elements between batch entries of out
  int epi;              // EPI_*; the gated FFN forms pass EPI_NONE
  int out_f32;
};

// Schedule helpers, shared with the host so that it can describe the order.
__host__ __device__ inline int remap_workgroup(int b, int G, int on) {
  if (!on || G < kNumXcd) return b;
  const int per = G / kNumXcd, rem = G % kNumXcd;
  const int xcd = b % kNumXcd, local = b / kNumXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Entry of the batched form that persistent unit u belongs to, its tile
// index inside the entry, and the entry's operand and output bases.
struct BatchView {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* B2;
  void* out;
  int tile;
};
__device__ __forceinline__ BatchView batch_view(const GemmParams& p, int u) {
  BatchView v{p.A, p.B, p.B2, p.out, u};
  if (p.batch > 1) {
    const int b = __builtin_amdgcn_readfirstlane(u / p.num_tiles);
    v.tile = u - b * p.num_tiles;
    v.A = p.A + (int64_t)b * p.stride_a;
    v.B = p.B + (int64_t)b * p.stride_b;
    v.B2 = p.B2 ? p.B2 + (int64_t)b * p.stride_b : nullptr;
    v.out = static_cast<char*>(p.out) + (int64_t)b * p.stride_out * (p.out_f32 ? 4 : 2);
  }
  return v;
}

__host__ __device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int* tm,
                                            int* tn) {
  const int band = group_m * tiles_n;
  const int g = t / band;
  const int first_m = g * group_m;
  const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int r = t - g * band;
  *tm = first_m + r % rows;
  *tn = r / rows;
}

// 16 zero bytes in device memory: the source of every direct-to-LDS copy
// whose chunk lies past K, so a ragged last k-step arrives zero-filled.
__device__ const u32x4 g_zero_chunk[1] = {{0u, 0u, 0u, 0u}};

// XOR swizzle of the 16-byte chunk index by the LDS row: chunk ^ (row & 7)
// ^ (bit 4 of row moved to bit 2).  Chosen by measuring SQ_LDS_BANK_CONFLICT
// for candidate XOR maps on the two ds_read_b128 fragment patterns used
// below (16 consecutive rows; and the comb of 4 runs of 4 rows 8 apart used
// by the permuted weight fragments): this one is conflict free on both, so a
// 1 KiB fragment read takes the minimum 4 LDS cycles.  The direct-to-LDS
// copies write whole rows and never conflict.  Depends on row bits 0..4 only.
__host__ __device__ __forceinline__ int lds_swz(int row) {
  return (row ^ ((row >> 2) & 4)) & 7;
}

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * kRowBytes + ((chunk ^ lds_swz(row)) << 4));
}

__device__ __forceinline__ u32x4 zero4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

__device__ __forceinline__ float gelu_tanh(float t) {
  // 0.5 t (1 + tanh z) == t / (1 + exp(-2 z)),  z = sqrt(2/pi) (t + 0.044715 t^3)
  const float z = 0.7978845608028654f * (t + 0.044715f * t * t * t);
  return t * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * z));
}

__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Two floats to a packed pair of bf16 (round to nearest even), low half
// first: one v_cvt_pk_bf16_f32 through a two-element vector conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Eight consecutive outputs of row m from column n on, into the [M][N]
// row-major `base` (fp32 or bf16): 16-byte stores when `vec` and the eight
// columns lie inside N, else element by element.
__device__ __forceinline__ void store_row8(void* base, int f32, int vec, int m, int N, int n,
                                           const float (&v)[8]) {
  if (f32) {
    float* o = reinterpret_cast<float*>(base) + (int64_t)m * N + n;
    if (vec && n + 8 <= N) {
      reinterpret_cast<f32x4*>(o)[0] = f32x4{v[0], v[1], v[2], v[3]};
      reinterpret_cast<f32x4*>(o)[1] = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (n + j < N) o[j] = v[j];
    }
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(base) + (int64_t)m * N + n;
    if (vec && n + 8 <= N) {
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

// ---------------------------------------------------------------------------
// Operand staging: global -> registers -> LDS, for one operand tile of ROWS
// LDS rows (rows = M or N indices) by 64 k.
// ---------------------------------------------------------------------------

// K-contiguous storage ([rows][K]): copied straight from global memory into
// LDS with global_load_lds_dwordx4 (no VGPR staging).  One instruction fills
// 1 KiB of LDS = 8 rows; lane L writes the 16 bytes at L*16, i.e. LDS row
// 8j + L/8, physical chunk L%8, so the XOR swizzle is applied by choosing
// which global chunk each lane fetches.  Chunks at k >= K copy 16 zero bytes
// instead, so a ragged last k-step needs no masking in the MFMA loop.
template <int ROWS, int T>
struct DirectStage {
  static constexpr int WAVES = T / 64;
  static constexpr int INSTR = ROWS / 8;
  static constexpr int PER_WAVE = INSTR / WAVES;
  static_assert(PER_WAVE >= 1 && INSTR % WAVES == 0, "tile too small for the wave count");

  template <typename RowSrc>
  __device__ __forceinline__ void issue(const RowSrc& row_src, char* lds_tile, int k0, int K,
                                        int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int j = i * WAVES + wave;
      const int rho = 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz(rho);
      const int k = k0 + 8 * c;
      const uint16_t* src = row_src(rho) + k;
      const uint16_t* g = k < K ? src : reinterpret_cast<const uint16_t*>(g_zero_chunk);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(g),
          (__attribute__((address_space(3))) void*)(lds_tile + j * 1024), 16, 0, 0);
    }
  }
};

// MN-contiguous storage ([K][extent]): each thread moves 8x8 blocks and
// transposes them in registers.  Lane order puts the 8 k-blocks of one
// column block on 8 consecutive lanes, so both the global reads (8 rows of
// 128 contiguous bytes per wave instruction) and the LDS writes are clean.
template <int ROWS, int T>
struct MNContigStage {
  static constexpr int NB = ROWS;  // 8x8 blocks in a ROWS x 64 tile
  static constexpr int BL = (NB + T - 1) / T;
  u32x4 v[BL][8];

  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int row0, int extent, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int q = 0; q < BL; ++q) {
      const int id = q * T + tid;
      const int kb = id & 7, nb = id >> 3;
      const int col = row0 + 8 * nb;
      const bool ok = (id < NB) && (col < extent);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + 8 * kb + i;
        v[q][i] = (ok && k < K) ? *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + col)
                                : zero4();
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < BL; ++q) {
      const int id = q * T + tid;
      if (id >= NB) continue;
      const int kb = id & 7, nb = id >> 3;
      // w[j] = 8 k-values of column j: element j of v[0..7]
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int word = j >> 1;
        const bool hi = j & 1;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = v[q][2 * e][word];
          const uint32_t b = v[q][2 * e + 1][word];
          w[e] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<u32x4*>(lds + lds_off(8 * nb + j, kb)) = w;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The kernel.
//   BM x BN   : LDS tile rows of A (M) and of B (N; for the FFN, gate+up)
//   WGM x WGN : wave grid; each wave owns (BM/WGM) x (BN/WGN)
//   A_KC      : A stored [M][K] (else [K][M]);  B_KC: B stored [N][K]
//   FFN       : B tile = W_gate and W_up rows for BN/2 output columns
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, bool A_KC, bool B_KC, bool FFN>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_persistent(GemmParams p) {
  constexpr int T = WGM * WGN * 64;
  constexpr int WTM = BM / WGM;      // wave rows of M
  constexpr int WTN = BN / WGN;      // wave rows of the B tile
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int OUT_BN = FFN ? BN / 2 : BN;  // output columns per tile
  static_assert(FN % 2 == 0, "fragment pairs");
  static_assert(!FFN || (FN % 4 == 0), "FFN wave tile holds gate and up pairs");
  static_assert(!FFN || B_KC, "FFN weights are [N][K]");
  constexpr int A_BYTES = BM * kRowBytes;
  constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave / WGN;
  const int wave_n = wave % WGN;
  const int G = gridDim.x;
  const int wg = remap_workgroup(blockIdx.x, G, p.xcd_remap);
  const int units = p.num_tiles * p.batch;
  if (wg >= units) return;
  const int my_tiles = (units - wg + G - 1) / G;
  const int KT = p.k_tiles;

  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = A_KC ? (int64_t)K : (int64_t)M;
  const int64_t ldb = B_KC ? (int64_t)K : (int64_t)N;

  // --- operand movers --------------------------------------------------------
  DirectStage<BM, T> da;
  DirectStage<BN, T> db;
  MNContigStage<A_KC ? 8 : BM, T> sa;  // register-staged only when not K-contiguous
  MNContigStage<B_KC ? 8 : BN, T> sb;

  auto kstep_of = [&](int tile_i, int kt) {
    return (p.k_alt && (tile_i & 1)) ? (KT - 1 - kt) : kt;
  };

  // Starts the global reads of one k-step: direct LDS copies for K-contiguous
  // operands (into buffer `buf`), register loads for the others.
  auto issue_loads = [&](int tile_i, int kt, int buf) {
    int tm, tn;
    const BatchView bview = batch_view(p, wg + tile_i * G);
    tile_coords(bview.tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    const int k0 = kstep_of(tile_i, kt) * kBK;
    const int m0 = tm * BM;
    const int n0 = tn * OUT_BN;
    char* stage = smem + buf * STAGE_BYTES;
    if constexpr (A_KC) {
      auto rowA = [&](int r) {
        int row = m0 + r;
        row = row < M ? row : M - 1;
        return bview.A + (int64_t)row * lda;
      };
      da.issue(rowA, stage, k0, K, wave, lane);
    } else {
      sa.load(bview.A, lda, m0, M, k0, K, tid);
    }
    if constexpr (B_KC) {
      auto rowB = [&](int r) {
        const uint16_t* base = bview.B;
        int row;
        if constexpr (FFN) {
          const int wb = r / WTN, within = r % WTN;
          const bool up = within >= WTN / 2;
          row = n0 + wb * (WTN / 2) + (up ? within - WTN / 2 : within);
          base = up ? bview.B2 : bview.B;
        } else {
          row = n0 + r;
        }
        row = row < N ? row : N - 1;
        return base + (int64_t)row * ldb;
      };
      db.issue(rowB, stage + A_BYTES, k0, K, wave, lane);
    } else {
      sb.load(bview.B, ldb, n0, N, k0, K, tid);
    }
  };

  // Writes the register-staged operands of a k-step into buffer `buf`.
  auto store_staged = [&](int buf) {
    char* stage = smem + buf * STAGE_BYTES;
    if constexpr (!A_KC) sa.store(stage, tid);
    if constexpr (!B_KC) sb.store(stage + A_BYTES, tid);
  };

  // --- per-lane fragment addressing --------------------------------------
  // X operand (B tile) fragment fn, lane row x = lane&15 (= 4g'+r') maps to
  // B-tile row  32*(fn>>1) + 8*(x>>2) + 4*(fn&1) + (x&3)  within the wave.
  const int lx = lane & 15;
  const int lk = lane >> 4;  // k-chunk within a 32-wide k slice
  const int wrow_a = wave_m * WTM;
  const int wrow_b = wave_n * WTN;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS byte offsets of the fragments.  Fragment rows differ from
  // these bases by multiples of 32 rows (B) or 16 rows (A); since the
  // swizzle depends on row bits 0..4 only, the swizzled chunk of fragment
  // (s, fn) is that of base [s][fn & 1] (B) or [s][fm & 1] (A), and the rest
  // of the offset is a compile-time constant.
  uint32_t boff[2][2], aoff[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rb = wrow_b + 8 * (lx >> 2) + 4 * h + (lx & 3);
      boff[s][h] = lds_off(rb, 4 * s + lk);
      const int ra = wrow_a + 16 * h + lx;
      aoff[s][h] = lds_off(ra, 4 * s + lk);
    }

  // One k-step of MFMAs from LDS buffer `buf` (chunks past K are zero).
  auto compute_stage = [&](int buf) {
    const char* As = smem + buf * STAGE_BYTES;
    const char* Bs = As + A_BYTES;
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      bf16x8 xb[FN], ya[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        xb[fn] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(Bs + boff[s][fn & 1] + (fn >> 1) * 32 * kRowBytes));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        ya[fm] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(As + aoff[s][fm & 1] + (fm & ~1) * 16 * kRowBytes));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[fn], ya[fm], acc[fm][fn], 0, 0, 0);
    }
  };

  // --- epilogue --------------------------------------------------------------
  auto epilogue = [&](int tile_i) {
    int tm, tn;
    const BatchView bview = batch_view(p, wg + tile_i * G);
    tile_coords(bview.tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
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
        if (has_bias && n + j < N) {
          const uint32_t h = p.bias[n + j];
          b = __builtin_bit_cast(float, h << 16);
        }
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
            y = a + bv[j];  // the pre-activation, activated after its store
          }
          v[j] = y;
        }
        if (m >= M) continue;
        if constexpr (!FFN) {
          if (p.out_pre) store_row8(p.out_pre, p.out_f32, p.out_vec, m, N, n, v);
          if (gelu) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = gelu_tanh(v[j]);
          }
        }
        if (p.out_f32) {
          float* o = reinterpret_cast<float*>(bview.out) + (int64_t)m * N + n;
          if (p.out_vec && n + 8 <= N) {
            reinterpret_cast<f32x4*>(o)[0] = f32x4{v[0], v[1], v[2], v[3]};
            reinterpret_cast<f32x4*>(o)[1] = f32x4{v[4], v[5], v[6], v[7]};
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (n + j < N) o[j] = v[j];
          }
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(bview.out) + (int64_t)m * N + n;
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

  // --- persistent tile loop around the K loop ---------------------------------
  // `it` counts k-steps over all of this workgroup's tiles; buffer it & 1
  // holds k-step `it`, so the ring position carries across tiles instead of
  // restarting at each one.  At the top of every k-step a wave waits for its
  // own outstanding loads (vmcnt 0) and the barrier makes every wave's copies
  // visible and guarantees that all waves have finished reading the other
  // buffer, which the next k-step's loads -- possibly the next tile's first --
  // then overwrite while this k-step computes (and this tile's epilogue runs).
  issue_loads(0, 0, 0);
  store_staged(0);
  int it = 0;
  for (int tile_i = 0; tile_i < my_tiles; ++tile_i) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < KT; ++kt, ++it) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // the k-step after this one: the next of this tile, or the next tile's first
      const bool last_k = (kt + 1 == KT);
      const bool has_next = !last_k || (tile_i + 1 < my_tiles);
      const int nt = last_k ? tile_i + 1 : tile_i;
      const int nk = last_k ? 0 : kt + 1;
      if (has_next) issue_loads(nt, nk, (it + 1) & 1);
      compute_stage(it & 1);
      if (has_next) store_staged((it + 1) & 1);
    }
    epilogue(tile_i);
  }
}

// K = 0: the sum over k of each output is empty, i.e. 0, so the output is
// the epilogue applied to 0 + bias[n] (GELU(bias[n]), bias[n] or 0), rounded
// once; the gated FFN forms give act(0) * 0 = 0.  One element per thread,
// batch entries and rows in order.
__global__ void __launch_bounds__(256) empty_k_fill(EmptyKParams p) {
  const int64_t per = p.M * p.N;
  const int64_t total = per * p.batch;
  const bool add_bias = p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU;
  const bool act = p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / per;
    const int64_t e = i - b * per;
    const int64_t o = b * p.stride_out + e;
    const float t = add_bias ? __builtin_bit_cast(float, (uint32_t)p.bias[e % p.N] << 16) : 0.0f;
    const float y = act ? gelu_tanh(t) : t;
    if (p.out_f32) {
      static_cast<float*>(p.out)[o] = y;
      if (p.out_pre) static_cast<float*>(p.out_pre)[o] = t;
    } else {
      static_cast<uint16_t*>(p.out)[o] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));
      if (p.out_pre) static_cast<uint16_t*>(p.out_pre)[o] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(t));
    }
  }
}

}  // namespace mmk
