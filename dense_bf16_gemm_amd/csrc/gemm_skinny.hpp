// Skinny products: at most 32 rows of activations against a large weight
// (the decode step of a served model at small batch: x [M][K], M <= 32,
// W [N][K]).
//
// Such a product is bound by reading W once from HBM; its MFMA work is small.
// The 256-row tiles of the slab kernel would spend almost all of their MFMAs
// on rows past M, so here a workgroup takes 64 of W's rows (64 output
// columns) and streams them once through a ring of three LDS stages of 256
// k.  Each wave-wide copy fills two rows' 512-byte runs straight from
// memory into LDS (buffer loads to LDS: no registers), the 16 or 32
// activation rows of the stage come the same way, and the four waves each
// multiply a quarter of the stage's k-steps with MFMAs whose fragments are
// read from LDS; the waves' parts meet in LDS in a fixed order at the end.
// With a workspace K may also be cut into S slices (when the workgroups
// would not keep HBM busy otherwise): each writes its fp32 sums to slice s
// of the workspace and skinny_reduce adds the slices in k order.  Results: fp32 sums of the bf16
// products, the epilogue on the sum, one rounding -- the contraction and
// epilogue of the other kernels.
//
// Whole-row runs matter: with fragments loaded straight into registers
// (each load reading 64 bytes of 16 rows) the same products ran at 3.0-3.3
// TB/s of weights; a streaming probe reading whole 1 KiB runs per load
// reached 5.1 TB/s.  Measured with the weights rotated over more than 1 GiB
// of copies (no cache reuse), in us against the register-fragment form and
// the platform BLAS: 16 x 28672 x 8192 144 -> 100 (116), 16 x 14336 x 4096
// 40 -> 28.2 (29.0), 16 x 4096 x 14336 41 -> 25.5 (25.8), 16 x 8192 x 8192
// 43 -> 32.9 (28.8).  Not kept: 32-row groups with 512-k stages (one row per
// copy; 33-35 us at 8192 x 8192, 115 us at 28672 x 8192), 48-row groups,
// four or five stages (no gain), and rotating each workgroup's first stage
// (faster at 14336 x 4096, 6 us slower at 8192 x 8192).  Rows 17-32 (two
// activation blocks, 48 KiB stages): 24 x 8192 x 8192 49.0 -> 35.9 us and
// 32 x 14336 x 4096 47.7 -> 30.9 against the tile kernels (BLAS 30.0, 26.2),
// 32 x 28672 x 8192 106.6 -> 102.3 (112.6).  Four blocks (64 rows, two 64
// KiB stages) lost to the tile kernels: 64 x 28672 x 8192 112.9 -> 134.3 us.
#pragma once

#include "gemm_kernel.hpp"
#include "gemm_nt_pipe.hpp"

namespace mmk {

struct SkinnyParams {
  const uint16_t* A;     // x [M][K]
  const uint16_t* B;     // W [N][K]
  const uint16_t* bias;  // [N] or null
  void* out;             // [M][N], bf16 or fp32
  float* part;           // [S][M][N] fp32 partial sums (S > 1), else null
  int M, N, K;
  int kc;      // k per workgroup slice (a multiple of 64); the last may be shorter
  int slices;  // S
  int epi;
  int out_f32;
};

constexpr int kSkinnyMaxM = 32;
constexpr int kSkinnyMaxSlices = 16;
// Per XB (blocks of 16 activation rows): weight rows per workgroup, k per
// stage (256: 512-byte runs, two rows per copy) and stages in the LDS ring
// (three, of 40 KiB for one block and 48 KiB for two).
__host__ __device__ constexpr int skinny_xb(int m) { return m <= 16 ? 1 : 2; }
__host__ __device__ constexpr int skinny_rows(int) { return 64; }
__host__ __device__ constexpr int skinny_kd(int) { return 256; }
__host__ __device__ constexpr int skinny_stages(int) { return 3; }
__host__ __device__ constexpr int skinny_stage_bytes(int xb) { return (skinny_rows(xb) + 16 * xb) * skinny_kd(xb) * 2; }

// s_waitcnt for the copies of `ahead` stages (at most A) left in flight
template <int PER, int A>
__device__ __forceinline__ void skinny_wait(int ahead) {
  if constexpr (A == 0) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  } else {
    if (ahead >= A)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(A * PER));
    else
      skinny_wait<PER, A - 1>(ahead);
  }
}

// epilogue of one output: + bias, activation, one rounding
__device__ __forceinline__ void skinny_store(const SkinnyParams& p, int m, int n, float v) {
  if (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU) v += __builtin_bit_cast(float, (uint32_t)p.bias[n] << 16);
  if (p.epi == EPI_GELU || p.epi == EPI_BIAS_GELU) v = gelu_tanh(v);
  if (p.out_f32)
    reinterpret_cast<float*>(p.out)[(int64_t)m * p.N + n] = v;
  else
    reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.N + n] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// XB: blocks of 16 activation rows (M <= 16 XB)
template <int XB>
__global__ void __launch_bounds__(256) gemm_skinny(SkinnyParams p) {
  constexpr int R = skinny_rows(XB), KD = skinny_kd(XB), NS = skinny_stages(XB), SB = skinny_stage_bytes(XB);
  constexpr int XM = 16 * XB;           // activation rows in a stage
  constexpr int P = KD * 2;             // bytes of a row in a stage
  constexpr int CPR = KD / 8;           // 16-byte chunks of a row in a stage
  constexpr int RPI = 64 / CPR;         // rows per wave-wide copy
  constexpr int WC = R / RPI / 4, XC = XM / RPI / 4;  // copies per wave and stage
  static_assert(CPR >= 16 && CPR <= 64 && R % (4 * RPI) == 0 && XM % (4 * RPI) == 0, "stage shape");
  static_assert(NS * SB <= 160 * 1024 && 3 * XB * (R / 16) * 1024 <= NS * SB, "LDS");
  constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
  constexpr uint32_t kOob = 0x80000000u;  // past every record count below
  __shared__ __attribute__((aligned(1024))) char smem[NS * SB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lx = lane & 15, lk = lane >> 4;
  const int ngroups = (p.N + R - 1) / R;
  const int s = __builtin_amdgcn_readfirstlane((int)blockIdx.x / ngroups);
  const int g = __builtin_amdgcn_readfirstlane((int)blockIdx.x - s * ngroups);
  const int M = p.M, N = p.N, K = p.K;
  const int64_t n0 = (int64_t)g * R;

  // the workgroup's slice [kbeg, kend) of K in stages of KD
  const int kbeg = s * p.kc;
  const int kend = min(K, kbeg + p.kc);
  const int nst = (kend - kbeg + KD - 1) / KD;

  // Copies: a stage holds KD k of the group's R weight rows and of the XM
  // activation rows; each wave-wide LDS copy fills RPI rows of it.  The
  // lane that fills chunk position c of row r fetches the row's 16-byte
  // chunk c ^ (r & 15), so that the fragment reads of 16 rows at one chunk
  // fall in 16 distinct bank groups.  Rows past N or M lie past the
  // descriptors' record counts and read as zeros; chunks past the slice's
  // end are pushed past them.
  const uint64_t rec_w64 = (uint64_t)(N - n0) * (uint64_t)K * 2u;
  // (clamped below bit 31: with K <= 2^23 the group's own rows end below
  // 2^30, far inside the clamped count at every k0)
  const uint32_t rec_w = rec_w64 > 0x7fffffffull ? 0x7fffffffu : (uint32_t)rec_w64;
  const uint32_t rec_x = (uint32_t)M * (uint32_t)K * 2u;
  uint32_t voff_w[WC], voff_x[XC];
  int chunk_w[WC], chunk_x[XC];
#pragma unroll
  for (int i = 0; i < WC; ++i) {
    const int r = (wave * WC + i) * RPI + lane / CPR;
    chunk_w[i] = (lane % CPR) ^ (r & 15);
    voff_w[i] = (uint32_t)r * (uint32_t)K * 2u + 16u * (uint32_t)chunk_w[i];
  }
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int r = (wave * XC + i) * RPI + lane / CPR;
    chunk_x[i] = (lane % CPR) ^ (r & 15);
    voff_x[i] = (uint32_t)r * (uint32_t)K * 2u + 16u * (uint32_t)chunk_x[i];
  }
  auto rsrc = [&](const uint16_t* base, uint32_t rec) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* ptr = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, (int)__builtin_amdgcn_readfirstlane(rec), kRsrcWord3);
  };
  auto copy_stage = [&](int st) __attribute__((always_inline)) {
    char* slot = smem + (st % NS) * SB;
    const int k0 = kbeg + st * KD;
    const int lim = kend - k0;  // k of the stage inside the slice
    // the descriptors start at k0: the record counts shrink by as much
    const __amdgpu_buffer_rsrc_t rw = rsrc(p.B + n0 * K + k0, rec_w - 2u * (uint32_t)k0);
    const __amdgpu_buffer_rsrc_t rx = rsrc(p.A + k0, rec_x - 2u * (uint32_t)k0);
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      const uint32_t off = voff_w[i] | (lim < KD && 8 * chunk_w[i] >= lim ? kOob : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(slot + (wave * WC + i) * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const uint32_t off = voff_x[i] | (lim < KD && 8 * chunk_x[i] >= lim ? kOob : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(slot + R * P + (wave * XC + i) * 1024), 16, off, 0, 0, 0);
    }
  };

  // wave w multiplies k-steps w*KS .. w*KS+KS-1 (32 k each) of every stage
  constexpr int KS = KD / 128;
  // acc[b * CB + c]: activation block b against weight block c
  constexpr int CB = R / 16, NA = XB * CB;
  f32x4 acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int st) __attribute__((always_inline)) {
    const char* slot = smem + (st % NS) * SB;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int pos = ((4 * (KS * wave + q) + lk) ^ lx) * 16;
      u32x4 xf[XB];
#pragma unroll
      for (int b = 0; b < XB; ++b) xf[b] = *reinterpret_cast<const u32x4*>(slot + (R + 16 * b + lx) * P + pos);
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const u32x4 wf = *reinterpret_cast<const u32x4*>(slot + (16 * c + lx) * P + pos);
#pragma unroll
        for (int b = 0; b < XB; ++b)
          acc[b * CB + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xf[b]), __builtin_bit_cast(bf16x8, wf), acc[b * CB + c], 0, 0, 0);
      }
    }
  };

  // ring of NS stages: stage st+NS-1 is fetched into the slot that stage
  // st-1 held, once every wave is past it
  constexpr int kCopies = WC + XC;  // per wave and stage
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nst) copy_stage(i);
  for (int st = 0; st < nst; ++st) {
#ifdef MM_DEBUG_FULL_SYNC
    // race-check build: every copy drained before the stage is read, and
    // every wave past its reads before the next copy is issued
    skinny_wait<kCopies, 0>(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    compute(st);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + NS - 1 < nst) copy_stage(st + NS - 1);
#else
    // stage st's copies are done when at most those of the stages after it
    // remain (a plain barrier: a fence here would wait for every copy)
    skinny_wait<kCopies, NS - 2>(min(NS - 2, nst - 1 - st));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + NS - 1 < nst) copy_stage(st + NS - 1);
    compute(st);
#endif
  }

  // the waves' k parts meet in LDS: waves 1..3 store, wave 0 adds in order
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < NA; ++a) red[((wave - 1) * NA + a) * 64 + lane] = acc[a];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const f32x4 v = red[(q * NA + a) * 64 + lane];
      acc[a] = f32x4{acc[a][0] + v[0], acc[a][1] + v[1], acc[a][2] + v[2], acc[a][3] + v[3]};
    }
  }
  // lane (lx, lk) holds rows 16 b + 4 lk + i, i = 0..3, of column
  // n0 + 16 c + lx
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int n = (int)n0 + 16 * c + lx;
    if (n >= N) continue;
#pragma unroll
    for (int b = 0; b < XB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * b + 4 * lk + i;
        if (m >= M) continue;
        if (p.slices > 1)
          p.part[((int64_t)s * M + m) * N + n] = acc[b * CB + c][i];
        else
          skinny_store(p, m, n, acc[b * CB + c][i]);
      }
    }
  }
}

// Second launch of a split skinny product: each output is the sum of its S
// slices in k order, then the epilogue and one rounding.  A thread takes
// four consecutive outputs (one 16-byte load per slice when M*N is a
// multiple of 4).
__global__ void __launch_bounds__(256) skinny_reduce(SkinnyParams p) {
  // 64-bit positions: M * N may pass 2^31 (32 rows of a vocabulary-sized N)
  const int64_t mn = (int64_t)p.M * p.N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  if ((mn & 3) == 0) {
    // every slice's load issued before the first add: one memory latency
    f32x4 w[kSkinnyMaxSlices];
#pragma unroll
    for (int s = 0; s < kSkinnyMaxSlices; ++s)
      if (s < p.slices) w[s] = *reinterpret_cast<const f32x4*>(p.part + s * mn + i);
    f32x4 v = w[0];
#pragma unroll
    for (int s = 1; s < kSkinnyMaxSlices; ++s)
      if (s < p.slices) v = f32x4{v[0] + w[s][0], v[1] + w[s][1], v[2] + w[s][2], v[3] + w[s][3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) skinny_store(p, (int)((i + e) / p.N), (int)((i + e) % p.N), v[e]);
    return;
  }
  for (int e = 0; e < 4 && i + e < mn; ++e) {
    float v = p.part[i + e];
    for (int s = 1; s < p.slices; ++s) v += p.part[s * mn + i + e];
    skinny_store(p, (int)((i + e) / p.N), (int)((i + e) % p.N), v);
  }
}

}  // namespace mmk
