// mm_api.hip -- the C ABI of libmm.so (declared in include/mm.h): argument
// validation, tile-configuration choice, kernel selection and launch.
//
// The pages' scheduler rejects schedules it cannot run instead of producing a
// wrong kernel (PR "Implement persistent matmul scheduling", reviewer guide:
// split-K and stream-K persistent schedules are refused with a check; PR
// "Translate MmaOp patterns properly on Hopper", commit list: compile-time
// reject reasons).  Here every unsupported request returns a status code
// before any HIP call, and the heuristic can be replaced by an explicit
// configuration (mm_set_config), as the pages' heuristic plugin replaces the
// default heuristic (same PR, review of MatmulSchedulerPluginTest).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mm.h"
#include "gemm_kernel.hpp"
#include "gemm_nt_pipe.hpp"
#include "gemm_pingpong.hpp"
#include "gemm_ws.hpp"
#include "gemm_pp.hpp"
#include "gemm_nt_slab.hpp"
#include "gemm_small.hpp"
#include "gemm_skinny.hpp"

// Split-K partial tiles of mm_matmul_noalloc: a fixed device array instead of
// a caller's workspace, for callers that cannot allocate.  64 MiB = one
// 256 x 256 fp32 slot for each of 256 workgroups (a chunk-major split on a
// 256-CU GPU).  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: the host uses the address hipGetSymbolAddress returns
// for the current device.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {

thread_local std::string g_last_error;

mm_status fail(mm_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

// ----------------------------------------------------------------------------
// Kernel registry: every instantiated (tile, wave grid, layout, form).
// ----------------------------------------------------------------------------
struct KernelEntry {
  int bm, bn, wgm, wgn;
  bool a_kc, b_kc, ffn;
  int pipe;  // 6: 64 x 64 tiles with all of K in LDS (gemm_small),
             // 5: two-group ping-pong (gemm_pp), 4: wave-specialized (gemm_ws),
             // 3: whole-line slab ring (gemm_nt_slab),
             // 2: ping-pong (gemm_pingpong),
             // 1: K-contiguous pipeline (gemm_nt_pipe), 0: gemm_persistent
  const void* fn;
  std::atomic<int> occupancy;  // resident workgroups per CU, 0 = not queried
  bool splitk = false;         // gemm_nt_slab<..., SPLITK>: needs a workspace
  bool pre = false;            // gemm_nt_slab<..., PRE>: stores the pre-activation too
  bool bstage = false;         // gemm_nt_slab<..., BSTAGE>: stages the bias through LDS
  bool ragged = false;         // gemm_nt_slab<..., RAGGED>: K not a multiple of 64
};

#define MM_K(BM, BN, WGM, WGN, AKC, BKC, FFN)                                              \
  {BM, BN, WGM, WGN, AKC, BKC, FFN, 0,                                                     \
   reinterpret_cast<const void*>(&mmk::gemm_persistent<BM, BN, WGM, WGN, AKC, BKC, FFN>), {0}}

#define MM_KP(BM, BN, WGM, WGN, FFN)                                                       \
  {BM, BN, WGM, WGN, true, true, FFN, 1,                                                   \
   reinterpret_cast<const void*>(&mmk::gemm_nt_pipe<BM, BN, WGM, WGN, FFN>), {0}}

#define MM_KPP(FFN)                                                                        \
  {256, 256, 2, 4, true, true, FFN, 2,                                                     \
   reinterpret_cast<const void*>(&mmk::gemm_pingpong<FFN>), {0}}

#define MM_KS(FFN)                                                                         \
  {256, 256, 2, 2, true, true, FFN, 3,                                                     \
   reinterpret_cast<const void*>(&mmk::gemm_nt_slab<256, 256, 2, 2, FFN>), {0}}

// split-K pieces, one instance per operand storage (K-contiguous or not)
#define MM_KSK(AKC, BKC)                                                                   \
  {256, 256, 2, 2, AKC, BKC, false, 3,                                                     \
   reinterpret_cast<const void*>(&mmk::gemm_nt_slab<256, 256, 2, 2, false, true, false, !(BKC), !(AKC)>), \
   {0}, true}

// split-K pieces on 256 x 192 or 256 x 128 tiles (K-contiguous operands): for
// products whose 256 x 256 tiles, split, would leave much of the grid idle
#define MM_KSKW(BN)                                                                        \
  {256, BN, 2, 2, true, true, false, 3,                                                    \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, BN, 2, 2, false, true, false, false, false, false>),        \
   {0}, true}

// the same pieces for a K that is not a multiple of 64 (the chunk holding the
// last super-step masks its partial copies)
#define MM_KSKR(AKC, BKC)                                                                  \
  {256, 256, 2, 2, AKC, BKC, false, 3,                                                     \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, 256, 2, 2, false, true, false, !(BKC), !(AKC), false, true>), \
   {0}, true, false, false, true}
#define MM_KSKWR(BN)                                                                       \
  {256, BN, 2, 2, true, true, false, 3,                                                    \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, BN, 2, 2, false, true, false, false, false, false, true>),  \
   {0}, true, false, false, true}

#define MM_KSP()                                                                           \
  {256, 256, 2, 2, true, true, false, 3,                                                   \
   reinterpret_cast<const void*>(&mmk::gemm_nt_slab<256, 256, 2, 2, false, false, true>), {0}, \
   false, true}

// [K][N] weights and/or [K][M] activations (MM_NN, MM_TN, MM_TT): the slab kernel
// with transpose-read fragments for the operands stored that way
#define MM_KSKN(AKC, BKC)                                                                  \
  {256, 256, 2, 2, AKC, BKC, false, 3,                                                     \
   reinterpret_cast<const void*>(&mmk::gemm_nt_slab<256, 256, 2, 2, false, false, false, !(BKC), !(AKC)>), {0}}

// the single-weight linear / plain form on 256 x 192 or 256 x 128 tiles
// (K-contiguous)
#define MM_KSW(BN)                                                                         \
  {256, BN, 2, 2, true, true, false, 3,                                                    \
   reinterpret_cast<const void*>(&mmk::gemm_nt_slab<256, BN, 2, 2, false>), {0}}

// K not a multiple of 64 (256 x 192 / 256 x 128 tiles and the FFN for
// K-contiguous operands only)
#define MM_KSR(BN, FFN)                                                                    \
  {256, BN, 2, 2, true, true, FFN, 3,                                                      \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, BN, 2, 2, FFN, false, false, false, false, false, true>),   \
   {0}, false, false, false, true}
#define MM_KSRKN(AKC, BKC)                                                                 \
  {256, 256, 2, 2, AKC, BKC, false, 3,                                                     \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, 256, 2, 2, false, false, false, !(BKC), !(AKC), false, true>), \
   {0}, false, false, false, true}

// the plain linear form with the bias brought into LDS under the K loop
#define MM_KSB()                                                                           \
  {256, 256, 2, 2, true, true, false, 3,                                                   \
   reinterpret_cast<const void*>(                                                          \
       &mmk::gemm_nt_slab<256, 256, 2, 2, false, false, false, false, false, true>),       \
   {0}, false, false, true}

#define MM_KWS()                                                                           \
  {256, 128, 2, 4, true, true, false, 4, reinterpret_cast<const void*>(&mmk::gemm_ws), {0}}

#define MM_KPPT()                                                                          \
  {256, 128, 2, 4, true, true, false, 5, reinterpret_cast<const void*>(&mmk::gemm_pp), {0}}

#define MM_KSM(AKC, BKC)                                                                   \
  {64, 64, 2, 2, AKC, BKC, false, 6, reinterpret_cast<const void*>(&mmk::gemm_small<AKC, BKC>), {0}}

#define MM_K_LAYOUTS(BM, BN, WGM, WGN)                                                      \
  MM_K(BM, BN, WGM, WGN, true, false, false), MM_K(BM, BN, WGM, WGN, true, true, false),   \
      MM_K(BM, BN, WGM, WGN, false, false, false), MM_K(BM, BN, WGM, WGN, false, true, false)

KernelEntry g_kernels[] = {
    MM_KSKN(true, false),
    MM_KSKN(false, false),
    MM_KSKN(false, true),
    MM_KSK(true, true),
    MM_KSK(true, false),
    MM_KSK(false, false),
    MM_KSK(false, true),
    MM_KSKW(192),
    MM_KSKW(128),
    MM_KSKR(true, true),
    MM_KSKR(true, false),
    MM_KSKR(false, false),
    MM_KSKR(false, true),
    MM_KSKWR(192),
    MM_KSKWR(128),
    MM_KSP(),
    MM_KSB(),
    MM_KWS(),
    MM_KPPT(),
    MM_KS(false),
    MM_KS(true),
    MM_KSW(192),
    MM_KSW(128),
    MM_KSR(256, false),
    MM_KSR(192, false),
    MM_KSR(128, false),
    MM_KSR(256, true),
    MM_KSRKN(true, false),
    MM_KSRKN(false, false),
    MM_KSRKN(false, true),
    MM_KPP(false),
    MM_KPP(true),
    MM_KP(256, 256, 2, 4, false),
    MM_KP(256, 256, 4, 2, false),
    MM_KP(256, 256, 2, 4, true),
    MM_KP(256, 256, 4, 2, true),
    MM_KP(256, 256, 2, 2, false),
    MM_KP(128, 128, 2, 2, false),
    MM_KP(256, 256, 2, 2, true),
    MM_KP(128, 256, 2, 2, true),
    MM_KP(128, 128, 2, 2, true),
    MM_K_LAYOUTS(256, 256, 2, 2),
    MM_K_LAYOUTS(128, 128, 2, 2),
    MM_K_LAYOUTS(64, 64, 2, 2),
    MM_KSM(true, false),
    MM_KSM(true, true),
    MM_KSM(false, false),
    MM_KSM(false, true),
    MM_K(256, 256, 2, 2, true, true, true),
    MM_K(128, 256, 2, 2, true, true, true),
    MM_K(128, 128, 2, 2, true, true, true),
};

KernelEntry* find_kernel(int bm, int bn, int wgm, int wgn, bool a_kc, bool b_kc, bool ffn, int pipe,
                         bool splitk = false, bool pre = false, bool bstage = false, bool ragged = false) {
  for (auto& k : g_kernels)
    if (k.bm == bm && k.bn == bn && k.wgm == wgm && k.wgn == wgn && k.a_kc == a_kc &&
        k.b_kc == b_kc && k.ffn == ffn && k.pipe == pipe && k.splitk == splitk && k.pre == pre &&
        k.bstage == bstage && k.ragged == ragged)
      return &k;
  return nullptr;
}

// ----------------------------------------------------------------------------
// Configuration: heuristic and override.
// ----------------------------------------------------------------------------
struct Config {
  int bm = 256, bn = 256, wgm = 2, wgn = 2;
  int group = 8;  // band height in tiles
  int xcd = 1;    // XCD-aware remap
  int kalt = 2;   // 0 never, 1 always, 2 automatic
  int grid = 0;   // 0 = CUs x occupancy
  int pipe = 3;   // preferred kernel family: 5 two-group ping-pong, 4 wave-specialized (both
                  // BN=128, WN=4), 3 slab ring, 2 split-phase, 1 pipeline, 0 basic
  int sk = 0;     // split-K slices when a workspace is given: 0 automatic, 1 off, n forced
  int bstage = 0; // 1: linear forms with a bias take the slab instance that stages it in LDS
  bool forced = false;  // set by mm_set_config / MM_FORCE_CONFIG (not by the heuristic)
};

std::mutex g_cfg_mu;
bool g_cfg_forced = false;
Config g_cfg_force;
std::once_flag g_env_once;

bool parse_config(const char* spec, Config* out) {
  Config c;
  std::string s(spec);
  size_t pos = 0;
  while (pos < s.size()) {
    size_t end = s.find(',', pos);
    if (end == std::string::npos) end = s.size();
    std::string item = s.substr(pos, end - pos);
    pos = end + 1;
    if (item.empty()) continue;
    size_t eq = item.find('=');
    if (eq == std::string::npos) return false;
    std::string key = item.substr(0, eq);
    char* ep = nullptr;
    long v = std::strtol(item.c_str() + eq + 1, &ep, 10);
    if (ep == item.c_str() + eq + 1 || *ep != '\0' || v < 0 || v > (1 << 20)) return false;
    if (key == "BM") c.bm = (int)v;
    else if (key == "BN") c.bn = (int)v;
    else if (key == "WM") c.wgm = (int)v;
    else if (key == "WN") c.wgn = (int)v;
    else if (key == "G") c.group = (int)v;
    else if (key == "XCD") c.xcd = (int)v;
    else if (key == "KALT") c.kalt = (int)v;
    else if (key == "GRID") c.grid = (int)v;
    else if (key == "PIPE") c.pipe = (int)v;
    else if (key == "SK") c.sk = (int)v;
    else if (key == "BSTAGE") c.bstage = (int)v;
    else return false;
  }
  if (c.group < 1 || c.xcd > 1 || c.kalt > 2 || c.pipe > 5 || c.sk > 64 || c.bstage > 1) return false;
  // the tile shape must be one that is instantiated (for some layout/form)
  bool any = false;
  for (auto& k : g_kernels)
    if (k.bm == c.bm && k.bn == c.bn && k.wgm == c.wgm && k.wgn == c.wgn) any = true;
  if (!any) return false;
  *out = c;
  return true;
}

void read_env_once() {
  std::call_once(g_env_once, [] {
    const char* e = std::getenv("MM_FORCE_CONFIG");
    if (e && *e) {
      Config c;
      if (parse_config(e, &c)) {
        std::lock_guard<std::mutex> g(g_cfg_mu);
        g_cfg_forced = true;
        g_cfg_force = c;
      } else {
        std::fprintf(stderr, "libmm: ignoring invalid MM_FORCE_CONFIG=\"%s\"\n", e);
      }
    }
  });
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The heuristic: the largest tile that still gives about a wave of work.
// Band height 4: a wave of 256 workgroups puts 32 consecutive tiles of the
// band order on each XCD, a 4 x 8 block (12 panels, as few as 8 x 4 reads);
// measured against 8 (three same-box alternations each): 4096^3
// linear+bias+GELU 99.8 -> 98.4 us, FFN 8192x14336x4096 1242.7 -> 1239.4 us,
// 8192^3 695.0 -> 694.3 us.
Config heuristic(bool ffn, int64_t M, int64_t N, int64_t K) {
  Config c;
  c.group = 4;
  if (ffn) {
    // B tile = gate + up rows, output tile BM x BN/2
    if (cdiv(M, 256) * cdiv(N, 128) >= 192) {
      c.bm = 256; c.bn = 256;
    } else if (cdiv(M, 128) * cdiv(N, 128) >= 128) {
      c.bm = 128; c.bn = 256;
    } else {
      c.bm = 128; c.bn = 128;
    }
  } else {
    // 256 x 256 tiles once they occupy half of the CUs: at 3072^3 (144 tiles)
    // linear + bias + GELU took 56.2 us on them against 112.5 us on 128 x 128
    // tiles (the 32-k pipeline); at 2560^3 (100 tiles) 48.5 against 49.4; at
    // 2048^3 (64 tiles) 40.7 against 25.9
    if (cdiv(M, 256) * cdiv(N, 256) >= 128) {
      c.bm = 256; c.bn = 256;
    } else if (cdiv(M, 128) * cdiv(N, 128) >= 64) {
      c.bm = 128; c.bn = 128;
    } else {
      c.bm = 64; c.bn = 64;
    }
  }
  (void)K;
  return c;
}

Config choose_config(bool ffn, int64_t M, int64_t N, int64_t K) {
  read_env_once();
  {
    std::lock_guard<std::mutex> g(g_cfg_mu);
    if (g_cfg_forced) {
      Config c = g_cfg_force;
      c.forced = true;
      return c;
    }
  }
  return heuristic(ffn, M, N, K);
}

// Band height that makes each XCD's share of a launch the most compact block
// of tiles: an XCD runs `per` consecutive tiles of the band order, which with
// band height g form a g x per/g block whose panels number g + per/g (the
// smallest such g).  2047 x 3001 x 65536 split in 2 (96 tiles of 8 x 12, 24
// workgroups per XCD): g = 4 gives 4 x 6 blocks (10 panels) instead of 8 x 3
// (11 panels): 644.3 -> 633.0 us per call (same-box A/B, three alternations).
int compact_band(int64_t per, int64_t tiles_m) {
  int best = 1;
  int64_t cost = INT64_MAX;
  for (int g = 1; g <= tiles_m && g <= 64; ++g) {
    const int64_t c = g + cdiv(per, g);
    if (c < cost) {
      cost = c;
      best = g;
    }
  }
  return best;
}

// K-direction alternation pays off once one tile's K panels no longer stay
// resident in an XCD's L2 (4 MiB) across tiles.
bool k_alt_enabled(const Config& c, int64_t K) {
  if (c.kalt != 2) return c.kalt == 1;
  return K * (int64_t)(c.bm + c.bn) * 2 > (int64_t)(2 << 20);
}

// ----------------------------------------------------------------------------
// Device attributes (cached per device).
// ----------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

mm_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MM_ERR_UNSUPPORTED, "device index out of range");
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0)
      return fail(MM_ERR_HIP, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return MM_OK;
}

// Device address of the static scratch on the current device, taken once per
// device with that device current (each GPU holds its own copy of the array
// at its own address).
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mm_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MM_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MM_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MM_OK;
}

mm_status kernel_occupancy(KernelEntry* k, int* occ) {
  int o = k->occupancy.load(std::memory_order_relaxed);
  if (o == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k->fn, k->wgm * k->wgn * 64, 0);
    if (e != hipSuccess)
      return fail(MM_ERR_HIP, std::string("hipOccupancyMaxActiveBlocksPerMultiprocessor: ") +
                                  hipGetErrorString(e));
    if (o < 1) return fail(MM_ERR_UNSUPPORTED, "kernel cannot be resident on a CU");
    k->occupancy.store(o, std::memory_order_relaxed);
  }
  *occ = o;
  return MM_OK;
}

// ----------------------------------------------------------------------------
// Validation and launch.
// ----------------------------------------------------------------------------
struct Request {
  const void* A;
  const void* B;
  const void* B2;
  const void* bias;
  void* out;
  int64_t M, N, K;
  int layout;
  int epi;  // mmk::EPI_*
  bool out_f32;
  bool ffn;
  void* ws = nullptr;     // caller's workspace (split-K), may be null
  int64_t ws_bytes = 0;
  int64_t batch = 1;      // batched form: entries and their element strides
  int64_t stride_a = 0, stride_b = 0, stride_out = 0;
  void* out_pre = nullptr;  // second output: the pre-activation (GELU epilogues)
  bool static_ws = false;   // ws is the library's static scratch (mm_matmul_noalloc)
};

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

mm_status validate(const Request& r) {
  if (r.M < 0 || r.N < 0 || r.K < 0) return fail(MM_ERR_INVALID_VALUE, "negative size");
  if (r.batch < 1) return fail(MM_ERR_INVALID_VALUE, "batch must be >= 1");
  if (r.stride_a < 0 || r.stride_b < 0 || r.stride_out < 0)
    return fail(MM_ERR_INVALID_VALUE, "negative batch stride");
  if (r.M >= (int64_t(1) << 31) || r.N >= (int64_t(1) << 31) || r.K >= (int64_t(1) << 31))
    return fail(MM_ERR_UNSUPPORTED, "M, N and K must be below 2^31");
  if (r.layout < MM_NN || r.layout > MM_TT) return fail(MM_ERR_INVALID_VALUE, "bad layout");
  if (r.M == 0 || r.N == 0) return MM_OK;
  // K == 0: the operands hold no elements and are never read (they may be
  // null); the output is the epilogue of an empty sum (empty_k_fill)
  const bool reads = r.K > 0;
  if (!r.out || (reads && (!r.A || !r.B))) return fail(MM_ERR_INVALID_VALUE, "null operand pointer");
  if (reads && r.ffn && !r.B2) return fail(MM_ERR_INVALID_VALUE, "null W_up pointer");
  const bool need_bias = (r.epi == mmk::EPI_BIAS || r.epi == mmk::EPI_BIAS_GELU);
  if (need_bias && !r.bias) return fail(MM_ERR_INVALID_VALUE, "epilogue needs a bias");
  const bool a_kc = (r.layout == MM_NN || r.layout == MM_NT);
  const bool b_kc = (r.layout == MM_NT || r.layout == MM_TT);
  if (reads && (!aligned(r.A, 16) || !aligned(r.B, 16) || (r.ffn && !aligned(r.B2, 16))))
    return fail(MM_ERR_MISALIGNED, "operand pointers must be 16-byte aligned");
  if (r.batch > 1) {
    if (reads && (r.stride_a % 8 != 0 || r.stride_b % 8 != 0))
      return fail(MM_ERR_MISALIGNED, "operand batch strides must be multiples of 8 elements");
    if (r.stride_out < r.M * r.N)
      return fail(MM_ERR_INVALID_VALUE, "output batch stride smaller than M * N: entries would overlap");
  }
  if (reads && (a_kc ? r.K : r.M) % 8 != 0)
    return fail(MM_ERR_MISALIGNED, "the contiguous extent of A must be a multiple of 8 elements");
  if (reads && (b_kc ? r.K : r.N) % 8 != 0)
    return fail(MM_ERR_MISALIGNED, "the contiguous extent of B must be a multiple of 8 elements");
  if (need_bias && !aligned(r.bias, 2)) return fail(MM_ERR_MISALIGNED, "bias must be 2-byte aligned");
  const int esize = r.out_f32 ? 4 : 2;
  if (!aligned(r.out, esize)) return fail(MM_ERR_MISALIGNED, "out must be aligned to its element size");
  // every extent (over all batch entries) below 2^60 elements, so that the
  // byte counts below cannot overflow
  const int64_t nb = r.batch - 1;
  const int64_t room = int64_t(1) << 60;
  auto fits = [&](int64_t stride, int64_t one) { return one <= room && (nb == 0 || stride <= (room - one) / nb); };
  if (!fits(r.stride_a, r.M * r.K) || !fits(r.stride_b, r.K * r.N) || !fits(r.stride_out, r.M * r.N))
    return fail(MM_ERR_UNSUPPORTED, "an operand or the output spans 2^60 elements or more");
  // byte extents over every batch entry
  const int64_t ob = (nb * r.stride_out + r.M * r.N) * esize;
  const int64_t ab = (nb * r.stride_a + r.M * r.K) * 2, bb = (nb * r.stride_b + r.K * r.N) * 2;
  if (overlaps(r.out, ob, r.A, ab) || overlaps(r.out, ob, r.B, bb) ||
      (r.ffn && overlaps(r.out, ob, r.B2, bb)) ||
      (need_bias && overlaps(r.out, ob, r.bias, r.N * 2)))
    return fail(MM_ERR_INVALID_VALUE, "out overlaps an input");
  if (r.out_pre) {
    if (r.ffn || r.batch != 1 || (r.epi != mmk::EPI_GELU && r.epi != mmk::EPI_BIAS_GELU))
      return fail(MM_ERR_INVALID_VALUE, "a pre-activation output needs an unbatched linear GELU epilogue");
    if (!aligned(r.out_pre, esize))
      return fail(MM_ERR_MISALIGNED, "preact must be aligned to its element size");
    if (overlaps(r.out_pre, ob, r.A, ab) || overlaps(r.out_pre, ob, r.B, bb) ||
        overlaps(r.out_pre, ob, r.out, ob) || (need_bias && overlaps(r.out_pre, ob, r.bias, r.N * 2)))
      return fail(MM_ERR_INVALID_VALUE, "preact overlaps an input or out");
  }
  if (r.ws_bytes < 0) return fail(MM_ERR_INVALID_VALUE, "negative workspace size");
  if (r.ws && (overlaps(r.ws, r.ws_bytes, r.out, ob) || overlaps(r.ws, r.ws_bytes, r.A, ab) ||
               overlaps(r.ws, r.ws_bytes, r.B, bb) ||
               (need_bias && overlaps(r.ws, r.ws_bytes, r.bias, r.N * 2))))
    return fail(MM_ERR_INVALID_VALUE, "workspace overlaps an operand or the output");
  return MM_OK;
}

struct Plan {
  KernelEntry* kernel = nullptr;
  mmk::GemmParams p;
  int grid;
  int threads;
};

// ----------------------------------------------------------------------------
// Split-K / stream-K: the pages name splitting the K loop over workgroups
// (split-K, and stages spread over SMs "a la stream-K") and leave both out of
// their persistent scheduler (PR "Implement persistent matmul scheduling",
// review notes).  Here: when a K-contiguous single-weight product has fewer
// 256 x 256 tiles than the grid has workgroups, each tile's K loop is cut into
// n chunks and the tiles * n chunks are dealt to the resident workgroups
// (one chunk each, or equal contiguous ranges: stream-K); every piece leaves
// its fp32 partial tile in a caller-provided workspace, and a second launch
// (splitk_reduce) adds them in k order.
// ----------------------------------------------------------------------------
constexpr int64_t kSkSlotBytes = 256 * 256 * 4;
constexpr int64_t kSkMaxWgs = 1024;  // bounds the workspace (at most 512 MiB)

// whether op(A) / op(B) are stored K-contiguous
bool a_kcontig(int layout) { return layout == MM_NN || layout == MM_NT; }
bool b_kcontig(int layout) { return layout == MM_NT || layout == MM_TT; }

// ----------------------------------------------------------------------------
// Cost model of the automatic tile and split choices.  Unit: one 64-k
// super-step of 256 x 256 slab tiles on a full grid.  Per-tile costs measured
// on one pass of 256 tiles at K = 2048 and 4096 (linear + bias + GELU, one
// box): a 256 x 192 slab tile 0.79 of a 256 x 256 one, 256 x 128 0.60, a
// 128 x 128 tile of the 32-k pipeline 0.46.  A pass with part of the grid
// idle runs its tiles faster (under the power limit the busy CUs clock
// higher): modelled as 0.6 + 0.4 x the busy fraction (2048^3 on 128 tiles of
// 256 x 128: 23.7-24.7 us against 33.5 for a full pass of them).  A split
// adds its partial tiles' write and read and the output's write at ~5 TB/s:
// one unit (~1.25 us) per 6.25 MB.
// ----------------------------------------------------------------------------
enum TileKind { kTile256 = 0, kTile192 = 1, kTile128 = 2, kPipe128 = 3 };
constexpr double kTileCost[] = {1.0, 0.79, 0.60, 0.46};
constexpr int64_t kModelGrid = 256;          // CUs of the target GPU
constexpr double kBytesPerUnit = 6.25e6;

double pass_units(int64_t tiles) {
  const int64_t full = tiles / kModelGrid, rem = tiles % kModelGrid;
  return (double)full + (rem ? 0.6 + 0.4 * (double)rem / (double)kModelGrid : 0.0);
}

int64_t kind_tiles(const Request& r, int kind) {
  switch (kind) {
    case kTile256: return cdiv(r.M, 256) * cdiv(r.N, 256);
    case kTile192: return cdiv(r.M, 256) * cdiv(r.N, 192);
    case kTile128: return cdiv(r.M, 256) * cdiv(r.N, 128);
    default: return cdiv(r.M, 128) * cdiv(r.N, 128);
  }
}

double unsplit_cost(const Request& r, int kind) {
  return kTileCost[kind] * pass_units(kind_tiles(r, kind)) * (double)cdiv(r.K, mmk::kSlabK);
}

// the narrower slab tiles and the 128 x 128 pipeline: K-contiguous
// single-weight single-output products of at least two super-steps
bool narrow_eligible(const Request& r) {
  return a_kcontig(r.layout) && b_kcontig(r.layout) && !r.ffn && !r.out_pre && r.batch == 1 &&
         r.K >= 2 * mmk::kSlabK && (int64_t)256 * r.K * 2 < (int64_t(1) << 31);
}

// the cheapest unsplit tile kind for a request (256 x 256 when only that runs)
int best_unsplit_kind(const Request& r, double* cost) {
  int best = kTile256;
  double bc = unsplit_cost(r, kTile256);
  if (narrow_eligible(r))
    for (int kind = kTile192; kind <= kPipe128; ++kind) {
      const double c = unsplit_cost(r, kind);
      if (c < bc) {
        bc = c;
        best = kind;
      }
    }
  if (cost) *cost = bc;
  return best;
}

// single-output products of one weight (plain or linear; the reduction
// applies the bias and GELU to the summed value) in the slab kernel's domain:
// at least two super-steps (the last may be partial), and 32-bit offsets
// within a tile's K-contiguous rows and a super-step's k-rows of an operand
// stored [K][M] / [K][N]
bool splitk_shape(const Request& r) {
  return r.batch == 1 && !r.ffn && !r.out_pre && r.K >= 2 * mmk::kSlabK &&
         (int64_t)256 * r.K * 2 < (int64_t(1) << 31) &&
         (a_kcontig(r.layout) || (int64_t)mmk::kSlabK * r.M * 2 < (int64_t(1) << 31)) &&
         (b_kcontig(r.layout) || (int64_t)mmk::kSlabK * r.N * 2 < (int64_t(1) << 31));
}

struct SkPlan {
  int n = 1;        // chunks per tile (1 = no split)
  int q = 0;        // chunks per workgroup range; 0 = chunk-major, one per workgroup
  int64_t wgs = 0;  // workgroups with work (the grid)
  int bn = 256;     // tile width: 256, or 192 / 128 (K-contiguous operands)
};

// Chunks and their dealing for `wgs` resident workgroups.  Automatic: only
// when every tile can take two chunks (2 T <= wgs), dealt chunk-major, one
// per workgroup: workgroups running side by side then read the same k range
// of neighbouring tiles' panels.  Dealt tile-major in ranges (stream-K), the
// k positions of neighbouring workgroups no longer match and their L2
// sharing is lost: 2047 x 3001 x 65536 (96 tiles on 256 CUs) 720 us
// chunk-major vs 785 us in ranges of 3/8 of a tile; 3584 x 3584 x 16384
// (196 tiles) 320 us unsplit vs 538 us in ranges of 7/8 of a tile.  Stream-K
// stays available through a forced chunk count (SK=n with n T > wgs).
SkPlan splitk_plan_bn(const Request& r, const Config& c, int64_t wgs, int bn) {
  SkPlan sp;
  sp.bn = bn;
  if (c.sk == 1 || !splitk_shape(r) || wgs > kSkMaxWgs) return sp;
  const int64_t T = cdiv(r.M, 256) * cdiv(r.N, bn);
  const int64_t KS = cdiv(r.K, mmk::kSlabK);
  int n;
  if (c.sk >= 2) {
    n = c.sk;
    if (KS / n < 2) return sp;  // a piece runs at least two super-steps
  } else if (2 * T <= wgs) {
    // fewest chunks that occupy three quarters of the grid: more chunks read
    // the operands from more places at once and were slower (2 chunks 745 us,
    // 4: 941, 5: 849, 8: 948, 16: 1287; unsplit 1165)
    n = (int)cdiv(3 * wgs, 4 * T);
    if (n > 16) n = 16;
    while (n > 2 && (KS / n < 32 || n * T > wgs)) --n;
    // a piece runs at least 32 super-steps (K >= 2048): shorter K loops do not
    // pay for the partial tiles and the second launch (linear + bias + GELU
    // at 2048^3: 39.5 us split in three against 25.9 unsplit; 1000 x 3001 x
    // 2048 in four: 34.1 against 28.2; 256^3 in two: 16.5 against 10.9),
    // longer ones do (1024 x 8192 x 8192 in two: 117.5 against 151.8)
    if (KS / n < 32) return sp;
  } else {
    return sp;
  }
  sp.n = n;
  if (n * T <= wgs) {  // chunk-major, one chunk per workgroup
    sp.q = 0;
    sp.wgs = n * T;
    return sp;
  }
  const int64_t q = cdiv(T * n, wgs);
  if (q >= n) return SkPlan();  // every range would be a whole tile
  sp.q = (int)q;
  sp.wgs = cdiv(T * n, q);
  return sp;
}

// The automatic split weighs every chunk-major plan -- tile width 256, and
// 192 or 128 for K-contiguous operands; 2 to 16 chunks per tile, each of at
// least 8 super-steps, all chunks resident at once -- by the cost model
// against the cheapest unsplit run, and takes the cheapest, or none.  The
// 2047 x 3001 x 65536 fp32 matmul splits in 2 on 128 tiles of 256 x 192 (all
// 256 CUs; 96 tiles of 256 x 256 in 2 chunks would leave 64 idle);
// 1024 x 4096 x 4096 stays unsplit (38.8-42.6 us; split in 2 on 256 x 256 or
// 256 x 192 tiles, 55 us), and so does every K below ~2048 at these sizes (the
// pieces' partial tiles cost more than the fuller grid gains).  A forced
// configuration (or chunk count) keeps 256 x 256 tiles and the rule of
// splitk_plan_bn.
SkPlan splitk_plan(const Request& r, const Config& c, int64_t wgs) {
  if (c.forced || c.sk >= 2) return splitk_plan_bn(r, c, wgs, 256);
  SkPlan best;  // n = 1: no split
  if (c.sk == 1 || !splitk_shape(r) || wgs > kSkMaxWgs) return best;
  double best_cost = 0.0;
  best_unsplit_kind(r, &best_cost);
  const int64_t KS = cdiv(r.K, mmk::kSlabK);
  const int widths[] = {256, 192, 128};
  for (int i = 0; i < 3; ++i) {
    if (i > 0 && !narrow_eligible(r)) break;
    const int bn = widths[i];
    const int64_t T = cdiv(r.M, 256) * cdiv(r.N, bn);
    for (int n = 2; n <= 16 && n * T <= wgs && KS / n >= 8; ++n) {
      const double bytes = 2.0 * (double)(n * T) * 256.0 * bn * 4.0 +
                           (double)r.M * (double)r.N * (r.out_f32 ? 4.0 : 2.0);
      const double cost = kTileCost[i] * pass_units(n * T) * (double)cdiv(KS, n) + bytes / kBytesPerUnit;
      if (cost < best_cost) {
        best_cost = cost;
        best.n = n;
        best.q = 0;
        best.wgs = n * T;
        best.bn = bn;
      }
    }
  }
  return best;
}

// one slot per chunk-major workgroup; two per stream-K workgroup (its range
// may end one tile and start the next)
int64_t splitk_ws_bytes(const SkPlan& sp) {
  if (sp.n <= 1) return 0;
  return (sp.q == 0 ? 1 : 2) * sp.wgs * kSkSlotBytes;
}

// Work units of a split-K launch are dealt to this many workgroups: one wave
// of resident workgroups (no workgroup waits for another, so residency is a
// matter of speed only).
int64_t splitk_wgs(const Config& c, int cus, int occ) {
  const int64_t resident = (int64_t)cus * occ;
  return c.grid > 0 && c.grid < resident ? c.grid : resident;
}


// Everything but the device-dependent grid size; no HIP calls.
mm_status plan_host(const Request& r, const Config& c_in, Plan* pl, const SkPlan& sp = SkPlan()) {
  const bool sk = sp.n > 1;
  const bool a_kc = (r.layout == MM_NN || r.layout == MM_NT);
  const bool b_kc = (r.layout == MM_NT || r.layout == MM_TT);
  if (r.ffn && !b_kc) return fail(MM_ERR_UNSUPPORTED, "FFN weights must be [N][K]");
  Config c = c_in;
  KernelEntry* k = nullptr;
  if (sk) {
    c.bm = 256;
    c.bn = sp.bn;
    c.wgm = c.wgn = 2;
    k = find_kernel(256, sp.bn, 2, 2, a_kc, b_kc, false, 3, true, false, false, r.K % mmk::kSlabK != 0);
  }
  // the wave-specialized kernel (a configuration override for comparison)
  // takes single-weight K-contiguous products with whole super-steps; other
  // shapes run the default tile under that override
  // as does the two-group ping-pong kernel
  if ((c.pipe == 4 || c.pipe == 5) &&
      !(b_kc && a_kc && !r.ffn && r.batch == 1 && !r.out_pre && !sk && r.K % mmk::kSlabK == 0 &&
        r.K >= 2 * mmk::kSlabK && (int64_t)256 * r.K * 2 < (int64_t(1) << 31))) {
    c.bm = c.bn = 256;
    c.wgm = c.wgn = 2;
    c.pipe = 3;
  }
  // 64 x 64 tiles of a short K take the kernel that holds all of K in LDS
  // (one global round trip per tile instead of one per 64-k step); the
  // basic kernel's own family (PIPE=0) keeps the basic kernel
  if (!sk && !r.ffn && c.bm == 64 && c.bn == 64 && c.wgm == 2 && c.wgn == 2 && c.pipe != 0 &&
      r.K <= mmk::kSmallKMax)
    k = find_kernel(64, 64, 2, 2, a_kc, b_kc, false, 6);
  // 256 x 192 and 256 x 128 slab tiles exist for the K-contiguous
  // single-weight single-output form only; other requests under such a
  // configuration run 256 x 256 tiles
  const bool narrow = c.bn == 192 || (c.bm == 256 && c.bn == 128 && c.wgm == 2 && c.wgn == 2 && c.pipe == 3);
  if (!sk && narrow &&
      !(a_kc && b_kc && !r.ffn && !r.out_pre && r.K >= 2 * mmk::kSlabK &&
        (int64_t)256 * r.K * 2 < (int64_t(1) << 31))) {
    c.bm = c.bn = 256;
    c.wgm = c.wgn = 2;
  }
  // the pipelined kernels address a tile's rows with 32-bit buffer offsets
  const int64_t span = (int64_t)(c.bm > c.bn ? c.bm : c.bn) * r.K * 2;
  for (int fam = c.pipe; fam >= 0 && !k && !sk; --fam) {
    if (fam > 0 && span >= (int64_t(1) << 31)) continue;
    // the batched form and the pre-activation output run on the slab and
    // basic kernels
    if ((r.batch > 1 || r.out_pre) && (fam == 1 || fam == 2)) continue;
    // the ping-pong and wave-specialized kernels only under their own
    // configuration (fam == c.pipe), never as another family's fallback
    if ((fam == 4 || fam == 5) && fam != c.pipe) continue;
    // the slab kernel runs super-steps of 64 k, two of them in flight; a K
    // that is not a multiple of 64 takes its RAGGED instance (single-output
    // products: the last super-step reads zeros past K)
    const bool ragged = fam == 3 && r.K % mmk::kSlabK != 0;
    if (fam == 3 && r.K < 2 * mmk::kSlabK) continue;
    if (ragged && r.out_pre) continue;
    // its [K][N]-weight and [K][M]-activation forms address a super-step's
    // 64 k-rows of such an operand with 32-bit buffer offsets
    if (fam == 3 && !b_kc && (int64_t)mmk::kSlabK * r.N * 2 >= (int64_t(1) << 31)) continue;
    if (fam == 3 && !a_kc && (int64_t)mmk::kSlabK * r.M * 2 >= (int64_t(1) << 31)) continue;
    // the bias-staging instance: K-contiguous single-weight linear forms
    // with a bias epilogue, when the configuration asks for it
    const bool bstage = fam == 3 && c.bstage && c.bn == 256 && a_kc && b_kc && !r.ffn && !r.out_pre && r.batch == 1 &&
                        !ragged && (r.epi == mmk::EPI_BIAS || r.epi == mmk::EPI_BIAS_GELU);
    k = find_kernel(c.bm, c.bn, c.wgm, c.wgn, a_kc, b_kc, r.ffn, fam, false, fam == 3 && r.out_pre, bstage,
                    ragged);
  }
  // layouts a wave grid is not built for run the 2 x 2 kernel of the same tile
  if (!k) k = find_kernel(c.bm, c.bn, 2, 2, a_kc, b_kc, r.ffn, 0);
  if (!k) return fail(MM_ERR_UNSUPPORTED, "no kernel for this tile configuration, layout and form");
  const int out_bn = r.ffn ? c.bn / 2 : c.bn;
  mmk::GemmParams& p = pl->p;
  std::memset(&p, 0, sizeof p);
  p.A = static_cast<const uint16_t*>(r.A);
  p.B = static_cast<const uint16_t*>(r.B);
  p.B2 = static_cast<const uint16_t*>(r.B2);
  p.bias = static_cast<const uint16_t*>(r.bias);
  p.out = r.out;
  p.out_pre = r.out_pre;
  p.M = (int)r.M;
  p.N = (int)r.N;
  p.K = (int)r.K;
  p.epi = r.epi;
  p.out_f32 = r.out_f32 ? 1 : 0;
  const int esize = r.out_f32 ? 4 : 2;
  p.out_vec = (aligned(r.out, 16) && (r.N * esize) % 16 == 0 &&
               (r.batch == 1 || (r.stride_out * esize) % 16 == 0) &&
               (!r.out_pre || aligned(r.out_pre, 16))) ? 1 : 0;
  const int64_t tm = cdiv(r.M, c.bm), tn = cdiv(r.N, out_bn);
  if (tm * tn * r.batch >= (int64_t(1) << 31)) return fail(MM_ERR_UNSUPPORTED, "too many tiles");
  p.batch = (int)r.batch;
  p.stride_a = r.stride_a;
  p.stride_b = r.stride_b;
  p.stride_out = r.stride_out;
  p.tiles_m = (int)tm;
  p.tiles_n = (int)tn;
  p.num_tiles = (int)(tm * tn);
  // the pipelined kernel runs k-steps of 32 in pairs: an even count, padded
  // with k-steps past K that read zeros
  p.k_tiles = k->pipe >= 3 ? (int)cdiv(r.K, mmk::kSlabK)
             : k->pipe == 2 ? (int)cdiv(r.K, mmk::kPipeBK)
             : k->pipe == 1 ? (int)(2 * cdiv(r.K, 2 * mmk::kPipeBK))
                            : (int)cdiv(r.K, mmk::kBK);
  // A band taller than the tile rows is one band of all of them: clamped,
  // the order is the same and tile_coords' band = group_m * tiles_n stays
  // below the tile count (< 2^31) instead of wrapping for a forced G.
  p.group_m = (int)(c.group < tm ? c.group : tm);
  p.xcd_remap = c.xcd;
  p.k_alt = k_alt_enabled(c, r.K) ? 1 : 0;
  p.sk_chunks = 1;
  if (sk) {
    p.k_alt = 0;
    p.sk_chunks = sp.n;
    p.sk_items = sp.q;
    p.sk_part = static_cast<float*>(r.ws);
  }
  pl->kernel = k;
  pl->threads = k->wgm * k->wgn * 64;  // the selected kernel's block size
  pl->grid = 0;
  return MM_OK;
}

// The heuristic's configuration for a request, refined by the cost model for
// K-contiguous single-weight products where the heuristic picked 256 x 256 or
// 128 x 128 tiles: the cheapest of 256 x 256, 256 x 192 and 256 x 128 slab
// tiles and 128 x 128 pipeline tiles.  8192^3 and 4096^3 keep 256 x 256
// (full passes), 6144^3 and 3072^3 take 256 x 192 (3 full passes against
// 2.25; 192 tiles against 144), 2560^3 and 2048^3 256 x 128 (200 and 128
// tiles: 51.2 -> 33.4 us and 26.2 -> 24.7 us against 128 x 128 pipeline
// tiles).  A forced configuration is kept as it is.
Config choose_config_for(const Request& r) {
  Config c = choose_config(r.ffn, r.M, r.N, r.K);
  if (c.forced || c.wgm != 2 || c.wgn != 2 || c.pipe != 3 || c.bstage) return c;
  if (!((c.bm == 256 && c.bn == 256) || (c.bm == 128 && c.bn == 128)) || !narrow_eligible(r)) return c;
  switch (best_unsplit_kind(r, nullptr)) {
    case kTile256: c.bm = 256; c.bn = 256; break;
    case kTile192: c.bm = 256; c.bn = 192; break;
    case kTile128: c.bm = 256; c.bn = 128; break;
    default: c.bm = 128; c.bn = 128; break;
  }
  return c;
}

// K == 0: one launch of empty_k_fill over every output element
mm_status run_empty_k(const Request& r, void* stream) {
  mmk::EmptyKParams p;
  p.bias = static_cast<const uint16_t*>(r.bias);
  p.out = r.out;
  p.out_pre = r.out_pre;
  p.M = r.M;
  p.N = r.N;
  p.batch = r.batch;
  p.stride_out = r.batch > 1 ? r.stride_out : r.M * r.N;
  p.epi = r.ffn ? mmk::EPI_NONE : r.epi;
  p.out_f32 = r.out_f32 ? 1 : 0;
  const int64_t blocks = std::min<int64_t>(cdiv(r.M * r.N * r.batch, 256), 8192);
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mmk::empty_k_fill), dim3((unsigned)blocks),
                                       dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MM_ERR_HIP, std::string("hipLaunchKernel (K = 0): ") + hipGetErrorString(e));
  return MM_OK;
}

// ----------------------------------------------------------------------------
// Skinny products (gemm_skinny): K-contiguous single-weight single-output
// products of at most 32 rows against at least 8 MiB of weights, unless a
// configuration is forced.  Without a workspace each block of 64 weight rows
// is one workgroup; with one, K may also be cut into S slices (at most 16, of
// at least one 256-k stage each) where the workgroups would not keep HBM busy.
// ----------------------------------------------------------------------------
constexpr int64_t kSkinnyCUs = 256;  // workgroups resident at once: one per CU (LDS)

bool skinny_shape(const Request& r) {
  return a_kcontig(r.layout) && b_kcontig(r.layout) && !r.ffn && !r.out_pre && r.batch == 1 &&
         r.M <= mmk::kSkinnyMaxM && r.K >= 256 && r.K <= (int64_t(1) << 23) && r.N * r.K >= (int64_t(1) << 22);
}

struct SkinnyPlan {
  int kc = 0;       // k per slice
  int slices = 1;   // S
};

// The number of slices S (at most max_slices) that minimises the modelled
// time, in bytes streamed at the full rate: the weight, slowed in proportion
// when fewer workgroups are resident than it takes to keep HBM busy (128 +
// 8 per activation row, at most 256: each row's copies slow a workgroup's
// stream), plus, when split, the second launch (about as long as streaming
// 18 MB) and the partial sums written and read back.  Measured with cold
// weights: one row at 8192 x 8192 runs best unsplit (30.9 us against 33.9
// in two slices), 16 rows at 4096 x 14336 in four slices (25.9 against 31.5
// in two).
SkinnyPlan skinny_plan(const Request& r, int64_t max_slices) {
  const int xb = mmk::skinny_xb((int)r.M);
  const int64_t rows = mmk::skinny_rows(xb);
  const int64_t ngroups = cdiv(r.N, rows);
  const double busy = (double)std::min<int64_t>(256, 128 + 8 * r.M);
  const double wbytes = 2.0 * (double)r.N * (double)r.K;
  // one slice (no workspace) is always possible
  const int64_t smax =
      std::max<int64_t>(1, std::min<int64_t>({mmk::kSkinnyMaxSlices, max_slices, r.K / mmk::skinny_kd(xb)}));
  SkinnyPlan sp;
  double best = -1.0;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t kc = cdiv(cdiv(r.K, S), 64) * 64;
    const int64_t slices = cdiv(r.K, kc);
    if (slices != S) continue;
    const double resident = (double)std::min<int64_t>(ngroups * slices, kSkinnyCUs);
    double cost = wbytes * std::max(1.0, busy / resident);
    if (slices > 1) cost += 18e6 + 2.0 * (double)(slices * r.M * r.N * 4);
    if (best < 0.0 || cost < best - 1e-9) {
      best = cost;
      sp.kc = (int)kc;
      sp.slices = (int)slices;
    }
  }
  return sp;
}

int64_t skinny_ws_bytes(const Request& r, const SkinnyPlan& sp) {
  return sp.slices > 1 ? (int64_t)sp.slices * r.M * r.N * 4 : 0;
}

mm_status run_skinny(const Request& r, void* stream) {
  // with the static scratch, as many slices as it holds
  const int64_t per_slice = r.M * r.N * 4;
  SkinnyPlan sp = skinny_plan(r, r.ws ? (r.static_ws ? r.ws_bytes / per_slice : mmk::kSkinnyMaxSlices) : 1);
  const int64_t need = skinny_ws_bytes(r, sp);
  if (need > 0) {
    if (r.ws_bytes < need) return fail(MM_ERR_INVALID_VALUE, "workspace smaller than mm_workspace_size reports");
    if (!aligned(r.ws, 256)) return fail(MM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  }
  mmk::SkinnyParams p;
  p.A = static_cast<const uint16_t*>(r.A);
  p.B = static_cast<const uint16_t*>(r.B);
  p.bias = static_cast<const uint16_t*>(r.bias);
  p.out = r.out;
  p.part = need > 0 ? static_cast<float*>(r.ws) : nullptr;
  p.M = (int)r.M;
  p.N = (int)r.N;
  p.K = (int)r.K;
  p.kc = sp.kc;
  p.slices = sp.slices;
  p.epi = r.epi;
  p.out_f32 = r.out_f32 ? 1 : 0;
  const int xb = mmk::skinny_xb((int)r.M);
  const int64_t grid = cdiv(r.N, mmk::skinny_rows(xb)) * sp.slices;
  void* args[] = {&p};
  // blocks of 16 activation rows the kernel carries
  const void* kern = xb == 1 ? reinterpret_cast<const void*>(&mmk::gemm_skinny<1>)
                              : reinterpret_cast<const void*>(&mmk::gemm_skinny<2>);
  hipError_t e = hipLaunchKernel(kern, dim3((unsigned)grid), dim3(256), args, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MM_ERR_HIP, std::string("hipLaunchKernel (skinny): ") + hipGetErrorString(e));
  if (sp.slices > 1) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mmk::skinny_reduce), dim3((unsigned)cdiv(r.M * r.N, 1024)),
                        dim3(256), args, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(MM_ERR_HIP, std::string("hipLaunchKernel (skinny reduction): ") + hipGetErrorString(e));
  }
  return MM_OK;
}

mm_status run(const Request& r, void* stream) {
  mm_status s = validate(r);
  if (s != MM_OK) return s;
  if (r.M == 0 || r.N == 0) return MM_OK;
  if (r.K == 0) return run_empty_k(r, stream);
  const Config c = choose_config_for(r);
  if (!c.forced && skinny_shape(r)) return run_skinny(r, stream);
  Plan pl;
  SkPlan sp;
  s = plan_host(r, c, &pl);
  if (s != MM_OK) return s;
  int cus = 0, occ = 0;
  if ((s = device_cus(&cus)) != MM_OK) return s;
  if (r.ws && splitk_shape(r) && c.sk != 1) {
    // the split-K kernel's grid: one wave of resident workgroups
    int sk_occ = 0;
    KernelEntry* sk = find_kernel(256, 256, 2, 2, a_kcontig(r.layout), b_kcontig(r.layout), false, 3, true);
    if ((s = kernel_occupancy(sk, &sk_occ)) != MM_OK) return s;
    sp = splitk_plan(r, c, splitk_wgs(c, cus, sk_occ));
    if (sp.n > 1) {
      if (r.static_ws && r.ws_bytes < splitk_ws_bytes(sp))
        return fail(MM_ERR_UNSUPPORTED,
                    "this shape's split-K needs " + std::to_string(splitk_ws_bytes(sp)) +
                        " bytes of scratch, more than the static scratch's " +
                        std::to_string(r.ws_bytes) + " (use mm_matmul_ws with a workspace)");
      if (r.ws_bytes < splitk_ws_bytes(sp))
        return fail(MM_ERR_INVALID_VALUE, "workspace smaller than mm_workspace_size reports");
      if (!aligned(r.ws, 256)) return fail(MM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
      // the split launch's own tile order (a forced configuration keeps its G)
      Config cs = c;
      if (!c.forced) cs.group = compact_band(cdiv(sp.wgs, mmk::kNumXcd), cdiv(r.M, 256));
      if ((s = plan_host(r, cs, &pl, sp)) != MM_OK) return s;
    }
  }
  if ((s = kernel_occupancy(pl.kernel, &occ)) != MM_OK) return s;
  const int64_t units = (int64_t)pl.p.num_tiles * pl.p.batch;
  int64_t grid = c.grid > 0 ? c.grid : (int64_t)cus * occ;
  if (grid > units) grid = units;
  if (sp.n > 1) grid = sp.wgs;  // one chunk range per workgroup, all resident
  if (std::getenv("MM_LOG"))
    std::fprintf(stderr, "libmm: M=%lld N=%lld K=%lld layout=%d ffn=%d -> BM=%d BN=%d WM=%d WN=%d G=%d "
                 "XCD=%d KALT=%d grid=%lld tiles=%d chunks=%d\n", (long long)r.M, (long long)r.N,
                 (long long)r.K, r.layout, (int)r.ffn, c.bm, c.bn, c.wgm, c.wgn, pl.p.group_m, c.xcd,
                 pl.p.k_alt, (long long)grid, pl.p.num_tiles, pl.p.sk_chunks);
  void* args[] = {&pl.p};
  hipError_t e = hipLaunchKernel(pl.kernel->fn, dim3((unsigned)grid), dim3(pl.threads), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MM_ERR_HIP, std::string("hipLaunchKernel: ") + hipGetErrorString(e));
  if (sp.n > 1) {
    // the pieces' partial tiles meet: 32 blocks of 8 rows per tile
    mmk::SkReduceParams rp;
    rp.part = pl.p.sk_part;
    rp.out = r.out;
    rp.M = (int)r.M;
    rp.N = (int)r.N;
    rp.tiles_m = pl.p.tiles_m;
    rp.tiles_n = pl.p.tiles_n;
    rp.num_tiles = pl.p.num_tiles;
    rp.group_m = pl.p.group_m;
    rp.chunks = sp.n;
    rp.items = sp.q;
    rp.out_f32 = pl.p.out_f32;
    rp.out_vec = pl.p.out_vec;
    rp.tile_n = sp.bn;
    rp.bias = static_cast<const uint16_t*>(r.bias);
    rp.epi = r.epi;
    void* rargs[] = {&rp};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mmk::splitk_reduce), dim3((unsigned)(32 * rp.num_tiles)),
                        dim3(256), rargs, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(MM_ERR_HIP, std::string("hipLaunchKernel (split-K reduction): ") + hipGetErrorString(e));
  }
  return MM_OK;
}

int map_epilogue(mm_epilogue e) {
  switch (e) {
    case MM_EPI_NONE: return mmk::EPI_NONE;
    case MM_EPI_BIAS: return mmk::EPI_BIAS;
    case MM_EPI_GELU_TANH: return mmk::EPI_GELU;
    case MM_EPI_BIAS_GELU_TANH: return mmk::EPI_BIAS_GELU;
  }
  return -1;
}

}  // namespace

extern "C" {

mm_status mm_matmul(const void* A, const void* B, void* out, int64_t M, int64_t N, int64_t K,
                    mm_layout layout, mm_out_dtype out_dtype, void* stream) {
  g_last_error.clear();
  if (out_dtype != MM_OUT_BF16 && out_dtype != MM_OUT_F32)
    return fail(MM_ERR_INVALID_VALUE, "bad output dtype");
  Request r{A, B, nullptr, nullptr, out, M, N, K, (int)layout, mmk::EPI_NONE,
            out_dtype == MM_OUT_F32, false};
  return run(r, stream);
}

mm_status mm_linear(const void* x, const void* W, const void* bias, void* out, int64_t M, int64_t N,
                    int64_t K, mm_layout layout, mm_epilogue epi, void* stream) {
  g_last_error.clear();
  const int e = map_epilogue(epi);
  if (e < 0) return fail(MM_ERR_INVALID_VALUE, "bad epilogue");
  Request r{x, W, nullptr, bias, out, M, N, K, (int)layout, e, false, false};
  return run(r, stream);
}

mm_status mm_linear_preact(const void* x, const void* W, const void* bias, void* out, void* preact,
                           int64_t M, int64_t N, int64_t K, mm_layout layout, mm_epilogue epi,
                           void* stream) {
  g_last_error.clear();
  const int e = map_epilogue(epi);
  if (e < 0) return fail(MM_ERR_INVALID_VALUE, "bad epilogue");
  if (!preact && M > 0 && N > 0) return fail(MM_ERR_INVALID_VALUE, "null preact pointer");
  Request r{x, W, nullptr, bias, out, M, N, K, (int)layout, e, false, false};
  r.out_pre = preact;
  if (M > 0 && N > 0 && e != mmk::EPI_GELU && e != mmk::EPI_BIAS_GELU)
    return fail(MM_ERR_INVALID_VALUE, "a pre-activation output needs a GELU epilogue");
  return run(r, stream);
}

mm_status mm_matmul_batched(const void* A, const void* B, void* out, int64_t batch, int64_t M,
                            int64_t N, int64_t K, int64_t stride_a, int64_t stride_b,
                            int64_t stride_out, mm_layout layout, mm_out_dtype out_dtype,
                            void* stream) {
  g_last_error.clear();
  if (out_dtype != MM_OUT_BF16 && out_dtype != MM_OUT_F32)
    return fail(MM_ERR_INVALID_VALUE, "bad output dtype");
  Request r{A, B, nullptr, nullptr, out, M, N, K, (int)layout, mmk::EPI_NONE,
            out_dtype == MM_OUT_F32, false};
  r.batch = batch;
  r.stride_a = stride_a;
  r.stride_b = stride_b;
  r.stride_out = stride_out;
  return run(r, stream);
}

mm_status mm_linear_batched(const void* x, const void* W, const void* bias, void* out, int64_t batch,
                            int64_t M, int64_t N, int64_t K, int64_t stride_x, int64_t stride_w,
                            int64_t stride_out, mm_layout layout, mm_epilogue epi, void* stream) {
  g_last_error.clear();
  const int e = map_epilogue(epi);
  if (e < 0) return fail(MM_ERR_INVALID_VALUE, "bad epilogue");
  Request r{x, W, nullptr, bias, out, M, N, K, (int)layout, e, false, false};
  r.batch = batch;
  r.stride_a = stride_x;
  r.stride_b = stride_w;
  r.stride_out = stride_out;
  return run(r, stream);
}

mm_status mm_workspace_size(int form, int64_t M, int64_t N, int64_t K, mm_layout layout,
                            int64_t* bytes) {
  g_last_error.clear();
  if (!bytes || (form != 0 && form != 1) || M < 0 || N < 0 || K < 0 || layout < MM_NN ||
      layout > MM_TT)
    return fail(MM_ERR_INVALID_VALUE, "bad arguments");
  *bytes = 0;
  Request r{nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, (int)layout, mmk::EPI_NONE,
            false, form == 1};
  if (M == 0 || N == 0 || K == 0) return MM_OK;
  const Config c = choose_config_for(r);
  if (!c.forced && skinny_shape(r)) {
    *bytes = skinny_ws_bytes(r, skinny_plan(r, mmk::kSkinnyMaxSlices));
    return MM_OK;
  }
  if (!splitk_shape(r) || c.sk == 1) return MM_OK;
  int cus = 0, occ = 0;
  mm_status s;
  if ((s = device_cus(&cus)) != MM_OK) return s;
  if ((s = kernel_occupancy(find_kernel(256, 256, 2, 2, a_kcontig(r.layout), b_kcontig(r.layout), false, 3, true),
                            &occ)) != MM_OK)
    return s;
  *bytes = splitk_ws_bytes(splitk_plan(r, c, splitk_wgs(c, cus, occ)));
  return MM_OK;
}

mm_status mm_matmul_ws(const void* A, const void* B, void* out, int64_t M, int64_t N, int64_t K,
                       mm_layout layout, mm_out_dtype out_dtype, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (out_dtype != MM_OUT_BF16 && out_dtype != MM_OUT_F32)
    return fail(MM_ERR_INVALID_VALUE, "bad output dtype");
  Request r{A, B, nullptr, nullptr, out, M, N, K, (int)layout, mmk::EPI_NONE,
            out_dtype == MM_OUT_F32, false, workspace, workspace ? workspace_bytes : 0};
  return run(r, stream);
}

mm_status mm_matmul_noalloc(const void* A, const void* B, void* out, int64_t M, int64_t N,
                            int64_t K, mm_layout layout, mm_out_dtype out_dtype, void* stream) {
  g_last_error.clear();
  if (out_dtype != MM_OUT_BF16 && out_dtype != MM_OUT_F32)
    return fail(MM_ERR_INVALID_VALUE, "bad output dtype");
  Request r{A, B, nullptr, nullptr, out, M, N, K, (int)layout, mmk::EPI_NONE,
            out_dtype == MM_OUT_F32, false};
  // argument errors first, before any HIP call
  mm_status s = validate(r);
  if (s != MM_OK || M == 0 || N == 0) return s;
  if ((s = scratch_address(&r.ws)) != MM_OK) return s;
  r.ws_bytes = kScratchBytes;
  r.static_ws = true;
  return run(r, stream);
}

mm_status mm_linear_ws(const void* x, const void* W, const void* bias, void* out, int64_t M,
                       int64_t N, int64_t K, mm_layout layout, mm_epilogue epi, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const int e = map_epilogue(epi);
  if (e < 0) return fail(MM_ERR_INVALID_VALUE, "bad epilogue");
  Request r{x, W, nullptr, bias, out, M, N, K, (int)layout, e, false, false, workspace,
            workspace ? workspace_bytes : 0};
  return run(r, stream);
}

mm_status mm_ffn_glu(const void* x, const void* W_gate, const void* W_up, void* out, int64_t M,
                     int64_t N, int64_t K, mm_glu_act act, void* stream) {
  g_last_error.clear();
  if (act != MM_GLU_SILU && act != MM_GLU_IDENTITY) return fail(MM_ERR_INVALID_VALUE, "bad activation");
  Request r{x, W_gate, W_up, nullptr, out, M, N, K, MM_NT,
            act == MM_GLU_SILU ? mmk::EPI_SWIGLU : mmk::EPI_GLU_ID, false, true};
  return run(r, stream);
}

mm_status mm_ffn_swiglu(const void* x, const void* W_gate, const void* W_up, void* out, int64_t M,
                        int64_t N, int64_t K, void* stream) {
  return mm_ffn_glu(x, W_gate, W_up, out, M, N, K, MM_GLU_SILU, stream);
}

mm_status mm_set_config(const char* spec) {
  g_last_error.clear();
  read_env_once();
  if (!spec || !*spec) {
    std::lock_guard<std::mutex> g(g_cfg_mu);
    g_cfg_forced = false;
    return MM_OK;
  }
  Config c;
  if (!parse_config(spec, &c))
    return fail(MM_ERR_UNSUPPORTED, std::string("invalid or unsupported configuration: ") + spec);
  std::lock_guard<std::mutex> g(g_cfg_mu);
  g_cfg_forced = true;
  g_cfg_force = c;
  return MM_OK;
}

mm_status mm_describe_config(int form, int64_t M, int64_t N, int64_t K, mm_layout layout, char* buf,
                             int64_t buflen) {
  g_last_error.clear();
  if (!buf || buflen <= 0 || (form != 0 && form != 1) || M < 0 || N < 0 || K < 0 ||
      layout < MM_NN || layout > MM_TT)
    return fail(MM_ERR_INVALID_VALUE, "bad arguments");
  const Request rq{nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, (int)layout, mmk::EPI_NONE,
                   false, form == 1};
  const Config c = choose_config_for(rq);
  // the kernel a call of this shape would launch (no HIP call is made)
  const char* kernel = M > 0 && N > 0 && K == 0 ? "empty_k_fill" : "none";
  if (M > 0 && N > 0 && K > 0) {
    const Request& r = rq;
    Plan pl;
    if (plan_host(r, c, &pl) == MM_OK)
      kernel = pl.kernel->pipe == 6   ? "gemm_small"
               : pl.kernel->pipe == 5 ? "gemm_pp"
               : pl.kernel->pipe == 4 ? "gemm_ws"
               : pl.kernel->pipe == 3 ? "gemm_nt_slab"
               : pl.kernel->pipe == 2 ? "gemm_pingpong"
               : pl.kernel->pipe      ? "gemm_nt_pipe"
                                      : "gemm_persistent";
    g_last_error.clear();
  }
  // a plain product that a workspace would split: chunks per tile and tile
  // width on the current device (queries the device; left out without one)
  char split[32] = "";
  const bool skinny = M > 0 && N > 0 && K > 0 && !c.forced && skinny_shape(rq);
  if (skinny) {
    // the skinny kernel (no device query): S slices of K with a workspace
    kernel = "gemm_skinny";
    const SkinnyPlan sp = skinny_plan(rq, mmk::kSkinnyMaxSlices);
    if (sp.slices > 1) std::snprintf(split, sizeof split, "SPLIT=%dx%d,", sp.slices,
                                        mmk::skinny_rows(mmk::skinny_xb((int)M)));
  } else if (M > 0 && N > 0 && K > 0 && form == 0 && c.sk != 1) {
    Request r{nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, (int)layout, mmk::EPI_NONE,
              false, false};
    int cus = 0, occ = 0;
    if (splitk_shape(r) && device_cus(&cus) == MM_OK &&
        kernel_occupancy(find_kernel(256, 256, 2, 2, a_kcontig(r.layout), b_kcontig(r.layout), false, 3, true),
                         &occ) == MM_OK) {
      const SkPlan sp = splitk_plan(r, c, splitk_wgs(c, cus, occ));
      if (sp.n > 1) std::snprintf(split, sizeof split, "SPLIT=%dx%d,", sp.n, sp.bn);
    }
    g_last_error.clear();
  }
  std::snprintf(buf, (size_t)buflen,
                "BM=%d,BN=%d,WM=%d,WN=%d,G=%d,XCD=%d,KALT=%d,GRID=%d,PIPE=%d,%s%sKERNEL=%s", c.bm, c.bn,
                c.wgm, c.wgn, c.group, c.xcd, k_alt_enabled(c, K) ? 1 : 0, c.grid, c.pipe,
                c.bstage ? "BSTAGE=1," : "", split, kernel);
  return MM_OK;
}

mm_status mm_debug_schedule(int form, int64_t M, int64_t N, int64_t K, mm_layout layout,
                            int64_t grid, int32_t* out, int64_t cap, int64_t* count) {
  g_last_error.clear();
  if ((form != 0 && form != 1) || M <= 0 || N <= 0 || K <= 0 || grid <= 0 || !count ||
      (cap > 0 && !out) || layout < MM_NN || layout > MM_TT)
    return fail(MM_ERR_INVALID_VALUE, "bad arguments");
  Request r{nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, (int)layout, mmk::EPI_NONE,
            false, form == 1};
  const Config c = choose_config_for(r);
  Plan pl;
  mm_status s = plan_host(r, c, &pl);
  if (s != MM_OK) return s;
  const int G = (int)(grid < pl.p.num_tiles ? grid : pl.p.num_tiles);
  int64_t n = 0;
  for (int b = 0; b < G; ++b) {
    const int wg = mmk::remap_workgroup(b, G, pl.p.xcd_remap);
    for (int i = 0; wg + (int64_t)i * G < pl.p.num_tiles; ++i) {
      int tm, tn;
      mmk::tile_coords(wg + i * G, pl.p.tiles_m, pl.p.tiles_n, pl.p.group_m, &tm, &tn);
      if (n < cap) {
        int32_t* o = out + 5 * n;
        o[0] = b;
        o[1] = i;
        o[2] = tm;
        o[3] = tn;
        o[4] = (pl.p.k_alt && (i & 1)) ? 1 : 0;
      }
      ++n;
    }
  }
  *count = n;
  return MM_OK;
}

const char* mm_status_string(mm_status s) {
  switch (s) {
    case MM_OK: return "MM_OK";
    case MM_ERR_INVALID_VALUE: return "MM_ERR_INVALID_VALUE";
    case MM_ERR_UNSUPPORTED: return "MM_ERR_UNSUPPORTED";
    case MM_ERR_MISALIGNED: return "MM_ERR_MISALIGNED";
    case MM_ERR_HIP: return "MM_ERR_HIP";
  }
  return "MM_ERR_UNKNOWN";
}

const char* mm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
