// Host runtime of libmicroadam: argument checks, state allocation, per-step
// constants and kernel launches on the caller's stream.  The C ABI is declared
// and documented in include/microadam.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "microadam.h"
#include "microadam_kernels.hpp"
#include "adamw_kernels.hpp"

using namespace microadam;

namespace {

thread_local int g_err = MA_OK;
thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
  g_err = code;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() {
  g_err = MA_OK;
  g_msg[0] = 0;
}

// Largest dynamic LDS the update kernel asks for: three of its workgroups,
// with their static LDS (under 1 KiB), fit one CU's 160 KiB.  A long window
// (m = 37 at k = d/100) then takes two slot passes per block; measured, that
// beats one pass at two workgroups per CU (and smaller budgets, with more
// passes, are slower again).
constexpr size_t kApplyLdsLimit = 53 * 1024 - 512;
// step_csu_kernel's LDS buffer (three workgroups per CU)
constexpr size_t kFusedCsuLdsLimit = 4 * (size_t)kFusedCsuWords;

// ---------------------------------------------------------------- ma_step_noalloc's scratch
// The per-step scratch of ma_step_noalloc lives in one file-scope device
// array, which each device the library runs on holds until the process ends:
// the compressor's deferred-block list (int64 per block) and its counters, and
// the global quantizer's per-block min / max (2 f32 per block), cut (2 u32 per
// block) and global pair.  Sized for kNoAllocMaxBlocks blocks: 24 MiB.  In
// host code `scratch` names a host-side stand-in; kernels get the device
// address from hipGetSymbolAddress, taken once per device.
constexpr int64_t kNoAllocMaxBlocks = int64_t(1) << 20;
constexpr size_t kNaDeferred = 0;                                  // int64[kNoAllocMaxBlocks]
constexpr size_t kNaCounts = kNaDeferred + 8 * kNoAllocMaxBlocks;  // u32[64]
constexpr size_t kNaBlkmm = kNaCounts + 256;                       // f32[2 * kNoAllocMaxBlocks]
constexpr size_t kNaSelinfo = kNaBlkmm + 8 * kNoAllocMaxBlocks;    // u32[2 * kNoAllocMaxBlocks]
constexpr size_t kNaGmm = kNaSelinfo + 8 * kNoAllocMaxBlocks;      // f32[2]
constexpr size_t kNoAllocScratchBytes = kNaGmm + 256;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev` (which must be current),
// looked up once per device; nullptr if the lookup fails.
void *noalloc_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

constexpr int kTimedKernels = 3;   // compress, adamstats_apply, fused step

struct ma_ctx {
  int64_t d = 0, k = 0, n_b = 0;
  int32_t B = 0, m = 0, b = 4;
  float beta1 = 0, beta2 = 0, eps = 0, lr = 0, wd = 0;
  uint64_t seed = 0;
  uint32_t flags = 0;
  int64_t t = 0;
  int device = 0;
  int cpt = 1;       // 4096-element chunks per thread
  int cap = 0;       // LDS slots per pass of the update kernel
  int ent_cap = 0;   // window entries of one block the update kernel keeps in LDS
  bool dense_default = false;   // stream the parameters in the update even without decay
  size_t apply_lds = 0;
  bool fused_ok = false;   // the block's window fits the fused kernel's LDS (kFusedEnt)
  bool csu_ok = false;     // the column-sorted update takes this shape (entries per thread, LDS)
  size_t csu_lds = 0;      // its dynamic LDS
  int32_t csu_slots = 0;
  bool fused_csu_ok = false;   // full blocks fit step_csu_kernel (three workgroups per CU)
  size_t fused_csu_lds = 0;
  int32_t fused_union_words = 0;
  int32_t thl_off = 0, thl_n = 0;   // step_csu_kernel: LDS chunk of the parameters (0: none)

  uint8_t *codes = nullptr;
  size_t codes_bytes = 0, codes_alloc = 0;
  float *stats = nullptr;
  uint32_t *window = nullptr;
  int64_t *off_tab = nullptr;
  float *betapow = nullptr;
  unsigned long long *touched = nullptr;
  bool count_touched = false;
  int64_t *deferred = nullptr;        // blocks handed from the full-block to the general compressor
  unsigned int *n_deferred = nullptr;
  // global quantizer (MA_FLAG_GLOBAL_QUANT): per-block min / max and cut, global pair
  float *blkmm = nullptr;
  uint32_t *selinfo = nullptr;
  float *gmm = nullptr;

  // last step's constants (for ma_debug_moments)
  float last_c1 = 0, last_c2 = 0;

  // device address of ma_step_noalloc's scratch on this handle's device
  // (looked up at create; nullptr if that failed)
  unsigned char *na_scratch = nullptr;

  // overlap of compress and update across block ranges (see ma_step)
  int chunks = 1;
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  std::vector<hipEvent_t> chunk_ev;

  bool timing = false;
  struct Ev { int kernel; hipEvent_t start, end; };
  std::vector<Ev> events;          // recorded, not yet read
  std::vector<hipEvent_t> pool;    // free timing events
  double acc_ms[kTimedKernels] = {0, 0, 0};
  int64_t acc_n[kTimedKernels] = {0, 0, 0};
};

namespace {

void free_all(ma_ctx *h) {
  // teardown: failures are ignored on purpose (nothing is left to undo)
  if (!h) return;
  (void)hipFree(h->codes);
  (void)hipFree(h->stats);
  (void)hipFree(h->window);
  (void)hipFree(h->off_tab);
  (void)hipFree(h->betapow);
  (void)hipFree(h->touched);
  (void)hipFree(h->deferred);
  (void)hipFree(h->n_deferred);
  (void)hipFree(h->blkmm);
  (void)hipFree(h->selinfo);
  (void)hipFree(h->gmm);
  for (auto &ev : h->events) {
    (void)hipEventDestroy(ev.start);
    (void)hipEventDestroy(ev.end);
  }
  for (auto e : h->pool) (void)hipEventDestroy(e);
  h->events.clear();
  h->pool.clear();
  for (auto e : h->chunk_ev) (void)hipEventDestroy(e);
  h->chunk_ev.clear();
  if (h->fork_ev) (void)hipEventDestroy(h->fork_ev);
  if (h->join_ev) (void)hipEventDestroy(h->join_ev);
  if (h->side) (void)hipStreamDestroy(h->side);
  h->fork_ev = h->join_ev = nullptr;
  h->side = nullptr;
}

// The side stream (default priority) and the events that order it against
// the caller's stream, for `chunks` block ranges.
bool ensure_pipeline(ma_ctx *h, int chunks) {
  if (!h->side && hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess) return false;
  if (!h->fork_ev && hipEventCreateWithFlags(&h->fork_ev, hipEventDisableTiming) != hipSuccess) return false;
  if (!h->join_ev && hipEventCreateWithFlags(&h->join_ev, hipEventDisableTiming) != hipSuccess) return false;
  while ((int)h->chunk_ev.size() < chunks) {
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return false;
    h->chunk_ev.push_back(ev);
  }
  return true;
}

hipEvent_t timing_event(ma_ctx *h) {
  if (!h->pool.empty()) {
    hipEvent_t e = h->pool.back();
    h->pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

// Takes n timing events, all or none: on failure the ones taken go back to
// the pool.  A step takes its events before it launches anything.
bool take_events(ma_ctx *h, hipEvent_t *ev, int n) {
  for (int i = 0; i < n; ++i) {
    ev[i] = timing_event(h);
    if (!ev[i]) {
      for (int q = 0; q < i; ++q) h->pool.push_back(ev[q]);
      return false;
    }
  }
  return true;
}

int64_t floor_mul_div(int64_t k, int64_t x, int64_t d) {
  const unsigned __int128 p = (unsigned __int128)(uint64_t)k * (uint64_t)x;
  return (int64_t)(p / (uint64_t)d);
}

// Device guard: runs with the handle's device current, restores afterwards.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Compressor launches for blocks [b0, b1): blocks below n_full take the
// bounds-free kernel (plus the kernel finishing what it deferred), the rest
// the general one.  a.deferred / a.n_deferred are this range's list; its
// counter must be zero on entry.
template <int CPT, bool AL, bool EF>
hipError_t launch_compress(const CompressArgs &a, int64_t b0, int64_t b1, int64_t n_full, hipStream_t s) {
  const int64_t f1 = std::min(b1, n_full);
  if (CPT <= 4 && AL && f1 > b0) {
    constexpr int C4 = CPT <= 4 ? CPT : 4;
    hipLaunchKernelGGL((compress_full_kernel<C4, EF>), dim3((unsigned)(f1 - b0)), dim3(kThreads), 0, s, a, b0);
    hipLaunchKernelGGL((compress_deferred_kernel<C4, EF>), dim3((unsigned)std::min<int64_t>(f1 - b0, 256)),
                       dim3(kThreads), 0, s, a);
  }
  const int64_t g0 = std::max(b0, (CPT <= 4 && AL) ? n_full : (int64_t)0);
  if (b1 > g0)
    hipLaunchKernelGGL((compress_kernel<CPT, AL, EF>), dim3((unsigned)(b1 - g0)), dim3(kThreads), 0, s, a, g0);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_compress_cpt(bool aligned, bool ef, const CompressArgs &a, int64_t b0, int64_t b1,
                               int64_t n_full, hipStream_t s) {
  if (ef)
    return aligned ? launch_compress<CPT, true, true>(a, b0, b1, n_full, s)
                   : launch_compress<CPT, false, true>(a, b0, b1, n_full, s);
  return aligned ? launch_compress<CPT, true, false>(a, b0, b1, n_full, s)
                 : launch_compress<CPT, false, false>(a, b0, b1, n_full, s);
}

hipError_t dispatch_compress(int cpt, bool aligned, bool ef, const CompressArgs &a, int64_t b0, int64_t b1,
                             int64_t n_full, hipStream_t s) {
  switch (cpt) {
    case 1: return launch_compress_cpt<1>(aligned, ef, a, b0, b1, n_full, s);
    case 2: return launch_compress_cpt<2>(aligned, ef, a, b0, b1, n_full, s);
    case 4: return launch_compress_cpt<4>(aligned, ef, a, b0, b1, n_full, s);
    default: return launch_compress_cpt<8>(aligned, ef, a, b0, b1, 0, s);
  }
}

// How the update runs: the column-sorted kernels (csu) or the row-by-row
// ones, with the dynamic LDS of the kind chosen.
struct UpdLaunch {
  bool csu;
  size_t lds;
  bool fused_csu;      // full blocks: step_csu_kernel instead of step_full_kernel
  size_t fused_lds;    // its dynamic LDS
  bool thl;            // step_csu_kernel with fp32 parameters through LDS (16-byte aligned ones)
};

template <int CPT, int MODE, bool AL, bool BF>
hipError_t launch_apply(const ApplyArgs &a, int64_t grid, const UpdLaunch &u, hipStream_t s) {
  if (u.csu)
    hipLaunchKernelGGL((apply_csu_kernel<CPT, MODE, AL, BF>), dim3((unsigned)grid), dim3(kThreads), u.lds, s, a);
  else
    hipLaunchKernelGGL((apply_kernel<CPT, MODE, AL, BF>), dim3((unsigned)grid), dim3(kThreads), u.lds, s, a);
  return hipGetLastError();
}

template <int CPT, bool BF>
hipError_t launch_apply_cpt(int mode, bool aligned, const ApplyArgs &a, int64_t grid, const UpdLaunch &lds,
                            hipStream_t s) {
  if (mode == kModeSparse)
    return aligned ? launch_apply<CPT, kModeSparse, true, BF>(a, grid, lds, s)
                   : launch_apply<CPT, kModeSparse, false, BF>(a, grid, lds, s);
  if (mode == kModeMoments) return launch_apply<CPT, kModeMoments, false, false>(a, grid, lds, s);
  return aligned ? launch_apply<CPT, kModeDense, true, BF>(a, grid, lds, s)
                 : launch_apply<CPT, kModeDense, false, BF>(a, grid, lds, s);
}

// bf: the parameters are bfloat16 (ApplyArgs::theta16)
hipError_t dispatch_apply(int cpt, int mode, bool aligned, const ApplyArgs &a, int64_t grid, const UpdLaunch &lds,
                          hipStream_t s, bool bf = false) {
  switch (cpt) {
    case 1: return bf ? launch_apply_cpt<1, true>(mode, aligned, a, grid, lds, s) : launch_apply_cpt<1, false>(mode, aligned, a, grid, lds, s);
    case 2: return bf ? launch_apply_cpt<2, true>(mode, aligned, a, grid, lds, s) : launch_apply_cpt<2, false>(mode, aligned, a, grid, lds, s);
    case 4: return bf ? launch_apply_cpt<4, true>(mode, aligned, a, grid, lds, s) : launch_apply_cpt<4, false>(mode, aligned, a, grid, lds, s);
    default: return bf ? launch_apply_cpt<8, true>(mode, aligned, a, grid, lds, s) : launch_apply_cpt<8, false>(mode, aligned, a, grid, lds, s);
  }
}

// The fused step for blocks [0, n_full): the fused kernel, then the blocks it
// deferred (compress, then update, from the device list).  QMODE kQGlobal1:
// the global quantizer's first pass in place of the compressor.
template <int CPT, bool EF, bool BF, int QMODE = kQBlock, int MODE = kModeSparse, bool PAL = false>
hipError_t launch_fused(const CompressArgs &c, const ApplyArgs &a, int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s) {
  bool launched = false;
  if constexpr (!BF && PAL && QMODE == kQBlock) {
    if (apply_lds.fused_csu && apply_lds.thl) {
      hipLaunchKernelGGL((step_csu_kernel<CPT, EF, BF, QMODE, MODE, PAL, true>), dim3((unsigned)n_full),
                         dim3(kThreads), 0, s, c, a, (int64_t)0);
      launched = true;
    }
  }
  if (launched) {
  } else if (apply_lds.fused_csu) {
    hipLaunchKernelGGL((step_csu_kernel<CPT, EF, BF, QMODE, MODE, PAL>), dim3((unsigned)n_full), dim3(kThreads), 0,
                       s, c, a, (int64_t)0);
  } else {
    // the kernel's LDS holds at most kFusedBeta decay factors (2m)
    if (2 * (int64_t)a.m > kFusedBeta) return hipErrorInvalidValue;
    hipLaunchKernelGGL((step_full_kernel<CPT, EF, BF, QMODE, MODE, PAL>), dim3((unsigned)n_full), dim3(kThreads), 0,
                       s, c, a, (int64_t)0);
  }
  const unsigned grid2 = (unsigned)std::min<int64_t>(n_full, 256);
  hipLaunchKernelGGL((compress_deferred_kernel<CPT, EF, QMODE>), dim3(grid2), dim3(kThreads), 0, s, c);
  ApplyArgs al = a;
  al.blocks = c.deferred;
  al.n_list = c.n_deferred;
  if (apply_lds.csu)
    hipLaunchKernelGGL((apply_csu_list_kernel<CPT, BF, MODE>), dim3(grid2), dim3(kThreads), apply_lds.lds, s, al);
  else
    hipLaunchKernelGGL((apply_list_kernel<CPT, BF, MODE>), dim3(grid2), dim3(kThreads), apply_lds.lds, s, al);
  return hipGetLastError();
}

template <bool BF>
hipError_t dispatch_fused_t(int cpt, bool ef, bool dense, bool p_al, const CompressArgs &c, const ApplyArgs &a,
                            int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s) {
  if (dense) {   // decoupled decay: every parameter streamed (aligned parameters only)
    switch (cpt) {
      case 1: return ef ? launch_fused<1, true, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s)
                        : launch_fused<1, false, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s);
      case 2: return ef ? launch_fused<2, true, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s)
                        : launch_fused<2, false, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s);
      default: return ef ? launch_fused<4, true, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s)
                         : launch_fused<4, false, BF, kQBlock, kModeDense, true>(c, a, n_full, apply_lds, s);
    }
  }
  // sparse: 16-byte aligned parameters go through the column-sorted update's
  // vector loads and stores (the row-by-row update gathers single parameters
  // either way)
  if (p_al && apply_lds.fused_csu) {
    switch (cpt) {
      case 1: return ef ? launch_fused<1, true, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s)
                        : launch_fused<1, false, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s);
      case 2: return ef ? launch_fused<2, true, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s)
                        : launch_fused<2, false, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s);
      default: return ef ? launch_fused<4, true, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s)
                         : launch_fused<4, false, BF, kQBlock, kModeSparse, true>(c, a, n_full, apply_lds, s);
    }
  }
  switch (cpt) {
    case 1: return ef ? launch_fused<1, true, BF>(c, a, n_full, apply_lds, s) : launch_fused<1, false, BF>(c, a, n_full, apply_lds, s);
    case 2: return ef ? launch_fused<2, true, BF>(c, a, n_full, apply_lds, s) : launch_fused<2, false, BF>(c, a, n_full, apply_lds, s);
    default: return ef ? launch_fused<4, true, BF>(c, a, n_full, apply_lds, s) : launch_fused<4, false, BF>(c, a, n_full, apply_lds, s);
  }
}

hipError_t dispatch_fused(int cpt, bool ef, bool dense, bool p_al, const CompressArgs &c, const ApplyArgs &a,
                          int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s, bool bf) {
  return bf ? dispatch_fused_t<true>(cpt, ef, dense, p_al, c, a, n_full, apply_lds, s)
            : dispatch_fused_t<false>(cpt, ef, dense, p_al, c, a, n_full, apply_lds, s);
}

// The global quantizer's launches over all blocks: pass 1 (full aligned
// blocks [0, n_full) by the staged kernel, the blocks it defers, then the
// rest), the global min / max, pass 2 (error feedback on).  a.n_deferred
// must be zero on entry.
template <int CPT, bool AL, int QMODE>
void launch_global_pass(const CompressArgs &a, int64_t n_b, int64_t n_full, hipStream_t s) {
  const dim3 blk(kThreads);
  if (CPT <= 4 && AL && n_full > 0) {
    constexpr int C4 = CPT <= 4 ? CPT : 4;
    hipLaunchKernelGGL((compress_full_kernel<C4, true, QMODE>), dim3((unsigned)n_full), blk, 0, s, a, (int64_t)0);
    if (QMODE == kQGlobal1)
      hipLaunchKernelGGL((compress_deferred_kernel<C4, true, QMODE>), dim3((unsigned)std::min<int64_t>(n_full, 256)),
                         blk, 0, s, a);
  }
  const int64_t g0 = (CPT <= 4 && AL) ? n_full : 0;
  if (n_b > g0)
    hipLaunchKernelGGL((compress_kernel<CPT, AL, true, QMODE>), dim3((unsigned)(n_b - g0)), blk, 0, s, a, g0);
}

template <int CPT, bool AL>
void launch_global_p1(const CompressArgs &a, int64_t n_b, int64_t n_full, hipStream_t s) {
  launch_global_pass<CPT, AL, kQGlobal1>(a, n_b, n_full, s);
  hipLaunchKernelGGL(global_minmax_kernel, dim3(1), dim3(kThreads), 0, s, (const float *)a.blkmm, n_b,
                     (float *)a.gmm);
}


// Pass 1 and the global min / max over all blocks; pass 2 for blocks
// [b0, b1) (no deferral there: pass 1 recorded every block's cut).
hipError_t dispatch_global_p1(int cpt, bool aligned, const CompressArgs &a, int64_t n_b, int64_t n_full,
                              hipStream_t s) {
  switch (cpt) {
    case 1: aligned ? launch_global_p1<1, true>(a, n_b, n_full, s) : launch_global_p1<1, false>(a, n_b, n_full, s); break;
    case 2: aligned ? launch_global_p1<2, true>(a, n_b, n_full, s) : launch_global_p1<2, false>(a, n_b, n_full, s); break;
    case 4: aligned ? launch_global_p1<4, true>(a, n_b, n_full, s) : launch_global_p1<4, false>(a, n_b, n_full, s); break;
    default: aligned ? launch_global_p1<8, true>(a, n_b, 0, s) : launch_global_p1<8, false>(a, n_b, 0, s); break;
  }
  return hipGetLastError();
}

// The global quantizer's first pass fused with the update: blocks [0, n_full)
// by the fused kernel (and its deferred blocks), the rest (a partial last
// block) by pass 1 and then the update; then the global min / max over all
// blocks.  The second pass follows on the same stream.
template <int CPT, bool BF, int MODE, bool PAL>
hipError_t launch_fused_global1(const CompressArgs &c, const ApplyArgs &a, int mode, bool p_al, int64_t n_b,
                                int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s) {
  hipError_t e = launch_fused<CPT, true, BF, kQGlobal1, MODE, PAL>(c, a, n_full, apply_lds, s);
  if (e == hipSuccess && n_b > n_full) {
    hipLaunchKernelGGL((compress_kernel<CPT, true, true, kQGlobal1>), dim3((unsigned)(n_b - n_full)), dim3(kThreads), 0,
                       s, c, n_full);
    ApplyArgs at = a;
    at.first_block = n_full;
    e = dispatch_apply(CPT, mode, p_al, at, n_b - n_full, apply_lds, s, BF);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(global_minmax_kernel, dim3(1), dim3(kThreads), 0, s, (const float *)c.blkmm, n_b, (float *)c.gmm);
  return hipGetLastError();
}

template <int MODE, bool PAL>
hipError_t dispatch_fused_global1_t(int cpt, bool bf, const CompressArgs &c, const ApplyArgs &a, int mode, bool p_al,
                                    int64_t n_b, int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s) {
  switch (cpt) {
    case 1: return bf ? launch_fused_global1<1, true, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s)
                      : launch_fused_global1<1, false, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s);
    case 2: return bf ? launch_fused_global1<2, true, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s)
                      : launch_fused_global1<2, false, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s);
    default: return bf ? launch_fused_global1<4, true, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s)
                       : launch_fused_global1<4, false, MODE, PAL>(c, a, mode, p_al, n_b, n_full, apply_lds, s);
  }
}

// mode kModeDense requires 16-byte aligned parameters (p_al)
hipError_t dispatch_fused_global1(int cpt, bool bf, const CompressArgs &c, const ApplyArgs &a, int mode, bool p_al,
                                  int64_t n_b, int64_t n_full, const UpdLaunch &apply_lds, hipStream_t s) {
  if (mode == kModeDense)
    return dispatch_fused_global1_t<kModeDense, true>(cpt, bf, c, a, mode, p_al, n_b, n_full, apply_lds, s);
  return (p_al && apply_lds.fused_csu)
             ? dispatch_fused_global1_t<kModeSparse, true>(cpt, bf, c, a, mode, p_al, n_b, n_full, apply_lds, s)
             : dispatch_fused_global1_t<kModeSparse, false>(cpt, bf, c, a, mode, p_al, n_b, n_full, apply_lds, s);
}

template <int CPT, bool AL>
hipError_t launch_global_p2(const CompressArgs &a, int64_t b0, int64_t b1, int64_t n_full, hipStream_t s) {
  const int64_t f1 = std::min(b1, n_full);
  if (CPT <= 4 && AL && f1 > b0) {
    constexpr int C4 = CPT <= 4 ? CPT : 4;
    hipLaunchKernelGGL((compress_full_kernel<C4, true, kQGlobal2>), dim3((unsigned)(f1 - b0)), dim3(kThreads), 0, s,
                       a, b0);
  }
  const int64_t g0 = std::max(b0, (CPT <= 4 && AL) ? n_full : (int64_t)0);
  if (b1 > g0)
    hipLaunchKernelGGL((compress_kernel<CPT, AL, true, kQGlobal2>), dim3((unsigned)(b1 - g0)), dim3(kThreads), 0, s,
                       a, g0);
  return hipGetLastError();
}

hipError_t dispatch_global_p2(int cpt, bool aligned, const CompressArgs &a, int64_t b0, int64_t b1, int64_t n_full,
                              hipStream_t s) {
  switch (cpt) {
    case 1: return aligned ? launch_global_p2<1, true>(a, b0, b1, n_full, s) : launch_global_p2<1, false>(a, b0, b1, n_full, s);
    case 2: return aligned ? launch_global_p2<2, true>(a, b0, b1, n_full, s) : launch_global_p2<2, false>(a, b0, b1, n_full, s);
    case 4: return aligned ? launch_global_p2<4, true>(a, b0, b1, n_full, s) : launch_global_p2<4, false>(a, b0, b1, n_full, s);
    default: return aligned ? launch_global_p2<8, true>(a, b0, b1, 0, s) : launch_global_p2<8, false>(a, b0, b1, 0, s);
  }
}


// The update kernels a step uses: column-sorted where the block's window fits
// them, unless MA_FLAG_ROW_SUMS asks for the row-by-row sums.  Full blocks
// run step_csu_kernel (column sums) where step_full_kernel's LDS cannot hold
// the window, for the dense update (decay), and for fp32 parameters from
// kCsuFusedMinWindow rows up; step_full_kernel (row-by-row sums, window
// preloaded during the compressor's staging) otherwise.  Measured (ms per
// step, column sums vs row sums, one process): m = 10: 7B 15.13 vs 15.50 and
// 13.18 vs 13.10 on two boxes, BERT-Base 0.291 vs 0.304, OPT-1.3B 2.96 vs
// 3.04, 13B 25.40 vs 25.25; 7B with decay 0.01 15.10 vs 17.50 (bf16 13.59 vs
// 16.40); 7B bf16 without decay 11.45 vs 11.13; 13B m = 4 20.4 vs 19.6, m = 1
// 16.75 vs 15.80; at m = 20 and 37 step_csu_kernel against the two kernels
// with row sums, when it came: 33.3 and 38.8 vs 33.7 and 69.9.
constexpr int kCsuFusedMinWindow = 10;

UpdLaunch upd_launch(const ma_ctx *h, bool dense = false, bool bf = false) {
  const bool csu = h->csu_ok && !(h->flags & MA_FLAG_ROW_SUMS);
  const bool prefer = dense || (!bf && h->m >= kCsuFusedMinWindow);
  const bool fcsu = csu && h->fused_csu_ok && (!h->fused_ok || prefer);
  const bool thl = fcsu && !bf && h->thl_n > 0 && !(h->flags & (MA_FLAG_FORCE_SPARSE | MA_FLAG_FORCE_DENSE));
  return UpdLaunch{csu, csu ? h->csu_lds : h->apply_lds, fcsu, h->fused_csu_lds, thl};
}

ApplyArgs make_apply_args(const ma_ctx *h, int64_t t, float c1, float c2, float decay) {
  ApplyArgs a{};
  a.G = h->window;
  a.off_tab = h->off_tab;
  a.betapow = h->betapow;
  a.d = h->d;
  a.k = h->k;
  a.n_b = h->n_b;
  a.B = h->B;
  a.m = h->m;
  a.tm = (int32_t)(t % h->m);
  a.cap = h->cap;
  a.ent_cap = h->ent_cap;
  a.csu_slots = h->csu_slots;
  a.fused_union_words = h->fused_union_words;
  a.thl_off = h->thl_off;
  a.thl_n = h->thl_n;
  a.c1 = c1;
  a.c2 = c2;
  a.lr = h->lr;
  a.eps = h->eps;
  a.decay = decay;
  return a;
}

}  // namespace

extern "C" {

int ma_last_error(void) { return g_err; }
const char *ma_last_error_message(void) { return g_msg; }

ma_ctx *ma_create(int64_t d, int32_t B_d, int64_t k, int32_t m, int32_t b, float beta1, float beta2,
                  float eps, float lr, float wd, uint64_t seed) {
  clear_error();
  if (d < 1) { fail(MA_EINVAL, "d must be >= 1 (got %lld)", (long long)d); return nullptr; }
  if (B_d < 1 || B_d >= 32767) { fail(MA_EINVAL, "B_d must be in [1, 32766] (got %d)", B_d); return nullptr; }
  if (k < 0 || k > d) { fail(MA_EINVAL, "k must be in [0, d] (got %lld)", (long long)k); return nullptr; }
  if (m < 1) { fail(MA_EINVAL, "m must be >= 1 (got %d)", m); return nullptr; }
  if (m > kMaxWindow) {
    fail(MA_EUNSUPPORTED, "windows of more than %d rows are not built (got m = %d)", kMaxWindow, m);
    return nullptr;
  }
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f)) {
    fail(MA_EINVAL, "betas must be in [0, 1)");
    return nullptr;
  }
  if (!(eps > 0.f) || !std::isfinite(eps)) { fail(MA_EINVAL, "eps must be positive and finite"); return nullptr; }
  if (!std::isfinite(lr)) { fail(MA_EINVAL, "lr must be finite"); return nullptr; }
  if (!(wd >= 0.f) || !std::isfinite(wd)) { fail(MA_EINVAL, "wd must be >= 0 and finite"); return nullptr; }
  if (b != 4) { fail(MA_EUNSUPPORTED, "only b = 4 bit error quantization is built (got b = %d)", b); return nullptr; }

  ma_ctx *h = new (std::nothrow) ma_ctx;
  if (!h) { fail(MA_ENOMEM, "host allocation failed"); return nullptr; }
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    fail(MA_EHIP, "no HIP device");
    return nullptr;
  }
  h->d = d; h->B = B_d; h->k = k; h->m = m; h->b = b;
  h->beta1 = beta1; h->beta2 = beta2; h->eps = eps; h->lr = lr; h->wd = wd; h->seed = seed;
  h->n_b = (d + B_d - 1) / B_d;
  h->cpt = B_d <= 4096 ? 1 : B_d <= 8192 ? 2 : B_d <= 16384 ? 4 : 8;

  // per-block window offsets floor(k*s_j/d), j = 0..n_b (s_{n_b} = d)
  std::vector<int64_t> off((size_t)h->n_b + 1);
  int64_t kb_max = 0;
  for (int64_t j = 0; j <= h->n_b; ++j) {
    const int64_t sj = j < h->n_b ? j * (int64_t)B_d : d;
    off[(size_t)j] = floor_mul_div(k, sj, d);
    if (j > 0) kb_max = std::max(kb_max, off[(size_t)j] - off[(size_t)j - 1]);
  }
  std::vector<float> bp(2 * (size_t)m);
  for (int32_t r = 0; r < m; ++r) {
    bp[(size_t)r] = (float)std::pow((double)beta1, (double)r);
    bp[(size_t)m + r] = (float)std::pow((double)beta2, (double)r);
  }
  // The update kernel's LDS: bitmap and slot bases (8 bytes per 32 positions),
  // the decay factors (8 bytes per window row), the block's window entries
  // when they fit in 5/8 of the budget (the rows are then read from global
  // memory once, not once per row pass), and 10 bytes per slot for at most
  // min(B_d, m*kb_max) touched positions.
  const int W = h->cpt * kChunkSpan / 32;
  const int64_t ents = (int64_t)m * kb_max;
  h->ent_cap = (4 * ents <= (int64_t)kApplyLdsLimit * 5 / 8) ? (int)ents : 0;
  const int64_t umax = std::min<int64_t>((int64_t)B_d, ents);
  const int64_t cap_limit =
      ((int64_t)kApplyLdsLimit - 8 * (int64_t)W - 8 * (int64_t)m - 4 * (int64_t)h->ent_cap) / 10;
  h->cap = (int)std::max<int64_t>(1, std::min<int64_t>(umax, cap_limit));
  h->apply_lds = 8 * (size_t)W + 8 * (size_t)m + 4 * (size_t)h->ent_cap + 10 * (size_t)h->cap;
  // expected fraction of positions present in a full window: 1 - (1 - k/d)^m
  h->dense_default = false;   // measured: gathering touched parameters wins at m = 1 and m = 10
  // fused kernel: full 4096-element chunks, CPT <= 4, the m window rows
  // (padded to 64 entries each) within kFusedEnt entries of LDS, and the 2m
  // decay factors within its kFusedBeta (checked on its own: with k = 0 the
  // rows take no space at any m)
  h->fused_ok = h->cpt <= 4 && B_d == h->cpt * kChunkSpan && (int64_t)m * ((kb_max + 63) & ~63LL) <= kFusedEnt &&
                2 * (int64_t)m <= kFusedBeta;
  // column-sorted update: every thread holds at most kCsuPerThread of the
  // block's m * k_b entries, its LDS (bitmap, slot bases, decay factors, a
  // word per slot and per entry) within the budget, keys of row << 16
  const int64_t csu_slots = std::min<int64_t>((int64_t)B_d, ents);
  h->csu_lds = 4 * (2 * (size_t)W + 2 * (size_t)m + (size_t)csu_slots + (size_t)ents);
  h->csu_ok = ents <= (int64_t)kThreads * kCsuPerThread && h->csu_lds <= kApplyLdsLimit && m <= 65535;
  h->csu_slots = (int32_t)csu_slots;
  // the fused kernel with the column-sorted update: one LDS buffer for the
  // compressor (CompressSmem + staging) and then the update, plus the new
  // window row; within a third of a CU's LDS
  {
    size_t comp_words = 0;
    switch (h->cpt) {
      case 1: comp_words = ((sizeof(CompressSmem<1>) + 15) / 16) * 4 + sizeof(FullBlockStage<1>) / 4; break;
      case 2: comp_words = ((sizeof(CompressSmem<2>) + 15) / 16) * 4 + sizeof(FullBlockStage<2>) / 4; break;
      default: comp_words = ((sizeof(CompressSmem<4>) + 15) / 16) * 4 + sizeof(FullBlockStage<4>) / 4; break;
    }
    const size_t union_words = std::max(comp_words, h->csu_lds / 4);
    h->fused_union_words = (int32_t)union_words;
    h->fused_csu_lds = 4 * (union_words + (size_t)kb_max);
    h->fused_csu_ok = h->csu_ok && h->cpt <= 4 && B_d == h->cpt * kChunkSpan && h->fused_csu_lds <= kFusedCsuLdsLimit;
    // fp32 parameters through LDS in the fused kernel, for windows of at most
    // four entries per thread (m * k_b <= 2048: m <= 12 at k = d/100 and
    // B_d = 16384); with longer windows the gather measured faster (LLaMA-2-13B
    // m = 20: 30.8 against 32.5 ms, m = 37: 39.6 against 42.8).  The chunk:
    // the largest power-of-two part of the block (at least 4 * kThreads
    // floats) that fits behind the update's bitmap, slot bases, decay factors
    // and slots (over the window entries, which are summed by then), 16-byte
    // aligned, within the static buffer
    const size_t thl_off = (2 * (size_t)W + 2 * (size_t)m + (size_t)csu_slots + 3) & ~(size_t)3;
    if (h->fused_csu_ok && ents <= 4 * (int64_t)kThreads)
      for (int64_t n = B_d; n >= 4 * kThreads; n /= 2)
        if (thl_off + (size_t)n <= (size_t)kFusedCsuWords) {
          h->thl_off = (int32_t)thl_off;
          h->thl_n = (int32_t)n;
          break;
        }
  }
  h->chunks = h->n_b >= 8192 ? 8 : 1;

  h->codes_bytes = (size_t)((d + 1) / 2);
  h->codes_alloc = (h->codes_bytes + 15) & ~(size_t)15;
  const size_t stats_b = 8 * (size_t)h->n_b;
  const size_t win_b = 4 * (size_t)m * (size_t)k;
  bool ok = hipMalloc(&h->codes, h->codes_alloc) == hipSuccess &&
            hipMalloc(&h->stats, stats_b) == hipSuccess &&
            hipMalloc(&h->window, win_b ? win_b : 4) == hipSuccess &&
            hipMalloc(&h->off_tab, 8 * off.size()) == hipSuccess &&
            hipMalloc(&h->betapow, 4 * bp.size()) == hipSuccess &&
            hipMalloc(&h->touched, kTouchedSlots * sizeof(unsigned long long)) == hipSuccess &&
            hipMalloc(&h->deferred, 8 * (size_t)h->n_b) == hipSuccess &&
            hipMalloc(&h->n_deferred, 64 * sizeof(unsigned int)) == hipSuccess &&
            hipMalloc(&h->blkmm, 8 * (size_t)h->n_b) == hipSuccess &&
            hipMalloc(&h->selinfo, 8 * (size_t)h->n_b) == hipSuccess &&
            hipMalloc(&h->gmm, 8) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    free_all(h);
    delete h;
    fail(MA_ENOMEM, "device allocation of the optimizer state failed (d = %lld, m = %d, k = %lld)",
         (long long)d, m, (long long)k);
    return nullptr;
  }
  ok = hipMemset(h->codes, 0, h->codes_alloc) == hipSuccess &&
       hipMemset(h->stats, 0, stats_b) == hipSuccess &&
       hipMemset(h->window, 0, win_b ? win_b : 4) == hipSuccess &&
       hipMemcpy(h->off_tab, off.data(), 8 * off.size(), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemcpy(h->betapow, bp.data(), 4 * bp.size(), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemset(h->touched, 0, kTouchedSlots * sizeof(unsigned long long)) == hipSuccess &&
       hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    const hipError_t e = hipGetLastError();
    free_all(h);
    delete h;
    fail(MA_EHIP, "initialising the optimizer state failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  // ma_step_noalloc's scratch: its address on this device, once per device
  // (a failure here only disables ma_step_noalloc on this handle)
  h->na_scratch = static_cast<unsigned char *>(noalloc_scratch(h->device));
  return h;
}

void ma_destroy(ma_ctx *h) {
  if (!h) return;
  DeviceGuard g(h->device);
  free_all(h);
  delete h;
}

size_t ma_state_bytes(const ma_ctx *h) {
  if (!h) return 0;
  return h->codes_bytes + 4 * (size_t)h->m * (size_t)h->k;
}

size_t ma_aux_bytes(const ma_ctx *h) {
  if (!h) return 0;
  return 8 * (size_t)h->n_b + 8 * ((size_t)h->n_b + 1) + 8 * (size_t)h->m +
         (h->codes_alloc - h->codes_bytes) + kTouchedSlots * sizeof(unsigned long long) +
         8 * (size_t)h->n_b + 64 * sizeof(unsigned int) + 16 * (size_t)h->n_b + 8;
}

int64_t ma_get_step(const ma_ctx *h) { return h ? h->t : -1; }
int64_t ma_num_blocks(const ma_ctx *h) { return h ? h->n_b : -1; }

int ma_set_step(ma_ctx *h, int64_t t) {
  clear_error();
  if (!h || t < 0) return fail(MA_EINVAL, "ma_set_step: null handle or negative step");
  h->t = t;
  return MA_OK;
}

int ma_set_flags(ma_ctx *h, uint32_t flags) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_set_flags: null handle");
  if (flags & ~(MA_FLAG_NO_EF | MA_FLAG_FORCE_DENSE | MA_FLAG_FORCE_SPARSE | MA_FLAG_UNFUSED | MA_FLAG_GLOBAL_QUANT |
                MA_FLAG_ROW_SUMS))
    return fail(MA_EINVAL, "ma_set_flags: unknown flag bits");
  h->flags = flags;
  return MA_OK;
}

int ma_set_lr(ma_ctx *h, float lr) {
  clear_error();
  if (!h || !std::isfinite(lr)) return fail(MA_EINVAL, "ma_set_lr: null handle or non-finite lr");
  h->lr = lr;
  return MA_OK;
}

namespace {

// One step for fp32 (bf false) or bfloat16 (bf true) parameters.  noalloc:
// the ma_step_noalloc variant: the step's scratch comes from the static
// `scratch` array instead of the handle's buffers, and every launch goes to
// `stream` (no side stream, no events): nothing is created or allocated.
int step_impl(ma_ctx *h, void *params, bool bf, const uint16_t *grads, hipStream_t stream, bool noalloc = false) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_step: null handle");
  if (!params || !grads) return fail(MA_EINVAL, "ma_step: null params or grads");
  if (((uintptr_t)params & (bf ? 1u : 3u)) || ((uintptr_t)grads & 1u))
    return fail(MA_EINVAL, "ma_step: params must be element-aligned and grads 2-byte aligned");
  if (noalloc && h->n_b > kNoAllocMaxBlocks)
    return fail(MA_EUNSUPPORTED, "ma_step_noalloc: %lld blocks exceed its static scratch of %lld blocks",
                (long long)h->n_b, (long long)kNoAllocMaxBlocks);
  if (noalloc && !h->na_scratch)
    return fail(MA_EHIP, "ma_step_noalloc: the address of its scratch on device %d is unknown", h->device);
  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(MA_EHIP, "ma_step: cannot select device %d", h->device);
  // the step's scratch: the deferred-block list and counters, the global
  // quantizer's per-block min / max, cut and pair
  int64_t *q_deferred = noalloc ? reinterpret_cast<int64_t *>(h->na_scratch + kNaDeferred) : h->deferred;
  unsigned int *q_counts = noalloc ? reinterpret_cast<unsigned int *>(h->na_scratch + kNaCounts) : h->n_deferred;
  float *q_blkmm = noalloc ? reinterpret_cast<float *>(h->na_scratch + kNaBlkmm) : h->blkmm;
  uint32_t *q_selinfo = noalloc ? reinterpret_cast<uint32_t *>(h->na_scratch + kNaSelinfo) : h->selinfo;
  float *q_gmm = noalloc ? reinterpret_cast<float *>(h->na_scratch + kNaGmm) : h->gmm;
  const bool timing = h->timing && !noalloc;

  const int64_t t = h->t + 1;
  const double b1 = (double)h->beta1, b2 = (double)h->beta2;
  const float c1 = (float)((1.0 - b1) / (1.0 - std::pow(b1, (double)t)));
  const float c2 = (float)((1.0 - b2) / (1.0 - std::pow(b2, (double)t)));
  const float decay = (float)(1.0 - (double)h->lr * (double)h->wd);

  CompressArgs ca{};
  ca.g = grads;
  ca.ef = h->codes;
  ca.stats = h->stats;
  ca.G = h->window;
  ca.off_tab = h->off_tab;
  ca.d = h->d;
  ca.k = h->k;
  ca.n_b = h->n_b;
  ca.t = t;
  ca.row_base = (t % h->m) * h->k;
  ca.seed = h->seed;
  ca.B = h->B;
  ca.deferred = q_deferred;
  ca.n_deferred = q_counts;

  ApplyArgs aa = make_apply_args(h, t, c1, c2, decay);
  aa.theta = bf ? nullptr : static_cast<float *>(params);
  aa.theta16 = bf ? static_cast<uint16_t *>(params) : nullptr;
  aa.touched = h->count_touched ? h->touched : nullptr;

  const bool b8 = (h->B % 8) == 0;
  const bool g_al = b8 && (((uintptr_t)grads & 15u) == 0);
  const bool p_al = b8 && (((uintptr_t)params & 15u) == 0);
  // Update mode: decoupled decay touches every parameter (dense); otherwise
  // only the touched parameters are gathered by slot (sparse), which measured
  // faster than streaming at both m = 1 and m = 10 on the LLaMA-2-7B shape.
  int mode = h->dense_default ? kModeDense : kModeSparse;
  if (h->flags & MA_FLAG_FORCE_DENSE) mode = kModeDense;
  if (h->flags & MA_FLAG_FORCE_SPARSE) mode = kModeSparse;
  if (decay != 1.0f) mode = kModeDense;
  const UpdLaunch ul = upd_launch(h, mode == kModeDense, bf);

  // The blocks are cut into h->chunks ranges.  Compress of range i runs on
  // the caller's stream; the update of range i runs on the library's side
  // stream once compress i is done, so it overlaps compress i+1 (one kernel
  // is bound by arithmetic, the other by memory).  The caller's stream waits
  // for the side stream at the end: ma_step stays one asynchronous step on
  // `stream`.
  const int64_t n_full = (g_al && h->B == h->cpt * kChunkSpan) ? h->d / h->B : 0;
  const bool ef = !(h->flags & MA_FLAG_NO_EF);
  hipError_t e = hipSuccess;

  // Global quantizer: the compressor's first pass (selection, window row,
  // each block's min / max and cut) and the global min / max over all blocks;
  // then the second pass (codes and statistics) on the caller's stream and,
  // concurrently on the side stream, the update, which reads only the window
  // and the parameters: neither writes what the other reads.
  if (ef && (h->flags & MA_FLAG_GLOBAL_QUANT)) {
    ca.blkmm = q_blkmm;
    ca.selinfo = q_selinfo;
    ca.gmm = q_gmm;
    if (!noalloc && !ensure_pipeline(h, 1)) return fail(MA_EHIP, "ma_step: creating the side stream failed");
    hipEvent_t tg[6] = {};
    if (timing && !take_events(h, tg, 6)) return fail(MA_EHIP, "ma_step: hipEventCreate failed");
    hipEvent_t t0 = tg[0], t1 = tg[1], t2 = tg[2], t3 = tg[3], t4 = tg[4], t5 = tg[5];
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, q_counts, 1);
    // Full blocks: the first pass fused with the update (the update needs only
    // the block's window, which the first pass completes), then the second
    // pass alone.  Neither writes what the other reads.  The dense update
    // (decoupled decay) is fused for 16-byte aligned parameters.
    if ((ul.fused_csu || h->fused_ok) && n_full > 0 && (mode == kModeSparse || p_al) && !(h->flags & MA_FLAG_UNFUSED)) {
      if (t0) (void)hipEventRecord(t0, stream);
      e = dispatch_fused_global1(h->cpt, bf, ca, aa, mode, p_al, h->n_b, n_full, ul, stream);
      if (t1) (void)hipEventRecord(t1, stream);
      if (e == hipSuccess) {
        if (t2) (void)hipEventRecord(t2, stream);
        e = dispatch_global_p2(h->cpt, g_al, ca, 0, h->n_b, n_full, stream);
        if (t3) (void)hipEventRecord(t3, stream);
      }
      if (t0) {
        h->events.push_back({2, t0, t1});
        h->events.push_back({0, t2, t3});
        h->pool.push_back(t4);
        h->pool.push_back(t5);
      }
      if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
      h->t = t;
      h->last_c1 = c1;
      h->last_c2 = c2;
      return MA_OK;
    }
    if (noalloc) {
      // everything on the caller's stream: pass 1, the update, pass 2
      e = dispatch_global_p1(h->cpt, g_al, ca, h->n_b, n_full, stream);
      if (e == hipSuccess) e = dispatch_apply(h->cpt, mode, p_al, aa, h->n_b, ul, stream, bf);
      if (e == hipSuccess) e = dispatch_global_p2(h->cpt, g_al, ca, 0, h->n_b, n_full, stream);
      if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
      h->t = t;
      h->last_c1 = c1;
      h->last_c2 = c2;
      return MA_OK;
    }
    if (t0) (void)hipEventRecord(t0, stream);
    e = dispatch_global_p1(h->cpt, g_al, ca, h->n_b, n_full, stream);
    if (t1) (void)hipEventRecord(t1, stream);
    if (e == hipSuccess) e = hipEventRecord(h->fork_ev, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork_ev, 0);
    if (e == hipSuccess) {
      if (t4) (void)hipEventRecord(t4, h->side);
      e = dispatch_apply(h->cpt, mode, p_al, aa, h->n_b, ul, h->side, bf);
      if (t5) (void)hipEventRecord(t5, h->side);
    }
    if (e == hipSuccess) {
      if (t2) (void)hipEventRecord(t2, stream);
      e = dispatch_global_p2(h->cpt, g_al, ca, 0, h->n_b, n_full, stream);
      if (t3) (void)hipEventRecord(t3, stream);
    }
    {
      hipError_t e2 = hipEventRecord(h->join_ev, h->side);
      if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, h->join_ev, 0);
      if (e == hipSuccess) e = e2;
    }
    if (t0) {
      h->events.push_back({0, t0, t1});
      h->events.push_back({0, t2, t3});
      h->events.push_back({1, t4, t5});
    }
    if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
    h->t = t;
    h->last_c1 = c1;
    h->last_c2 = c2;
    return MA_OK;
  }

  // Fused path: every full block runs compress and update in one workgroup;
  // a partial last block (if any) runs the two kernels, on the library's
  // side stream concurrently with the fused kernel (its block, window segment
  // and parameters are its own; the side stream joins the caller's before
  // ma_step returns), or after it on the caller's stream for the
  // no-allocation entry point.  The dense update (decoupled decay) is fused
  // for 16-byte aligned parameters.
  if ((ul.fused_csu || h->fused_ok) && n_full > 0 && (mode == kModeSparse || p_al) && !(h->flags & MA_FLAG_UNFUSED)) {
    const bool part = n_full < h->n_b;
    const bool beside = part && !noalloc;
    if (beside && !ensure_pipeline(h, 1)) return fail(MA_EHIP, "ma_step: creating the side stream failed");
    hipEvent_t tf[2] = {};
    if (timing && !take_events(h, tf, 2)) return fail(MA_EHIP, "ma_step: hipEventCreate failed");
    hipEvent_t t0 = tf[0], t1 = tf[1];
    ApplyArgs at = aa;
    at.first_block = n_full;
    hipStream_t ps = beside ? h->side : stream;   // the partial block's stream
    if (beside) {
      e = hipEventRecord(h->fork_ev, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork_ev, 0);
      if (e == hipSuccess) e = dispatch_compress(h->cpt, g_al, ef, ca, n_full, h->n_b, n_full, ps);
      if (e == hipSuccess) e = dispatch_apply(h->cpt, mode, p_al, at, h->n_b - n_full, ul, ps, bf);
    }
    if (e == hipSuccess) {
      hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, q_counts, 1);
      e = hipGetLastError();
    }
    if (t0) (void)hipEventRecord(t0, stream);
    if (e == hipSuccess) e = dispatch_fused(h->cpt, ef, mode == kModeDense, p_al, ca, aa, n_full, ul, stream, bf);
    if (t1) {
      (void)hipEventRecord(t1, stream);
      h->events.push_back({2, t0, t1});
    }
    if (e == hipSuccess && part && !beside) {
      e = dispatch_compress(h->cpt, g_al, ef, ca, n_full, h->n_b, n_full, stream);
      if (e == hipSuccess) e = dispatch_apply(h->cpt, mode, p_al, at, h->n_b - n_full, ul, stream, bf);
    }
    if (beside) {
      hipError_t e2 = hipEventRecord(h->join_ev, h->side);
      if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, h->join_ev, 0);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
    h->t = t;
    h->last_c1 = c1;
    h->last_c2 = c2;
    return MA_OK;
  }

  const int chunks = noalloc ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>(h->chunks, h->n_b));
  if (chunks > 1 && !ensure_pipeline(h, chunks)) return fail(MA_EHIP, "ma_step: creating the side stream failed");
  // per range: compress start / end, update start / end
  std::vector<hipEvent_t> tp(timing ? 4 * (size_t)chunks : 0, nullptr);
  if (!tp.empty() && !take_events(h, tp.data(), (int)tp.size())) return fail(MA_EHIP, "ma_step: hipEventCreate failed");
  hipStream_t upd = chunks > 1 ? h->side : stream;
  if (chunks > 1) {
    e = hipEventRecord(h->fork_ev, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork_ev, 0);
  }
  // every range's deferred-block counter starts at zero
  if (e == hipSuccess && n_full > 0) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, q_counts, chunks);
    e = hipGetLastError();
  }
  for (int i = 0; i < chunks && e == hipSuccess; ++i) {
    const int64_t b0 = h->n_b * i / chunks, b1 = h->n_b * (i + 1) / chunks;
    CompressArgs cai = ca;
    cai.deferred = q_deferred + b0;
    cai.n_deferred = q_counts + i;
    hipEvent_t t0 = tp.empty() ? nullptr : tp[4 * (size_t)i], t1 = tp.empty() ? nullptr : tp[4 * (size_t)i + 1];
    if (t0) (void)hipEventRecord(t0, stream);
    e = dispatch_compress(h->cpt, g_al, ef, cai, b0, b1, n_full, stream);
    if (t1) {
      (void)hipEventRecord(t1, stream);
      h->events.push_back({0, t0, t1});
      tp[4 * (size_t)i] = tp[4 * (size_t)i + 1] = nullptr;
    }
    if (e != hipSuccess) break;
    if (chunks > 1) {
      e = hipEventRecord(h->chunk_ev[i], stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->chunk_ev[i], 0);
      if (e != hipSuccess) break;
    }
    ApplyArgs aai = aa;
    aai.first_block = b0;
    hipEvent_t u0 = tp.empty() ? nullptr : tp[4 * (size_t)i + 2], u1 = tp.empty() ? nullptr : tp[4 * (size_t)i + 3];
    if (u0) (void)hipEventRecord(u0, upd);
    e = dispatch_apply(h->cpt, mode, p_al, aai, b1 - b0, ul, upd, bf);
    if (u1) {
      (void)hipEventRecord(u1, upd);
      h->events.push_back({1, u0, u1});
      tp[4 * (size_t)i + 2] = tp[4 * (size_t)i + 3] = nullptr;
    }
  }
  // events of ranges a failed launch left unused go back to the pool
  for (hipEvent_t ev : tp)
    if (ev) h->pool.push_back(ev);
  if (chunks > 1) {
    hipError_t e2 = hipEventRecord(h->join_ev, h->side);
    if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, h->join_ev, 0);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
  h->t = t;
  h->last_c1 = c1;
  h->last_c2 = c2;
  return MA_OK;
}

}  // namespace

int ma_step(ma_ctx *h, float *params, const uint16_t *grads, hipStream_t stream) {
  return step_impl(h, params, false, grads, stream);
}

int ma_step_bf16(ma_ctx *h, uint16_t *params, const uint16_t *grads, hipStream_t stream) {
  return step_impl(h, params, true, grads, stream);
}

int ma_step_noalloc(ma_ctx *h, float *params, const uint16_t *grads, hipStream_t stream) {
  return step_impl(h, params, false, grads, stream, true);
}

int ma_adamw_step(int64_t n, int64_t t, float beta1, float beta2, float eps, float lr, float wd, float *theta,
                  const uint16_t *grads, float *m, float *v, hipStream_t stream) {
  clear_error();
  if (n < 0 || t < 1) return fail(MA_EINVAL, "ma_adamw_step: n must be >= 0 and t >= 1");
  if (n == 0) return MA_OK;
  if (!theta || !grads || !m || !v) return fail(MA_EINVAL, "ma_adamw_step: null pointer");
  if (((uintptr_t)theta & 3u) || ((uintptr_t)m & 3u) || ((uintptr_t)v & 3u) || ((uintptr_t)grads & 1u))
    return fail(MA_EINVAL, "ma_adamw_step: misaligned pointer");
  AdamwArgs a;
  a.theta = theta;
  a.g = grads;
  a.m = m;
  a.v = v;
  a.n = n;
  a.b1 = beta1;
  a.b2 = beta2;
  a.omb1 = (float)(1.0 - (double)beta1);
  a.omb2 = (float)(1.0 - (double)beta2);
  a.r1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)t)));
  a.r2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)t)));
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  a.lr = lr;
  a.eps = eps;
  const bool al = (((uintptr_t)theta | (uintptr_t)m | (uintptr_t)v | (uintptr_t)grads) & 15u) == 0;
  const int64_t runs = (n + 7) / 8;
  const unsigned grid = (unsigned)std::min<int64_t>((runs + kAdamwThreads - 1) / kAdamwThreads, 256 * 16);
  if (al)
    hipLaunchKernelGGL(adamw_kernel<true>, dim3(grid), dim3(kAdamwThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(adamw_kernel<false>, dim3(grid), dim3(kAdamwThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MA_EHIP, "ma_adamw_step: launch failed: %s", hipGetErrorString(e));
  return MA_OK;
}

int ma_adamw8_step(int64_t n, int64_t t, float beta1, float beta2, float eps, float lr, float wd, float *theta,
                   const uint16_t *grads, int8_t *cm, uint8_t *cv, float *sm, float *sr, hipStream_t stream) {
  clear_error();
  if (n < 0 || t < 1) return fail(MA_EINVAL, "ma_adamw8_step: n must be >= 0 and t >= 1");
  if (n == 0) return MA_OK;
  if (!theta || !grads || !cm || !cv || !sm || !sr) return fail(MA_EINVAL, "ma_adamw8_step: null pointer");
  if (((uintptr_t)theta & 3u) || ((uintptr_t)grads & 1u) || ((uintptr_t)sm & 3u) || ((uintptr_t)sr & 3u))
    return fail(MA_EINVAL, "ma_adamw8_step: misaligned pointer");
  Adamw8Args a;
  a.theta = theta;
  a.g = grads;
  a.cm = cm;
  a.cv = cv;
  a.sm = sm;
  a.sr = sr;
  a.n = n;
  a.b1 = beta1;
  a.b2 = beta2;
  a.omb1 = (float)(1.0 - (double)beta1);
  a.omb2 = (float)(1.0 - (double)beta2);
  a.r1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)t)));
  a.r2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)t)));
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  a.lr = lr;
  a.eps = eps;
  // every lane's run of 4 starts at a multiple of 4 elements
  const bool al = ((uintptr_t)theta & 15u) == 0 && ((uintptr_t)grads & 7u) == 0 && ((uintptr_t)cm & 3u) == 0 &&
                  ((uintptr_t)cv & 3u) == 0;
  const int64_t nq = (n + kQ8Block - 1) / kQ8Block;
  const unsigned grid = (unsigned)std::min<int64_t>((nq + 3) / 4, 256 * 32);
  if (al)
    hipLaunchKernelGGL(adamw8_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(adamw8_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MA_EHIP, "ma_adamw8_step: launch failed: %s", hipGetErrorString(e));
  return MA_OK;
}

int ma_read_state(const ma_ctx *h, int which, uint64_t byte_offset, uint64_t nbytes, void *host_dst) {
  clear_error();
  if (!h || !host_dst) return fail(MA_EINVAL, "ma_read_state: null argument");
  const uint8_t *base;
  uint64_t size;
  switch (which) {
    case MA_STATE_CODES: base = h->codes; size = h->codes_bytes; break;
    case MA_STATE_STATS: base = reinterpret_cast<const uint8_t *>(h->stats); size = 8ull * h->n_b; break;
    case MA_STATE_WINDOW: base = reinterpret_cast<const uint8_t *>(h->window); size = 4ull * h->m * h->k; break;
    default: return fail(MA_EINVAL, "ma_read_state: unknown state buffer %d", which);
  }
  if (byte_offset > size || nbytes > size - byte_offset) return fail(MA_EINVAL, "ma_read_state: range outside the buffer");
  if (!nbytes) return MA_OK;
  DeviceGuard guard(h->device);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(host_dst, base + byte_offset, nbytes, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MA_EHIP, "ma_read_state: copy failed: %s", hipGetErrorString(hipGetLastError()));
  return MA_OK;
}

int ma_write_state(ma_ctx *h, int which, uint64_t byte_offset, uint64_t nbytes, const void *host_src) {
  clear_error();
  if (!h || !host_src) return fail(MA_EINVAL, "ma_write_state: null argument");
  uint8_t *base;
  uint64_t size;
  switch (which) {
    case MA_STATE_CODES: base = h->codes; size = h->codes_bytes; break;
    case MA_STATE_STATS: base = reinterpret_cast<uint8_t *>(h->stats); size = 8ull * h->n_b; break;
    case MA_STATE_WINDOW: base = reinterpret_cast<uint8_t *>(h->window); size = 4ull * h->m * h->k; break;
    default: return fail(MA_EINVAL, "ma_write_state: unknown state buffer %d", which);
  }
  if (byte_offset > size || nbytes > size - byte_offset) return fail(MA_EINVAL, "ma_write_state: range outside the buffer");
  if (!nbytes) return MA_OK;
  DeviceGuard guard(h->device);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(base + byte_offset, host_src, nbytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    return fail(MA_EHIP, "ma_write_state: copy failed: %s", hipGetErrorString(hipGetLastError()));
  return MA_OK;
}

int ma_export_state(const ma_ctx *h, void *codes, void *stats, void *window, int64_t *t) {
  clear_error();
  if (!h || !codes || !stats || !t) return fail(MA_EINVAL, "ma_export_state: null argument");
  const uint64_t wbytes = 4ull * h->m * h->k;
  if (wbytes && !window) return fail(MA_EINVAL, "ma_export_state: null window buffer");
  int rc = ma_read_state(h, MA_STATE_CODES, 0, h->codes_bytes, codes);
  if (rc == MA_OK) rc = ma_read_state(h, MA_STATE_STATS, 0, 8ull * h->n_b, stats);
  if (rc == MA_OK && wbytes) rc = ma_read_state(h, MA_STATE_WINDOW, 0, wbytes, window);
  if (rc == MA_OK) *t = h->t;
  return rc;
}

int ma_import_state(ma_ctx *h, const void *codes, const void *stats, const void *window, int64_t t) {
  clear_error();
  if (!h || !codes || !stats) return fail(MA_EINVAL, "ma_import_state: null argument");
  if (t < 0) return fail(MA_EINVAL, "ma_import_state: negative step");
  const uint64_t wbytes = 4ull * h->m * h->k;
  if (wbytes && !window) return fail(MA_EINVAL, "ma_import_state: null window buffer");
  int rc = ma_write_state(h, MA_STATE_CODES, 0, h->codes_bytes, codes);
  if (rc == MA_OK) rc = ma_write_state(h, MA_STATE_STATS, 0, 8ull * h->n_b, stats);
  if (rc == MA_OK && wbytes) rc = ma_write_state(h, MA_STATE_WINDOW, 0, wbytes, window);
  if (rc == MA_OK) h->t = t;
  return rc;
}

int ma_debug_moments(ma_ctx *h, const int64_t *blocks, int64_t nblocks, float *mhat_out, float *vhat_out,
                     hipStream_t stream) {
  clear_error();
  if (!h || !blocks || !mhat_out || !vhat_out || nblocks < 0)
    return fail(MA_EINVAL, "ma_debug_moments: null argument");
  if (h->t < 1) return fail(MA_EINVAL, "ma_debug_moments: no step has run yet");
  if (nblocks == 0) return MA_OK;
  if (nblocks > 0x7fffffff) return fail(MA_EINVAL, "ma_debug_moments: too many blocks");
  for (int64_t q = 0; q < nblocks; ++q)
    if (blocks[q] < 0 || blocks[q] >= h->n_b) return fail(MA_EINVAL, "ma_debug_moments: block %lld out of range", (long long)blocks[q]);
  DeviceGuard guard(h->device);
  int64_t *dblocks = nullptr;
  if (hipMalloc(&dblocks, 8 * (size_t)nblocks) != hipSuccess) return fail(MA_ENOMEM, "ma_debug_moments: allocation failed");
  hipError_t e = hipMemcpyAsync(dblocks, blocks, 8 * (size_t)nblocks, hipMemcpyHostToDevice, stream);
  ApplyArgs a = make_apply_args(h, h->t, h->last_c1, h->last_c2, 1.0f);
  a.mhat = mhat_out;
  a.vhat = vhat_out;
  a.blocks = dblocks;
  if (e == hipSuccess) e = dispatch_apply(h->cpt, kModeMoments, false, a, nblocks, upd_launch(h), stream);
  // the block list must outlive the kernel
  const hipError_t e2 = hipStreamSynchronize(stream);
  (void)hipFree(dblocks);
  if (e != hipSuccess || e2 != hipSuccess)
    return fail(MA_EHIP, "ma_debug_moments: %s", hipGetErrorString(e != hipSuccess ? e : e2));
  return MA_OK;
}

namespace {

// Test hook for the first line of the step (first paragraph of the MicroAdam
// page): the accumulator a_t = f32(g_t) + Q^-1(e_t, delta_t, Delta_t) of the
// listed blocks, from the current codes and statistics, with the compressor's
// arithmetic (step (Delta - delta) / 15, then one fmaf and one add).  Row q of
// out holds block blocks[q]; positions past the block's end are 0.
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t *g, const uint8_t *codes, const float *stats,
                                                       const int64_t *blocks, int64_t d, int32_t B, int ef,
                                                       float *out) {
  const int64_t j = blocks[blockIdx.x];
  const int64_t s = j * (int64_t)B;
  const int64_t L = (d - s) < (int64_t)B ? (d - s) : (int64_t)B;
  float lo = 0.f, step = 0.f;
  if (ef) {
    lo = stats[2 * j];
    step = (stats[2 * j + 1] - lo) / 15.0f;
  }
  for (int i = (int)threadIdx.x; i < B; i += (int)blockDim.x) {
    float v = 0.f;
    if (i < L) {
      const int64_t gi = s + i;
      const float gf = __uint_as_float((uint32_t)g[gi] << 16);
      v = gf;
      if (ef) {
        const uint32_t code = (codes[gi >> 1] >> (4 * (int)(gi & 1))) & 15u;
        v = gf + fmaf((float)code, step, lo);
      }
    }
    out[(int64_t)blockIdx.x * B + i] = v;
  }
}

}  // namespace

int ma_debug_residual(ma_ctx *h, const uint16_t *grads, const int64_t *blocks, int64_t nblocks, float *a_out,
                      hipStream_t stream) {
  clear_error();
  if (!h || !grads || !blocks || !a_out || nblocks < 0)
    return fail(MA_EINVAL, "ma_debug_residual: null argument");
  if (nblocks == 0) return MA_OK;
  if (nblocks > 0x7fffffff) return fail(MA_EINVAL, "ma_debug_residual: too many blocks");
  for (int64_t q = 0; q < nblocks; ++q)
    if (blocks[q] < 0 || blocks[q] >= h->n_b)
      return fail(MA_EINVAL, "ma_debug_residual: block %lld out of range", (long long)blocks[q]);
  DeviceGuard guard(h->device);
  int64_t *dblocks = nullptr;
  if (hipMalloc(&dblocks, 8 * (size_t)nblocks) != hipSuccess) return fail(MA_ENOMEM, "ma_debug_residual: allocation failed");
  hipError_t e = hipMemcpyAsync(dblocks, blocks, 8 * (size_t)nblocks, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, grads,
                       (const uint8_t *)h->codes, (const float *)h->stats, (const int64_t *)dblocks, h->d, h->B,
                       (h->flags & MA_FLAG_NO_EF) ? 0 : 1, a_out);
    e = hipGetLastError();
  }
  // the block list must outlive the kernel
  const hipError_t e2 = hipStreamSynchronize(stream);
  (void)hipFree(dblocks);
  if (e != hipSuccess || e2 != hipSuccess)
    return fail(MA_EHIP, "ma_debug_residual: %s", hipGetErrorString(e != hipSuccess ? e : e2));
  return MA_OK;
}

int ma_set_timing(ma_ctx *h, int on) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_set_timing: null handle");
  DeviceGuard guard(h->device);
  if (hipDeviceSynchronize() != hipSuccess) return fail(MA_EHIP, "ma_set_timing: device synchronize failed");
  for (auto &ev : h->events) {
    h->pool.push_back(ev.start);
    h->pool.push_back(ev.end);
  }
  h->events.clear();
  for (int i = 0; i < kTimedKernels; ++i) {
    h->acc_ms[i] = 0;
    h->acc_n[i] = 0;
  }
  h->timing = on != 0;
  return MA_OK;
}

int ma_kernel_times(ma_ctx *h, double *ms_out, int64_t *launches_out, int nk) {
  clear_error();
  if (!h || !ms_out || !launches_out || nk < 0 || nk > kTimedKernels)
    return fail(MA_EINVAL, "ma_kernel_times: bad argument");
  DeviceGuard guard(h->device);
  for (auto &ev : h->events) {
    float ms = 0;
    if (hipEventSynchronize(ev.end) != hipSuccess || hipEventElapsedTime(&ms, ev.start, ev.end) != hipSuccess)
      return fail(MA_EHIP, "ma_kernel_times: reading an event failed");
    h->acc_ms[ev.kernel] += ms;
    h->acc_n[ev.kernel] += 1;
    h->pool.push_back(ev.start);
    h->pool.push_back(ev.end);
  }
  h->events.clear();
  for (int i = 0; i < nk; ++i) {
    ms_out[i] = h->acc_ms[i];
    launches_out[i] = h->acc_n[i];
  }
  return MA_OK;
}

int ma_get_pipeline(const ma_ctx *h) {
  return h ? (int)std::max<int64_t>(1, std::min<int64_t>(h->chunks, h->n_b)) : -1;
}

int ma_set_pipeline(ma_ctx *h, int chunks) {
  clear_error();
  if (!h || chunks < 1 || chunks > 64) return fail(MA_EINVAL, "ma_set_pipeline: chunks must be in [1, 64]");
  h->chunks = chunks;
  return MA_OK;
}

int ma_set_count_touched(ma_ctx *h, int on) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_set_count_touched: null handle");
  DeviceGuard guard(h->device);
  if (on && (hipDeviceSynchronize() != hipSuccess ||
             hipMemset(h->touched, 0, kTouchedSlots * sizeof(unsigned long long)) != hipSuccess ||
             hipDeviceSynchronize() != hipSuccess))
    return fail(MA_EHIP, "ma_set_count_touched: clearing the counter failed");
  h->count_touched = on != 0;
  return MA_OK;
}

int64_t ma_touched_count(ma_ctx *h) {
  clear_error();
  if (!h || !h->count_touched) return -1;
  DeviceGuard guard(h->device);
  std::vector<unsigned long long> v(kTouchedSlots);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(v.data(), h->touched, kTouchedSlots * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess) {
    fail(MA_EHIP, "ma_touched_count: copy failed");
    return -1;
  }
  unsigned long long sum = 0;
  for (auto x : v) sum += x;
  return (int64_t)sum;
}

}  // extern "C"
