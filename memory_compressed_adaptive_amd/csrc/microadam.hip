// Host runtime of libmicroadam: argument checks, state allocation, per-step
// constants and kernel launches on the caller's stream.  The C ABI is declared
// and documented in include/microadam.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "microadam.h"
#include "microadam_kernels.hpp"

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

// Largest LDS the update kernel asks for: two of its workgroups fit one CU.
constexpr size_t kApplyLdsLimit = 64 * 1024;

}  // namespace

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
  size_t apply_lds = 0;

  uint8_t *codes = nullptr;
  size_t codes_bytes = 0, codes_alloc = 0;
  float *stats = nullptr;
  uint32_t *window = nullptr;
  int64_t *off_tab = nullptr;
  float *betapow = nullptr;
  unsigned long long *touched = nullptr;
  bool count_touched = false;

  // last step's constants (for ma_debug_moments)
  float last_c1 = 0, last_c2 = 0;

  bool timing = false;
  struct Ev { hipEvent_t e[3]; };
  std::vector<Ev> events;   // recorded, not yet read
  std::vector<Ev> pool;     // free
  double acc_ms[2] = {0, 0};
  int64_t acc_n[2] = {0, 0};
};

namespace {

void free_all(ma_ctx *h) {
  if (!h) return;
  hipFree(h->codes);
  hipFree(h->stats);
  hipFree(h->window);
  hipFree(h->off_tab);
  hipFree(h->betapow);
  hipFree(h->touched);
  for (auto &ev : h->events)
    for (auto e : ev.e) hipEventDestroy(e);
  for (auto &ev : h->pool)
    for (auto e : ev.e) hipEventDestroy(e);
  h->events.clear();
  h->pool.clear();
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

template <int CPT, bool AL, bool EF>
hipError_t launch_compress(const CompressArgs &a, int64_t n_full, int64_t n_b, hipStream_t s) {
  if (CPT <= 4 && AL && n_full > 0)
    hipLaunchKernelGGL((compress_full_kernel<(CPT <= 4 ? CPT : 4), EF>), dim3((unsigned)n_full), dim3(kThreads), 0,
                       s, a);
  if (n_b > n_full)
    hipLaunchKernelGGL((compress_kernel<CPT, AL, EF>), dim3((unsigned)(n_b - n_full)), dim3(kThreads), 0, s, a,
                       n_full);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_compress_cpt(bool aligned, bool ef, const CompressArgs &a, int64_t n_full, int64_t n_b,
                               hipStream_t s) {
  if (ef)
    return aligned ? launch_compress<CPT, true, true>(a, n_full, n_b, s)
                   : launch_compress<CPT, false, true>(a, n_full, n_b, s);
  return aligned ? launch_compress<CPT, true, false>(a, n_full, n_b, s)
                 : launch_compress<CPT, false, false>(a, n_full, n_b, s);
}

// Blocks 0 .. n_full-1 take the bounds-free kernel; the rest the general one.
hipError_t dispatch_compress(int cpt, bool aligned, bool ef, const CompressArgs &a, int64_t n_full, int64_t n_b,
                             hipStream_t s) {
  switch (cpt) {
    case 1: return launch_compress_cpt<1>(aligned, ef, a, n_full, n_b, s);
    case 2: return launch_compress_cpt<2>(aligned, ef, a, n_full, n_b, s);
    case 4: return launch_compress_cpt<4>(aligned, ef, a, n_full, n_b, s);
    default: return launch_compress_cpt<8>(aligned, ef, a, 0, n_b, s);
  }
}

template <int CPT, int MODE, bool AL>
hipError_t launch_apply(const ApplyArgs &a, int64_t grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((apply_kernel<CPT, MODE, AL>), dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_apply_cpt(int mode, bool aligned, const ApplyArgs &a, int64_t grid, size_t lds, hipStream_t s) {
  if (mode == kModeSparse) return launch_apply<CPT, kModeSparse, false>(a, grid, lds, s);
  if (mode == kModeMoments) return launch_apply<CPT, kModeMoments, false>(a, grid, lds, s);
  return aligned ? launch_apply<CPT, kModeDense, true>(a, grid, lds, s)
                 : launch_apply<CPT, kModeDense, false>(a, grid, lds, s);
}

hipError_t dispatch_apply(int cpt, int mode, bool aligned, const ApplyArgs &a, int64_t grid, size_t lds,
                          hipStream_t s) {
  switch (cpt) {
    case 1: return launch_apply_cpt<1>(mode, aligned, a, grid, lds, s);
    case 2: return launch_apply_cpt<2>(mode, aligned, a, grid, lds, s);
    case 4: return launch_apply_cpt<4>(mode, aligned, a, grid, lds, s);
    default: return launch_apply_cpt<8>(mode, aligned, a, grid, lds, s);
  }
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
  // the block's window entries when they fit in a quarter of the budget, and
  // 10 bytes per slot for at most min(B_d, m*kb_max) touched positions.
  const int W = h->cpt * kChunkSpan / 32;
  const int64_t ents = (int64_t)m * kb_max;
  h->ent_cap = (4 * ents <= (int64_t)kApplyLdsLimit / 4) ? (int)ents : 0;
  const int64_t umax = std::min<int64_t>((int64_t)B_d, ents);
  const int64_t cap_limit = ((int64_t)kApplyLdsLimit - 8 * (int64_t)W - 4 * (int64_t)h->ent_cap) / 10;
  h->cap = (int)std::max<int64_t>(1, std::min<int64_t>(umax, cap_limit));
  h->apply_lds = 8 * (size_t)W + 4 * (size_t)h->ent_cap + 10 * (size_t)h->cap;

  h->codes_bytes = (size_t)((d + 1) / 2);
  h->codes_alloc = (h->codes_bytes + 15) & ~(size_t)15;
  const size_t stats_b = 8 * (size_t)h->n_b;
  const size_t win_b = 4 * (size_t)m * (size_t)k;
  bool ok = hipMalloc(&h->codes, h->codes_alloc) == hipSuccess &&
            hipMalloc(&h->stats, stats_b) == hipSuccess &&
            hipMalloc(&h->window, win_b ? win_b : 4) == hipSuccess &&
            hipMalloc(&h->off_tab, 8 * off.size()) == hipSuccess &&
            hipMalloc(&h->betapow, 4 * bp.size()) == hipSuccess &&
            hipMalloc(&h->touched, sizeof(unsigned long long)) == hipSuccess;
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
       hipMemset(h->touched, 0, sizeof(unsigned long long)) == hipSuccess &&
       hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    const hipError_t e = hipGetLastError();
    free_all(h);
    delete h;
    fail(MA_EHIP, "initialising the optimizer state failed: %s", hipGetErrorString(e));
    return nullptr;
  }
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
         (h->codes_alloc - h->codes_bytes) + sizeof(unsigned long long);
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
  if (flags & ~(MA_FLAG_NO_EF | MA_FLAG_FORCE_DENSE)) return fail(MA_EINVAL, "ma_set_flags: unknown flag bits");
  h->flags = flags;
  return MA_OK;
}

int ma_set_lr(ma_ctx *h, float lr) {
  clear_error();
  if (!h || !std::isfinite(lr)) return fail(MA_EINVAL, "ma_set_lr: null handle or non-finite lr");
  h->lr = lr;
  return MA_OK;
}

int ma_step(ma_ctx *h, float *params, const uint16_t *grads, hipStream_t stream) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_step: null handle");
  if (!params || !grads) return fail(MA_EINVAL, "ma_step: null params or grads");
  if (((uintptr_t)params & 3u) || ((uintptr_t)grads & 1u))
    return fail(MA_EINVAL, "ma_step: params must be 4-byte and grads 2-byte aligned");
  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(MA_EHIP, "ma_step: cannot select device %d", h->device);

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

  ApplyArgs aa = make_apply_args(h, t, c1, c2, decay);
  aa.theta = params;
  aa.touched = h->count_touched ? h->touched : nullptr;

  const bool b8 = (h->B % 8) == 0;
  const bool g_al = b8 && (((uintptr_t)grads & 15u) == 0);
  const bool p_al = b8 && (((uintptr_t)params & 15u) == 0);
  const int mode = (decay != 1.0f || (h->flags & MA_FLAG_FORCE_DENSE)) ? kModeDense : kModeSparse;

  ma_ctx::Ev ev{};
  if (h->timing) {
    if (!h->pool.empty()) {
      ev = h->pool.back();
      h->pool.pop_back();
    } else {
      for (auto &e : ev.e)
        if (hipEventCreate(&e) != hipSuccess) return fail(MA_EHIP, "ma_step: hipEventCreate failed");
    }
    hipEventRecord(ev.e[0], stream);
  }
  const int64_t n_full = (g_al && h->B == h->cpt * kChunkSpan) ? h->d / h->B : 0;
  hipError_t e = dispatch_compress(h->cpt, g_al, !(h->flags & MA_FLAG_NO_EF), ca, n_full, h->n_b, stream);
  if (e == hipSuccess && h->timing) hipEventRecord(ev.e[1], stream);
  if (e == hipSuccess) e = dispatch_apply(h->cpt, mode, p_al, aa, h->n_b, h->apply_lds, stream);
  if (h->timing) {
    hipEventRecord(ev.e[2], stream);
    h->events.push_back(ev);
  }
  if (e != hipSuccess) return fail(MA_EHIP, "ma_step: kernel launch failed: %s", hipGetErrorString(e));
  h->t = t;
  h->last_c1 = c1;
  h->last_c2 = c2;
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

int ma_debug_moments(ma_ctx *h, const int64_t *blocks, int64_t nblocks, float *mhat_out, float *vhat_out,
                     hipStream_t stream) {
  clear_error();
  if (!h || !blocks || !mhat_out || !vhat_out || nblocks < 0)
    return fail(MA_EINVAL, "ma_debug_moments: null argument");
  if (h->t < 1) return fail(MA_EINVAL, "ma_debug_moments: no step has run yet");
  if (nblocks == 0) return MA_OK;
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
  if (e == hipSuccess) e = dispatch_apply(h->cpt, kModeMoments, false, a, nblocks, h->apply_lds, stream);
  // the block list must outlive the kernel
  const hipError_t e2 = hipStreamSynchronize(stream);
  hipFree(dblocks);
  if (e != hipSuccess || e2 != hipSuccess)
    return fail(MA_EHIP, "ma_debug_moments: %s", hipGetErrorString(e != hipSuccess ? e : e2));
  return MA_OK;
}

int ma_set_timing(ma_ctx *h, int on) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_set_timing: null handle");
  DeviceGuard guard(h->device);
  for (auto &ev : h->events) h->pool.push_back(ev);
  h->events.clear();
  h->acc_ms[0] = h->acc_ms[1] = 0;
  h->acc_n[0] = h->acc_n[1] = 0;
  h->timing = on != 0;
  return MA_OK;
}

int ma_kernel_times(ma_ctx *h, double *ms_out, int64_t *launches_out, int nk) {
  clear_error();
  if (!h || !ms_out || !launches_out || nk < 0 || nk > 2) return fail(MA_EINVAL, "ma_kernel_times: bad argument");
  DeviceGuard guard(h->device);
  for (auto &ev : h->events) {
    if (hipEventSynchronize(ev.e[2]) != hipSuccess) return fail(MA_EHIP, "ma_kernel_times: event wait failed");
    float a = 0, b = 0;
    if (hipEventElapsedTime(&a, ev.e[0], ev.e[1]) != hipSuccess ||
        hipEventElapsedTime(&b, ev.e[1], ev.e[2]) != hipSuccess)
      return fail(MA_EHIP, "ma_kernel_times: elapsed time failed");
    h->acc_ms[0] += a;
    h->acc_ms[1] += b;
    h->acc_n[0] += 1;
    h->acc_n[1] += 1;
    h->pool.push_back(ev);
  }
  h->events.clear();
  for (int i = 0; i < nk; ++i) {
    ms_out[i] = h->acc_ms[i];
    launches_out[i] = h->acc_n[i];
  }
  return MA_OK;
}

int ma_set_count_touched(ma_ctx *h, int on) {
  clear_error();
  if (!h) return fail(MA_EINVAL, "ma_set_count_touched: null handle");
  DeviceGuard guard(h->device);
  if (on && (hipDeviceSynchronize() != hipSuccess ||
             hipMemset(h->touched, 0, sizeof(unsigned long long)) != hipSuccess ||
             hipDeviceSynchronize() != hipSuccess))
    return fail(MA_EHIP, "ma_set_count_touched: clearing the counter failed");
  h->count_touched = on != 0;
  return MA_OK;
}

int64_t ma_touched_count(ma_ctx *h) {
  clear_error();
  if (!h || !h->count_touched) return -1;
  DeviceGuard guard(h->device);
  unsigned long long v = 0;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&v, h->touched, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) {
    fail(MA_EHIP, "ma_touched_count: copy failed");
    return -1;
  }
  return (int64_t)v;
}

}  // extern "C"
