// Seeded synthetic inputs for the MicroAdam benchmark and tests: fp32
// parameters ~ N(mean, std) and bf16 gradients with per-tensor scales.  Every
// value is a pure function of (seed, step, element index), drawn from
// Philox4x32-10 (Salmon et al., SC'11) and Box-Muller, so a run can be
// regenerated and sampled on the host side for comparison.  Nothing here is
// part of the optimizer step.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint32_t h0 = __umulhi(0xD2511F53u, c0), l0 = 0xD2511F53u * c0;
    const uint32_t h1 = __umulhi(0xCD9E8D57u, c2), l1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
    c0 = n0; c1 = l1; c2 = n2; c3 = l0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// uniform in (0, 1) from the top 24 bits
__device__ __forceinline__ float u01(uint32_t u) { return ((float)(u >> 8) + 0.5f) * (1.0f / 16777216.0f); }

__device__ __forceinline__ void box_muller(uint32_t a, uint32_t b, float &z0, float &z1) {
  const float r = sqrtf(-2.0f * logf(u01(a)));
  float sn, cs;
  sincosf(6.28318530717958647692f * u01(b), &sn, &cs);
  z0 = r * cs;
  z1 = r * sn;
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ void normal_f32_kernel(float *out, int64_t n, uint64_t seed, float mean, float sd) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const U4 r = philox((uint32_t)i, (uint32_t)((uint64_t)i >> 32), 0u, 0x70u, (uint32_t)seed, (uint32_t)(seed >> 32));
    float z0, z1;
    box_muller(r.x, r.y, z0, z1);
    out[i] = mean + sd * z0;
  }
}

// kind 0: N(0, scale) with outliers (probability p, multiplied by mult)
// kind 1: scale * Student-t with 3 degrees of freedom
__global__ void grads_bf16_kernel(uint16_t *out, int64_t n, uint64_t seed, int64_t step, int kind,
                                  const int64_t *seg_end, const float *seg_scale, int nseg, float p, float mult) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    int lo = 0, hi = nseg - 1;   // first segment whose end is > i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (seg_end[mid] > i) hi = mid; else lo = mid + 1;
    }
    const float scale = seg_scale[lo];
    const U4 r = philox((uint32_t)i, (uint32_t)((uint64_t)i >> 32), (uint32_t)step, 0x67u,
                        (uint32_t)seed, (uint32_t)(seed >> 32));
    float z0, z1, v;
    box_muller(r.x, r.y, z0, z1);
    if (kind == 0) {
      v = z0 * scale;
      if (u01(r.z) < p) v *= mult;
    } else {
      float z2, z3;
      box_muller(r.z, r.w, z2, z3);
      v = scale * z0 / sqrtf((z1 * z1 + z2 * z2 + z3 * z3) * (1.0f / 3.0f));
    }
    out[i] = to_bf16(v);
  }
}

__global__ void copy_f32_kernel(float *__restrict__ dst, const float *__restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<float4 *>(dst)[i] = reinterpret_cast<const float4 *>(src)[i];
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

extern "C" {

int masyn_normal_f32(float *out, int64_t n, uint64_t seed, float mean, float sd, hipStream_t s) {
  if (!out || n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(normal_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, seed, mean, sd);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int masyn_grads_bf16(uint16_t *out, int64_t n, uint64_t seed, int64_t step, int kind, const int64_t *seg_end,
                     const float *seg_scale, int nseg, float p_outlier, float outlier_mult, hipStream_t s) {
  if (!out || n < 0 || !seg_end || !seg_scale || nseg < 1 || (kind != 0 && kind != 1)) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(grads_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, out, n, seed, step, kind, seg_end,
                     seg_scale, nseg, p_outlier, outlier_mult);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// A plain streaming copy (16 B per lane): the reference kernel for HBM
// bandwidth and for scaling the FETCH_SIZE / WRITE_SIZE counters.
int masyn_copy_f32(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (!dst || !src || n < 0) return -1;
  if (n == 0) return 0;
  const int64_t n4 = n / 4;
  const int64_t g = (n4 + 255) / 256;
  const unsigned grid = (unsigned)(g < 1 ? 1 : (g > (1 << 20) ? (1 << 20) : g));
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid), dim3(256), 0, s, dst, src, n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
