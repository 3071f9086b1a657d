// The fp32 AdamW baseline for gfx950: the comparison optimizer of the page
// "MicroAdam (Sparse-Gradient Adaptive Optimization with Quantized Error
// Feedback)", second paragraph (8 bytes of state per parameter).  A streaming
// kernel: per parameter 26 bytes move (parameter, m and v read and written,
// the bf16 gradient read), so it is bound by HBM bandwidth.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace microadam {

struct AdamwArgs {
  float *theta;
  const uint16_t *g;
  float *m, *v;
  int64_t n;
  float b1, b2, omb1, omb2, r1, r2, decay, lr, eps;
};

constexpr int kAdamwThreads = 256;

// one element, each operation rounded once (built without contraction)
__device__ __forceinline__ void adamw_elem(const AdamwArgs &A, float &th, float g, float &m, float &v) {
  m = A.b1 * m + A.omb1 * g;
  v = A.b2 * v + A.omb2 * (g * g);
  const float mh = m * A.r1;
  const float vh = v * A.r2;
  th = th * A.decay - A.lr * (mh / (sqrtf(vh) + A.eps));
}

// Grid-stride over runs of 8 elements.  ALIGNED: theta, m, v and g are 16-byte
// aligned, so each run is two 16-byte accesses per fp32 array and one for g.
template <bool ALIGNED>
__global__ __launch_bounds__(kAdamwThreads) void adamw_kernel(AdamwArgs A) {
  const int64_t stride = (int64_t)gridDim.x * kAdamwThreads * 8;
  for (int64_t i0 = ((int64_t)blockIdx.x * kAdamwThreads + threadIdx.x) * 8; i0 < A.n; i0 += stride) {
    if (ALIGNED && i0 + 8 <= A.n) {
      float4 t0 = *reinterpret_cast<const float4 *>(A.theta + i0), t1 = *reinterpret_cast<const float4 *>(A.theta + i0 + 4);
      float4 m0 = *reinterpret_cast<const float4 *>(A.m + i0), m1 = *reinterpret_cast<const float4 *>(A.m + i0 + 4);
      float4 v0 = *reinterpret_cast<const float4 *>(A.v + i0), v1 = *reinterpret_cast<const float4 *>(A.v + i0 + 4);
      const uint4 gw = *reinterpret_cast<const uint4 *>(A.g + i0);
      float th[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = (e & 1) ? __uint_as_float(gg[e >> 1] & 0xffff0000u) : __uint_as_float(gg[e >> 1] << 16);
        adamw_elem(A, th[e], g, mm[e], vv[e]);
      }
      *reinterpret_cast<float4 *>(A.theta + i0) = make_float4(th[0], th[1], th[2], th[3]);
      *reinterpret_cast<float4 *>(A.theta + i0 + 4) = make_float4(th[4], th[5], th[6], th[7]);
      *reinterpret_cast<float4 *>(A.m + i0) = make_float4(mm[0], mm[1], mm[2], mm[3]);
      *reinterpret_cast<float4 *>(A.m + i0 + 4) = make_float4(mm[4], mm[5], mm[6], mm[7]);
      *reinterpret_cast<float4 *>(A.v + i0) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      *reinterpret_cast<float4 *>(A.v + i0 + 4) = make_float4(vv[4], vv[5], vv[6], vv[7]);
    } else {
      for (int64_t i = i0; i < i0 + 8 && i < A.n; ++i) {
        float th = A.theta[i], m = A.m[i], v = A.v[i];
        adamw_elem(A, th, __uint_as_float((uint32_t)A.g[i] << 16), m, v);
        A.theta[i] = th;
        A.m[i] = m;
        A.v[i] = v;
      }
    }
  }
}

}  // namespace microadam
