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

namespace microadam {

// ------------------------------------------------------------------ 8-bit AdamW
// The page's other comparison point (2 bytes of state per parameter).  The
// page fixes no 8-bit scheme; this one: blocks of 256 elements with two fp32
// scales; m as int8 codes of m * (127 / max|m|), v as uint8 codes of
// sqrt(v) * (255 / max sqrt(v)), both rounded to nearest even.  A step
// dequantizes, applies the AdamW recurrence and update above, and requantizes
// the new moments with the block's new scales.  One wave per block, 4
// consecutive elements per lane; the block maxima are wave reductions.

constexpr int kQ8Block = 256;

struct Adamw8Args {
  float *theta;
  const uint16_t *g;
  int8_t *cm;
  uint8_t *cv;
  float *sm, *sr;
  int64_t n;
  float b1, b2, omb1, omb2, r1, r2, decay, lr, eps;
};

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <bool ALIGNED>
__global__ __launch_bounds__(256) void adamw8_kernel(Adamw8Args A) {
  const int lane = (int)(threadIdx.x & 63u);
  const int64_t nq = (A.n + kQ8Block - 1) / kQ8Block;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  for (int64_t q = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); q < nq; q += wstride) {
    const int64_t i0 = q * kQ8Block + 4 * lane;
    const float qm = A.sm[q] / 127.0f, qr = A.sr[q] / 255.0f;
    float th[4], m[4], v[4];
    bool in[4];
    const bool full = ALIGNED && i0 + 4 <= A.n;
    uint32_t cmw = 0, cvw = 0;
    uint2 gw = make_uint2(0u, 0u);
    float4 tv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (full) {
      tv = *reinterpret_cast<const float4 *>(A.theta + i0);
      gw = *reinterpret_cast<const uint2 *>(A.g + i0);
      cmw = *reinterpret_cast<const uint32_t *>(A.cm + i0);
      cvw = *reinterpret_cast<const uint32_t *>(A.cv + i0);
    }
    const float tt[4] = {tv.x, tv.y, tv.z, tv.w};
    float amax = 0.f, rmax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      in[e] = i < A.n;
      float gi = 0.f, mo = 0.f, ro = 0.f;
      th[e] = 0.f;
      if (full) {
        th[e] = tt[e];
        const uint32_t gh = (e < 2) ? gw.x : gw.y;
        gi = (e & 1) ? __uint_as_float(gh & 0xffff0000u) : __uint_as_float(gh << 16);
        mo = (float)(int8_t)(cmw >> (8 * e)) * qm;
        ro = (float)((cvw >> (8 * e)) & 0xffu) * qr;
      } else if (in[e]) {
        th[e] = A.theta[i];
        gi = __uint_as_float((uint32_t)A.g[i] << 16);
        mo = (float)A.cm[i] * qm;
        ro = (float)A.cv[i] * qr;
      }
      const float vo = ro * ro;
      m[e] = A.b1 * mo + A.omb1 * gi;
      v[e] = A.b2 * vo + A.omb2 * (gi * gi);
      const float mh = m[e] * A.r1;
      const float vh = v[e] * A.r2;
      th[e] = th[e] * A.decay - A.lr * (mh / (sqrtf(vh) + A.eps));
      if (in[e]) {
        amax = fmaxf(amax, fabsf(m[e]));
        rmax = fmaxf(rmax, sqrtf(v[e]));
      }
    }
    amax = wave_max_f(amax);
    rmax = wave_max_f(rmax);
    const float im = (amax > 0.f) ? 127.0f / amax : 0.f;
    const float ir = (rmax > 0.f) ? 255.0f / rmax : 0.f;
    uint32_t cmo = 0, cvo = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = fminf(fmaxf(rintf(m[e] * im), -127.f), 127.f);
      const float dq = fminf(rintf(sqrtf(v[e]) * ir), 255.f);
      cmo |= ((uint32_t)(int32_t)c & 0xffu) << (8 * e);
      cvo |= ((uint32_t)dq) << (8 * e);
    }
    if (full) {
      *reinterpret_cast<float4 *>(A.theta + i0) = make_float4(th[0], th[1], th[2], th[3]);
      *reinterpret_cast<uint32_t *>(A.cm + i0) = cmo;
      *reinterpret_cast<uint32_t *>(A.cv + i0) = cvo;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (in[e]) {
          A.theta[i0 + e] = th[e];
          A.cm[i0 + e] = (int8_t)(cmo >> (8 * e));
          A.cv[i0 + e] = (uint8_t)(cvo >> (8 * e));
        }
    }
    if (lane == 0) {
      A.sm[q] = amax;
      A.sr[q] = rmax;
    }
  }
}

}  // namespace microadam
