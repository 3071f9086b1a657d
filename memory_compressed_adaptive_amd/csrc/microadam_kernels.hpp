// HIP kernels of the MicroAdam step for CDNA4 (gfx950).
//
// The step is the one on the page "MicroAdam (Sparse-Gradient Adaptive
// Optimization with Quantized Error Feedback)", first paragraph.  Its five
// stages run as two kernels, each launched with one 512-thread workgroup
// (8 wave64s) per B_d-block:
//
//   compress_kernel  = ef_dequant_accumulate + block_topk + zeroing +
//                      ef_requant + ring_write.  The block's accumulator a_t
//                      lives only in registers (8 consecutive elements per
//                      thread per 4096-element chunk); g and the 4-bit codes
//                      are read once and the codes written once.
//   apply_kernel     = adamstats_apply.  The m window segments of the block are
//                      turned into a bitmap of touched positions, each touched
//                      position gets a compact LDS slot, the rows are summed
//                      into the slots in row order (a barrier per row), and
//                      only the touched parameters are read and written.
//
// Bit-exactness with the CPU oracle rests on: fp32 with one rounding per
// operation (built with -ffp-contract=off), the explicit fmaf of the
// dequantizer, correctly rounded division and square root, the same host
// constants, and a fixed accumulation order (rows in physical order; indices
// within a row are unique).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace microadam {

constexpr int kThreads = 512;                   // one workgroup per block
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8;                       // consecutive elements per thread
constexpr int kChunkSpan = kThreads * kChunk;   // 4096 elements per chunk
constexpr int kCandMax = 512;                   // candidates one wave selects from (8 per lane)
constexpr int kCoarseLowBit = 16;               // candidate threshold keeps key bits 30..16
constexpr uint32_t kFlagNoEF = 1u;

// ------------------------------------------------------------------ scalars

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return u2f(h << 16); }

// fp32 -> bfloat16 bits, round to nearest even (the window stores bfloat16
// values).  Adding 0x7fff plus the kept half's lowest bit carries into the
// kept half exactly when the dropped half is above one half, or equal to it
// with an odd kept half.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = f2u(x);
  uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  if ((u & 0x7fffffffu) > 0x7f800000u) r = (u >> 16) | 0x40u;
  return r;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) reduced to the one output
// word the step uses: counter (j lo, j hi, t lo, t hi), key (seed lo, seed hi).
__device__ __forceinline__ uint32_t philox_block_key(uint64_t seed, int64_t t, int64_t j) {
  uint32_t x0 = (uint32_t)(uint64_t)j, x1 = (uint32_t)((uint64_t)j >> 32);
  uint32_t x2 = (uint32_t)(uint64_t)t, x3 = (uint32_t)((uint64_t)t >> 32);
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t p0_hi = __umulhi(0xD2511F53u, x0), p0_lo = 0xD2511F53u * x0;
    const uint32_t p1_hi = __umulhi(0xCD9E8D57u, x2), p1_lo = 0xCD9E8D57u * x2;
    const uint32_t y0 = p1_hi ^ x1 ^ k0;
    const uint32_t y2 = p0_hi ^ x3 ^ k1;
    x0 = y0; x1 = p1_lo; x2 = y2; x3 = p0_lo;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return x0;
}

// pcg_hash of Jarzynski and Olano (JCGT 2020): a PCG-32 LCG step followed by
// the RXS-M-XS output permutation.  One call gives the 16-bit uniforms of two
// neighbouring elements (low half: even element, high half: odd element).
__device__ __forceinline__ uint32_t pcg_hash(uint32_t x) {
  const uint32_t st = x * 747796405u + 2891336453u;
  const uint32_t w = ((st >> ((st >> 28u) + 4u)) ^ st) * 277803737u;
  return (w >> 22u) ^ w;
}

// ------------------------------------------------------------------ wave and block helpers

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over the workgroup (two barriers; s_red holds kWaves words).
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *s_red) {
  v = wave_sum(v);
  if (lane_id() == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += s_red[w];
  __syncthreads();
  return tot;
}

// Positions in block order for per-thread, per-chunk counts.  Block order of
// element (chunk c, thread tid, element e) is c*4096 + tid*8 + e, i.e.
// (chunk, wave, lane, element) lexicographic; so the exclusive prefix over
// (c, wave) totals plus the in-wave lane prefix gives each thread the first
// output position of its chunk-c elements.  s_cnt holds NC*kWaves + 1 words.
template <int NC>
__device__ __forceinline__ void ordered_offsets(const uint32_t (&cnt)[NC], uint32_t (&pos)[NC],
                                                uint32_t &total, uint32_t *s_cnt) {
  static_assert(NC * kWaves <= 64, "one wave scans the (chunk, wave) totals");
  const int lane = lane_id(), wv = (int)(threadIdx.x >> 6);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t inc = wave_incl_scan(cnt[c]);
    pos[c] = inc - cnt[c];
    if (lane == 63) s_cnt[c * kWaves + wv] = inc;
  }
  __syncthreads();
  if (wv == 0) {
    constexpr int n = NC * kWaves;
    const uint32_t v = lane < n ? s_cnt[lane] : 0u;
    const uint32_t inc = wave_incl_scan(v);
    if (lane < n) s_cnt[lane] = inc - v;
    if (lane == 63) s_cnt[n] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) pos[c] += s_cnt[c * kWaves + wv];
  total = s_cnt[NC * kWaves];
  __syncthreads();
}

// Blocks are handed out so that each XCD (workgroups are dealt round-robin to
// the 8 XCDs) walks one contiguous run of blocks; neighbouring blocks share
// cache lines of the window rows, which then stay in one L2.
__device__ __forceinline__ int64_t xcd_block(int64_t w, int64_t n) {
  const int64_t x = w & 7, i = w >> 3;
  const int64_t per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + i;
}

// ------------------------------------------------------------------ compress

struct CompressArgs {
  const uint16_t *g;        // bf16 gradients [d]
  uint8_t *ef;              // packed 4-bit codes, element i in nibble i
  float *stats;             // [2*n_b] {delta, Delta}
  uint32_t *G;              // window [m][k]
  const int64_t *off_tab;   // [n_b + 1] floor(k*s_j/d)
  int64_t d, k, n_b, t;
  int64_t row_base;         // (t mod m) * k
  uint64_t seed;
  int32_t B;
  uint32_t flags;
};

// One block of the compressor.  CPT = 4096-element chunks per thread.
// ALIGNED: B_d % 8 == 0 and the gradient pointer is 16-byte aligned, so a
// thread's 8 elements are one 16-byte gradient load and one 4-byte code word.
template <int CPT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs A) {
  __shared__ uint32_t s_red[kWaves];
  __shared__ float s_redf[2 * kWaves];
  __shared__ uint32_t s_cnt[CPT * kWaves + 1];
  __shared__ uint32_t s_candA[kCandMax];
  __shared__ uint16_t s_candI[kCandMax];
  __shared__ uint32_t s_sel[2];

  const int tid = (int)threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int64_t j = xcd_block((int64_t)blockIdx.x, A.n_b);
  const int64_t s = j * (int64_t)A.B;
  const int L = (int)((A.d - s) < (int64_t)A.B ? (A.d - s) : (int64_t)A.B);
  const int64_t off = A.off_tab[j];
  const int kb = (int)(A.off_tab[j + 1] - off);
  const bool use_ef = !(A.flags & kFlagNoEF);

  // ---------------- ef_dequant_accumulate: a = f32(g) + fmaf(code, s, delta)
  float lo = 0.f, step = 0.f;
  if (use_ef) {
    lo = A.stats[2 * j];
    const float hi = A.stats[2 * j + 1];
    step = (hi - lo) / 15.0f;
  }
  float a[CPT][kChunk];
  uint32_t oldc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i0 = c * kChunkSpan + tid * kChunk;
    if (ALIGNED && i0 + kChunk <= L) {
      const uint4 gv = *reinterpret_cast<const uint4 *>(A.g + s + i0);
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
      const uint32_t cw = use_ef ? *reinterpret_cast<const uint32_t *>(A.ef + ((s + i0) >> 1)) : 0u;
      oldc[c] = cw;
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const uint32_t gb = (e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffffu);
        const float gf = bf16_bits_to_f32(gb);
        a[c][e] = use_ef ? gf + fmaf((float)((cw >> (4 * e)) & 15u), step, lo) : gf;
      }
    } else {
      uint32_t cw = 0;
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = i0 + e;
        float v = 0.f;
        if (i < L) {
          const int64_t gi = s + i;
          const float gf = bf16_bits_to_f32(A.g[gi]);
          if (use_ef) {
            const uint32_t code = (A.ef[gi >> 1] >> (4 * (int)(gi & 1))) & 15u;
            cw |= code << (4 * e);
            v = gf + fmaf((float)code, step, lo);
          } else {
            v = gf;
          }
        }
        a[c][e] = v;
      }
      oldc[c] = cw;
    }
  }

  // ---------------- block_topk: the k_b largest |a| (as 31-bit patterns),
  // ties to the lower index.  Result: threshold key T and the index of the
  // last selected element with key T; selected <=> key > T or (key == T and
  // index <= idx_last).
  uint32_t T = 0xffffffffu;
  int idx_last = -1;
  if (kb > 0) {
    bool done = false;
    const int q = (kb + kWaves - 1) / kWaves;
    if (q <= 64 && kb < L) {
      // (1) a candidate threshold tau with at least k_b keys >= tau: every wave
      // finds a value its q-th largest lane maximum reaches; tau is their
      // minimum, so at least kWaves*q >= k_b distinct elements reach tau.
      uint32_t lanemax = 0;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          const uint32_t key = f2u(a[c][e]) & 0x7fffffffu;
          if (i < L && key > lanemax) lanemax = key;
        }
      uint32_t P = 0;
      for (int b = 30; b >= kCoarseLowBit; --b) {
        const uint32_t cand = P | (1u << b);
        if ((int)__popcll(__ballot(lanemax >= cand)) >= q) P = cand;
      }
      if (lane == 0) s_red[wv] = P;
      __syncthreads();
      uint32_t tau = s_red[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) tau = min(tau, s_red[w]);
      // (2) gather the candidates (key >= tau) into LDS in index order
      uint32_t cnt[CPT], pos[CPT], C;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          n += (i < L && (f2u(a[c][e]) & 0x7fffffffu) >= tau) ? 1u : 0u;
        }
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, C, s_cnt);
      if (C <= (uint32_t)kCandMax) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          if (cnt[c] == 0) continue;
          uint32_t p = pos[c];
#pragma unroll
          for (int e = 0; e < kChunk; ++e) {
            const int i = c * kChunkSpan + tid * kChunk + e;
            if (i < L && (f2u(a[c][e]) & 0x7fffffffu) >= tau) {
              s_candA[p] = f2u(a[c][e]);
              s_candI[p] = (uint16_t)i;
              ++p;
            }
          }
        }
        __syncthreads();
        // (3) one wave: exact k_b-th largest key by MSB-first bit search over
        // the candidates, the tie cut in index order, and the ordered write
        // of (I, bf16(V)) into the window row (ring_write).
        if (wv == 0) {
          const int R = ((int)C + 63) >> 6;
          uint32_t ck[kCandMax / 64];
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r) {
            const int cidx = r * 64 + lane;
            ck[r] = (r < R && cidx < (int)C) ? (s_candA[cidx] & 0x7fffffffu) : 0u;
          }
          // padding lanes hold key 0 but are excluded by the index test
          uint32_t Pk = 0;
          for (int b = 30; b >= 0; --b) {
            const uint32_t cand = Pk | (1u << b);
            int n = 0;
#pragma unroll
            for (int r = 0; r < kCandMax / 64; ++r)
              if (r < R) n += (int)__popcll(__ballot(r * 64 + lane < (int)C && ck[r] >= cand));
            if (n >= kb) Pk = cand;
          }
          int ngt = 0;
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r)
            if (r < R) ngt += (int)__popcll(__ballot(r * 64 + lane < (int)C && ck[r] > Pk));
          const int need = kb - ngt;   // >= 1 ties at key Pk are taken
          int run = 0, last = -1;
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r) {
            if (r < R && last < 0) {
              const bool tie = r * 64 + lane < (int)C && ck[r] == Pk;
              const uint64_t m = __ballot(tie);
              const int pc = (int)__popcll(m);
              if (run + pc >= need) {
                const bool hit = tie && (int)lanes_below(m) == need - run - 1;
                const uint64_t hm = __ballot(hit);
                const int src = __ffsll((long long)hm) - 1;
                last = __shfl((int)s_candI[r * 64 + lane], src, 64);
              }
              run += pc;
            }
          }
          // ring_write: selected candidates, already in index order
          uint32_t *dst = A.G + A.row_base + off;
          int wrote = 0;
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r) {
            if (r < R) {
              const int cidx = r * 64 + lane;
              const bool in = cidx < (int)C;
              const int idx = in ? (int)s_candI[cidx] : 0;
              const bool sel = in && (ck[r] > Pk || (ck[r] == Pk && idx <= last));
              const uint64_t m = __ballot(sel);
              if (sel) {
                const float v = u2f(s_candA[cidx]);
                dst[wrote + (int)lanes_below(m)] = (uint32_t)idx | (f32_to_bf16_rne(v) << 16);
              }
              wrote += (int)__popcll(m);
            }
          }
          if (lane == 0) { s_sel[0] = Pk; s_sel[1] = (uint32_t)last; }
        }
        __syncthreads();
        T = s_sel[0];
        idx_last = (int)s_sel[1];
        done = true;
      }
    }
    if (!done) {
      // General path (k_b > 8*64, k_b == L, or too many candidates): exact
      // MSB-first bit search over the whole block with workgroup counts.
      uint32_t P = 0;
      for (int b = 30; b >= 0; --b) {
        const uint32_t cand = P | (1u << b);
        uint32_t n = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
          for (int e = 0; e < kChunk; ++e) {
            const int i = c * kChunkSpan + tid * kChunk + e;
            n += (i < L && (f2u(a[c][e]) & 0x7fffffffu) >= cand) ? 1u : 0u;
          }
        if ((int)block_sum(n, s_red) >= kb) P = cand;
      }
      uint32_t ngt = 0;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          ngt += (i < L && (f2u(a[c][e]) & 0x7fffffffu) > P) ? 1u : 0u;
        }
      const int need = kb - (int)block_sum(ngt, s_red);
      // the need-th tie (key == P) in index order
      uint32_t cnt[CPT], pos[CPT], tot;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          n += (i < L && (f2u(a[c][e]) & 0x7fffffffu) == P) ? 1u : 0u;
        }
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, tot, s_cnt);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t p = pos[c];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          if (i < L && (f2u(a[c][e]) & 0x7fffffffu) == P) {
            if ((int)p == need - 1) s_sel[1] = (uint32_t)i;
            ++p;
          }
        }
      }
      __syncthreads();
      T = P;
      idx_last = (int)s_sel[1];
      // ring_write of every selected element, in index order
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          const uint32_t key = f2u(a[c][e]) & 0x7fffffffu;
          n += (i < L && (key > T || (key == T && i <= idx_last))) ? 1u : 0u;
        }
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, tot, s_cnt);
      uint32_t *dst = A.G + A.row_base + off;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t p = pos[c];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          const uint32_t key = f2u(a[c][e]) & 0x7fffffffu;
          if (i < L && (key > T || (key == T && i <= idx_last))) {
            dst[p] = (uint32_t)i | (f32_to_bf16_rne(a[c][e]) << 16);
            ++p;
          }
        }
      }
    }
  }

  if (!use_ef) return;   // no error feedback: codes and statistics are left as they are

  // ---------------- zero the selected entries; block min / max of the residual
  float mn = __int_as_float(0x7f800000), mx = -__int_as_float(0x7f800000);
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      const int i = c * kChunkSpan + tid * kChunk + e;
      const uint32_t key = f2u(a[c][e]) & 0x7fffffffu;
      if (key > T || (key == T && i <= idx_last)) a[c][e] = 0.0f;
      if (i < L) {
        mn = fminf(mn, a[c][e]);
        mx = fmaxf(mx, a[c][e]);
      }
    }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { s_redf[wv] = mn; s_redf[kWaves + wv] = mx; }
  __syncthreads();
  mn = s_redf[0];
  mx = s_redf[kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    mn = fminf(mn, s_redf[w]);
    mx = fmaxf(mx, s_redf[kWaves + w]);
  }
  mn = mn + 0.0f;   // a zero extreme is stored as +0
  mx = mx + 0.0f;

  // ---------------- ef_requant: unbiased stochastic 4-bit rounding
  const bool flat = (mx == mn);
  const float inv = flat ? 0.f : 15.0f / (mx - mn);
  const uint32_t bkey = philox_block_key(A.seed, A.t, j);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i0 = c * kChunkSpan + tid * kChunk;
    uint32_t packed = 0;
#pragma unroll
    for (int pr = 0; pr < kChunk / 2; ++pr) {
      const uint32_t h = pcg_hash(bkey + (uint32_t)((i0 >> 1) + pr));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int e = 2 * pr + half;
        const uint32_t u = half ? (h >> 16) : (h & 0xffffu);
        uint32_t code = 0;
        if (!flat) {
          const float y = (a[c][e] - mn) * inv;
          const float f = floorf(y);
          const float frac = y - f;
          code = (uint32_t)f + (((float)u < frac * 65536.0f) ? 1u : 0u);
          code = min(code, 15u);
        }
        if (i0 + e >= L) code = 0;
        packed |= code << (4 * e);
      }
    }
    if (ALIGNED) {
      if (i0 < L) *reinterpret_cast<uint32_t *>(A.ef + ((s + i0) >> 1)) = packed;
    } else {
      // neighbouring blocks (and threads) may share a code byte: change only
      // this element's nibble, by xor-ing old ^ new into its 32-bit word
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = i0 + e;
        if (i < L) {
          const int64_t gi = s + i;
          const uint32_t diff = ((packed >> (4 * e)) ^ (oldc[c] >> (4 * e))) & 15u;
          if (diff) {
            const int64_t byte = gi >> 1;
            uint32_t *word = reinterpret_cast<uint32_t *>(A.ef + (byte & ~(int64_t)3));
            atomicXor(word, diff << (8 * (int)(byte & 3) + 4 * (int)(gi & 1)));
          }
        }
      }
    }
  }
  if (tid == 0) {
    A.stats[2 * j] = mn;
    A.stats[2 * j + 1] = mx;
  }
}

// ------------------------------------------------------------------ adamstats_apply

struct ApplyArgs {
  float *theta;             // parameters [d] (MODE 0, 1)
  const uint32_t *G;        // window [m][k]
  const int64_t *off_tab;   // [n_b + 1]
  const float *betapow;     // [2m]: beta1^r, then beta2^r, r = 0..m-1
  float *mhat, *vhat;       // MODE 2 outputs [nblocks][B]
  const int64_t *blocks;    // MODE 2 block list
  unsigned long long *touched;   // optional: sum of touched positions
  int64_t d, k, n_b;
  int32_t B, m, tm, cap;    // tm = t mod m; cap = LDS slots per pass
  float c1, c2, lr, eps, decay;
};

enum { kModeSparse = 0, kModeDense = 1, kModeMoments = 2 };

// MODE 0: only touched parameters are read and written (decay must be 1).
// MODE 1: the block's parameters are streamed through registers; decoupled
//         decay on all, the Adam step on the touched ones.
// MODE 2: write m_hat and v_hat of listed blocks; parameters untouched.
template <int CPT, int MODE, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void apply_kernel(ApplyArgs A) {
  extern __shared__ uint32_t smem[];
  constexpr int W = CPT * kChunkSpan / 32;          // bitmap words
  constexpr int WPT = (W + kThreads - 1) / kThreads;
  uint32_t *s_bits = smem;
  uint32_t *s_wbase = smem + W;
  float *s_z1 = reinterpret_cast<float *>(smem + 2 * W);
  float *s_z2 = s_z1 + A.cap;
  uint16_t *s_pos = reinterpret_cast<uint16_t *>(s_z2 + A.cap);
  __shared__ uint32_t s_cnt[kWaves + 1];

  const int tid = (int)threadIdx.x;
  const int64_t j = (MODE == kModeMoments) ? A.blocks[blockIdx.x] : xcd_block((int64_t)blockIdx.x, A.n_b);
  const int64_t s = j * (int64_t)A.B;
  const int L = (int)((A.d - s) < (int64_t)A.B ? (A.d - s) : (int64_t)A.B);
  const int64_t off = A.off_tab[j];
  const int kb = (int)(A.off_tab[j + 1] - off);

  float th[CPT][kChunk];
  if (MODE == kModeDense) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i0 = c * kChunkSpan + tid * kChunk;
      if (ALIGNED && i0 + kChunk <= L) {
        const float4 v0 = *reinterpret_cast<const float4 *>(A.theta + s + i0);
        const float4 v1 = *reinterpret_cast<const float4 *>(A.theta + s + i0 + 4);
        th[c][0] = v0.x; th[c][1] = v0.y; th[c][2] = v0.z; th[c][3] = v0.w;
        th[c][4] = v1.x; th[c][5] = v1.y; th[c][6] = v1.z; th[c][7] = v1.w;
      } else {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) th[c][e] = (i0 + e < L) ? A.theta[s + i0 + e] : 0.f;
      }
    }
  }

  // ---------------- union of the window's positions in this block
  for (int w = tid; w < W; w += kThreads) s_bits[w] = 0;
  __syncthreads();
  for (int i = 0; i < A.m; ++i) {
    const uint32_t *row = A.G + (int64_t)i * A.k + off;
    for (int q = tid; q < kb; q += kThreads) {
      const uint32_t e = row[q];
      // a zero value adds nothing (unwritten rows are all zero); an index
      // outside the block (only possible in an imported state) is ignored
      if ((e & 0x7fff0000u) && (int)(e & 0xffffu) < L) atomicOr(&s_bits[(e & 0xffffu) >> 5], 1u << (e & 31u));
    }
  }
  __syncthreads();

  // ---------------- compact slots: slot(p) = #touched positions below p
  uint32_t wc[WPT], mine = 0;
#pragma unroll
  for (int r = 0; r < WPT; ++r) {
    const int w = tid * WPT + r;
    wc[r] = (w < W) ? (uint32_t)__popc(s_bits[w]) : 0u;
    mine += wc[r];
  }
  uint32_t cnt1[1] = {mine}, pos1[1], U;
  ordered_offsets<1>(cnt1, pos1, U, s_cnt);
  {
    uint32_t b = pos1[0];
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid * WPT + r;
      if (w < W) s_wbase[w] = b;
      b += wc[r];
    }
  }
  if (MODE != kModeMoments && A.touched && tid == 0) atomicAdd(A.touched, (unsigned long long)U);
  __syncthreads();

  if (MODE == kModeDense) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) th[c][e] = th[c][e] * A.decay;
  }
  if (MODE == kModeMoments) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = c * kChunkSpan + tid * kChunk + e;
        if (i < L) {
          A.mhat[(int64_t)blockIdx.x * A.B + i] = 0.f;
          A.vhat[(int64_t)blockIdx.x * A.B + i] = 0.f;
        }
      }
  }

  for (uint32_t s0 = 0; s0 < U; s0 += (uint32_t)A.cap) {
    const uint32_t n = min((uint32_t)A.cap, U - s0);
    for (uint32_t x = (uint32_t)tid; x < n; x += kThreads) { s_z1[x] = 0.f; s_z2[x] = 0.f; }
    if (MODE == kModeSparse) {
#pragma unroll
      for (int r = 0; r < WPT; ++r) {
        const int w = tid * WPT + r;
        if (w < W) {
          uint32_t bits = s_bits[w];
          uint32_t sl = s_wbase[w];
          while (bits) {
            const int bit = __ffs(bits) - 1;
            if (sl - s0 < n) s_pos[sl - s0] = (uint16_t)(w * 32 + bit);
            ++sl;
            bits &= bits - 1u;
          }
        }
      }
    }
    __syncthreads();
    // AdamStats: z[I] += beta^r V, rows in physical order, one row at a time
    for (int i = 0; i < A.m; ++i) {
      int r = A.tm - i;
      if (r < 0) r += A.m;
      const float f1 = A.betapow[r], f2 = A.betapow[A.m + r];
      const uint32_t *row = A.G + (int64_t)i * A.k + off;
      for (int q = tid; q < kb; q += kThreads) {
        const uint32_t e = row[q];
        const uint32_t I = e & 0xffffu;
        if (!(e & 0x7fff0000u) || (int)I >= L) continue;
        const float V = bf16_bits_to_f32(e >> 16);
        const uint32_t sl = s_wbase[I >> 5] + (uint32_t)__popc(s_bits[I >> 5] & ((1u << (I & 31u)) - 1u)) - s0;
        if (sl < n) {
          s_z1[sl] = s_z1[sl] + f1 * V;
          s_z2[sl] = s_z2[sl] + f2 * (V * V);
        }
      }
      __syncthreads();
    }
    // m_hat = c1 z1, v_hat = c2 z2; theta -= lr * m_hat / (sqrt(v_hat) + eps)
    if (MODE == kModeSparse) {
      for (uint32_t x = (uint32_t)tid; x < n; x += kThreads) {
        const int p = s_pos[x];
        const float mh = A.c1 * s_z1[x];
        const float vh = A.c2 * s_z2[x];
        float *tp = A.theta + s + p;
        const float upd = A.lr * (mh / (sqrtf(vh) + A.eps));
        *tp = *tp - upd;
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          if (i < L) {
            const uint32_t word = s_bits[i >> 5];
            if ((word >> (i & 31)) & 1u) {
              const uint32_t sl = s_wbase[i >> 5] + (uint32_t)__popc(word & ((1u << (i & 31)) - 1u)) - s0;
              if (sl < n) {
                const float mh = A.c1 * s_z1[sl];
                const float vh = A.c2 * s_z2[sl];
                if (MODE == kModeDense) {
                  th[c][e] = th[c][e] - A.lr * (mh / (sqrtf(vh) + A.eps));
                } else {
                  A.mhat[(int64_t)blockIdx.x * A.B + i] = mh;
                  A.vhat[(int64_t)blockIdx.x * A.B + i] = vh;
                }
              }
            }
          }
        }
    }
    __syncthreads();
  }

  if (MODE == kModeDense) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i0 = c * kChunkSpan + tid * kChunk;
      if (ALIGNED && i0 + kChunk <= L) {
        *reinterpret_cast<float4 *>(A.theta + s + i0) = make_float4(th[c][0], th[c][1], th[c][2], th[c][3]);
        *reinterpret_cast<float4 *>(A.theta + s + i0 + 4) = make_float4(th[c][4], th[c][5], th[c][6], th[c][7]);
      } else {
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
          if (i0 + e < L) A.theta[s + i0 + e] = th[c][e];
      }
    }
  }
}

}  // namespace microadam
