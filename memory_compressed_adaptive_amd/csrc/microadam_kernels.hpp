// HIP kernels of the MicroAdam step for CDNA4 (gfx950).
//
// The step is the one on the page "MicroAdam (Sparse-Gradient Adaptive
// Optimization with Quantized Error Feedback)", first paragraph.  Its stages
// are two phases of work per B_d-block, each run by one 512-thread workgroup
// (8 wave64s):
//
//   compress  = ef_dequant_accumulate + block_topk + zeroing + ef_requant +
//               ring_write.  The block's accumulator a_t lives only in
//               registers (8 consecutive elements per thread per 4096-element
//               chunk); g and the 4-bit codes are read once and the codes
//               written once.
//   apply     = adamstats_apply.  The m window segments of the block are
//               turned into a bitmap of touched positions and each touched
//               position gets a compact LDS slot.  Then either the rows are
//               summed into the slots one row at a time (apply_block, short
//               windows), or the entries are sorted by slot (a counting sort
//               in LDS) and each slot's column is summed by one thread
//               (apply_block_csu, long windows).  Only the touched parameters
//               are read and written (sparse mode), or all of them with
//               decoupled decay (dense mode).
//
// step_full_kernel (row sums) and step_csu_kernel (column sums) run both
// phases of a block in one workgroup: the default for full, aligned blocks.
// The host picks one per step by window length, update mode and parameter
// type (step_full_kernel only where its LDS holds the window).
// compress_full_kernel / compress_kernel and apply_kernel / apply_csu_kernel
// run them as two kernels (a partial last block, windows too long for either
// fused kernel, unaligned inputs).
//
// Bit-exactness with the CPU oracle rests on: fp32 with one rounding per
// operation (built with -ffp-contract=off), the explicit fmaf of the
// dequantizer, correctly rounded division and square root, the same host
// constants, and a fixed accumulation order (each position's entries added
// in physical row order, by either algorithm).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace microadam {

constexpr int kThreads = 512;                   // one workgroup per block
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 8;                       // consecutive elements per thread
constexpr int kChunkSpan = kThreads * kChunk;   // 4096 elements per chunk
constexpr int kCandMax = 512;                   // candidates one wave selects from (8 per lane)
constexpr int kCacheStream = 2;                // cache-policy bits of a non-temporal (streaming) access
constexpr int kCoarseLowBit = 16;               // candidate threshold keeps key bits 30..16
#ifndef MA_FULL_WAVES
#define MA_FULL_WAVES 6   // 80 VGPRs: three 512-thread blocks per CU
#endif

// ------------------------------------------------------------------ scalars

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return u2f(h << 16); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data read exactly once (streamed past the caches)
__device__ __forceinline__ u32x4 load_stream16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

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
// pcg_out is its output permutation of the LCG state st: hashes of counters
// x and x + n have states n * 747796405 apart (mod 2^32), so a run of
// counters steps the state by an addition instead of a multiplication.
constexpr uint32_t kPcgMul = 747796405u;
__device__ __forceinline__ uint32_t pcg_out(uint32_t st) {
  const uint32_t w = ((st >> ((st >> 28u) + 4u)) ^ st) * 277803737u;
  return (w >> 22u) ^ w;
}
__device__ __forceinline__ uint32_t pcg_state(uint32_t x) { return x * kPcgMul + 2891336453u; }
__device__ __forceinline__ uint32_t pcg_hash(uint32_t x) { return pcg_out(pcg_state(x)); }

// Top-k keys.  The key of a value is the 31-bit pattern of |x|: for finite
// values that is the order of |x|, +-Inf is above every finite value and NaN
// above that.  Every NaN takes the key of the canonical quiet NaN, so neither
// the selection nor the window depends on the payload or sign a NaN carries.
constexpr uint32_t kKeyInf = 0x7f800000u;
constexpr uint32_t kKeyNaN = 0x7fc00000u;
__device__ __forceinline__ uint32_t topk_key(float x) {
  const uint32_t k = f2u(x) & 0x7fffffffu;
  return k > kKeyInf ? kKeyNaN : k;
}
// The window value of a selected element (its fp32 bits and key): bfloat16,
// round to nearest even; a NaN is stored as the canonical 0x7fc0.
__device__ __forceinline__ uint32_t window_bf16(uint32_t bits, uint32_t key) {
  return key == kKeyNaN ? 0x7fc0u : f32_to_bf16_rne(u2f(bits));
}

// ------------------------------------------------------------------ wave and block helpers

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Cross-lane steps use DPP: row_shr:n shifts within 16-lane rows (zero fill
// at the row start), row_ror:n rotates within rows, row_bcast:15 / :31 carry
// lane 15 / 31 into the following rows.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(0u, v);   // row_shr:1
  v += dpp_u32<0x112, 0xf>(0u, v);   // row_shr:2
  v += dpp_u32<0x114, 0xf>(0u, v);   // row_shr:4
  v += dpp_u32<0x118, 0xf>(0u, v);   // row_shr:8
  v += dpp_u32<0x142, 0xa>(0u, v);   // row_bcast:15 into rows 1, 3
  v += dpp_u32<0x143, 0xc>(0u, v);   // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}

// min / max over the 64 lanes, returned uniformly (lane 63 ends with the result)
template <bool MAX>
__device__ __forceinline__ float wave_minmax(float v) {
#define MA_STEP(CTRL, RM)                                                            \
  {                                                                                 \
    const float o = u2f(dpp_u32<CTRL, RM>(f2u(v), f2u(v)));                         \
    v = MAX ? fmaxf(v, o) : fminf(v, o);                                            \
  }
  MA_STEP(0x121, 0xf)   // row_ror:1
  MA_STEP(0x122, 0xf)   // row_ror:2
  MA_STEP(0x124, 0xf)   // row_ror:4
  MA_STEP(0x128, 0xf)   // row_ror:8
  MA_STEP(0x142, 0xa)   // row_bcast:15
  MA_STEP(0x143, 0xc)   // row_bcast:31
#undef MA_STEP
  return u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 63));
}
__device__ __forceinline__ float wave_min(float v) { return wave_minmax<false>(v); }
__device__ __forceinline__ float wave_max(float v) { return wave_minmax<true>(v); }

// the same over unsigned integers (Top-k keys, NaN keys included)
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
#define MA_STEP(CTRL, RM)                                                            \
  {                                                                                 \
    const uint32_t o = dpp_u32<CTRL, RM>(v, v);                                     \
    v = MAX ? max(v, o) : min(v, o);                                                \
  }
  MA_STEP(0x121, 0xf)
  MA_STEP(0x122, 0xf)
  MA_STEP(0x124, 0xf)
  MA_STEP(0x128, 0xf)
  MA_STEP(0x142, 0xa)
  MA_STEP(0x143, 0xc)
#undef MA_STEP
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the workgroup (two barriers; s_red holds kWaves words).
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *s_red) {
  v = wave_sum(v);
  if (lane_id() == 63) s_red[threadIdx.x >> 6] = v;
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
// output position of its chunk-c elements.  Every wave scans the NC*kWaves
// totals itself, so one barrier suffices.  s_cnt holds NC*kWaves words and
// must not be written again before the next barrier.
template <int NC>
__device__ __forceinline__ void ordered_offsets(const uint32_t (&cnt)[NC], uint32_t (&pos)[NC],
                                                uint32_t &total, uint32_t *s_cnt) {
  static_assert(NC * kWaves <= 64, "one wave scans the (chunk, wave) totals");
  constexpr int n = NC * kWaves;
  const int lane = lane_id(), wv = (int)(threadIdx.x >> 6);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t inc = wave_incl_scan(cnt[c]);
    pos[c] = inc - cnt[c];
    if (lane == 63) s_cnt[c * kWaves + wv] = inc;
  }
  __syncthreads();
  const uint32_t v = lane < n ? s_cnt[lane] : 0u;
  const uint32_t inc = wave_incl_scan(v);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
  for (int c = 0; c < NC; ++c) pos[c] += (uint32_t)__builtin_amdgcn_readlane((int)(inc - v), c * kWaves + wvu);
  total = (uint32_t)__builtin_amdgcn_readlane((int)inc, n - 1);
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
  int64_t *deferred;        // blocks the full-block kernel hands to the general path
  unsigned int *n_deferred; // their count
  // one (delta, Delta) over all d (two passes, QMODE 1 and 2)
  float *blkmm;             // [2*n_b] each block's residual min / max (pass 1)
  uint32_t *selinfo;        // [2*n_b] each block's cut: T, idx_last (0x7fffffff: every key T taken)
  const float *gmm;         // [2] the reduced global min / max (pass 2)
};

// Quantizer modes of the compressor: per block (0), or one pair over all d:
// pass 1 selects, writes the window row and records the block's residual
// min / max and its cut, leaving codes and statistics; pass 2 recomputes the
// residual from the same inputs, zeroes by the recorded cut and quantizes with
// the global pair (which it stores as every block's statistics).
enum { kQBlock = 0, kQGlobal1 = 1, kQGlobal2 = 2 };

template <int CPT>
struct CompressSmem {
  uint32_t red[kWaves];
  float redf[2 * kWaves];
  uint32_t cnt[CPT * kWaves + 1];
  uint2 cand[kCandMax];     // {bits of a, index}
  uint32_t sel[4];          // T, idx_last, exact cut
};

// Quantization code of one element (the third paragraph's unbiased Q):
// code = floor(y) + [u < frac(y) * 2^16], capped at 15, with y = (v - lo) * inv
// and u the element's 16-bit uniform.  With xi = u * 2^-16 this is
// min(ceil(y - xi), 15): for y >= xi the difference is exact in fp32 (y < 16,
// so y and xi are multiples of ulp(y) <= 2^-20, and so is their difference,
// which is at most y), and ceil(n + f - xi) = n + [f > xi]; for y < xi (so
// floor(y) = 0 and u > 2^16 y) it is <= 0.  Returned as a float holding the
// integer code (or -0).
__device__ __forceinline__ float quant_code_f(float v, float lo, float inv, uint32_t u) {
  const float y = (v - lo) * inv;
  const float z = fmaf((float)u, -1.0f / 65536.0f, y);
  return fminf(ceilf(z), 15.0f);
}

// One block of the compressor, templated on the chunk count (CPT), on whether
// every element of the thread's chunks exists (FULL: no bounds tests, vector
// loads), on 16-byte alignment of the gradient / 8-element alignment of the
// block (ALIGNED: one 16-byte gradient load and one 4-byte code word per
// thread and chunk) and on error feedback being on (EF).
// Inputs of one full block, staged ahead of its processing: the gradients and
// the packed codes go straight from global memory into LDS (LDS-DMA loads,
// no registers held while in flight), the block statistics and the window
// offsets into registers.
template <int CPT>
struct FullBlockStage {
  u32x4 g[CPT][kThreads];     // thread t's 8 gradients of chunk c at [c][t]
  uint32_t ef[CPT][kThreads]; // thread t's 8 codes of chunk c at [c][t]
};

template <int CPT>
struct FullBlockInputs {
  float lo, hi;
  int64_t off;
  int kb;
};

typedef __attribute__((address_space(3))) void lds_void_t;

template <int CPT, bool EF>
__device__ __forceinline__ void stage_full_block(const CompressArgs &A, int64_t j, FullBlockStage<CPT> &st,
                                                 FullBlockInputs<CPT> &in) {
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wbase = tid & ~63;   // a wave's lanes fill 64 consecutive LDS slots
  const int64_t s = j * (int64_t)A.B;
  // uniform block bases plus 32-bit lane offsets (scalar-base addressing)
  const u32x4 *gb = reinterpret_cast<const u32x4 *>(A.g + s);
  const uint32_t *eb = reinterpret_cast<const uint32_t *>(A.ef + (s >> 1));
  // the codes are streamed (non-temporal): the quantizer overwrites them with
  // streaming stores, and nothing else reads them this step
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(gb + (c * kThreads + tid)),
                                     (lds_void_t *)(&st.g[c][wbase]), 16, 0, 0);
    if (EF)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(eb + (c * kThreads + tid)),
                                       (lds_void_t *)(&st.ef[c][wbase]), 4, 0, kCacheStream);
  }
  in.lo = EF ? A.stats[2 * j] : 0.f;
  in.hi = EF ? A.stats[2 * j + 1] : 0.f;
  in.off = A.off_tab[j];
  in.kb = (int)(A.off_tab[j + 1] - in.off);
}

// Waits until this wave's outstanding vector-memory operations (including its
// LDS-DMA loads) are complete; the empty asm statements keep the compiler from
// moving LDS reads across the wait.
__device__ __forceinline__ void wait_vm_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt not waited on
  asm volatile("" ::: "memory");
}

// FULL path: st / raw hold the block's staged inputs.
// DEFER: a block the candidate path cannot finish (too many candidates, e.g.
// massive ties) is appended to A.deferred untouched, for the general path.
// The fused step's window bitmap, built by the compressor's idle waves.
struct FusedBits {
  uint32_t *bits;          // CPT * kChunkSpan / 32 words
  const uint32_t *ent;     // the block's window rows in LDS, row i at ent + i * es
  int es, M, tm;
};

// lds_row (optional): the window row is also written there, from index 0.
// lds_hash (optional, FULL only): LDS for the block's L/2 random words; while
// wave 0 selects, the other waves fill it, and the quantizer reads it.
// fb (optional): while wave 0 selects, the other waves build the bitmap of
// the positions in the window rows other than row tm, and wave 0 adds the
// positions it selects.
// Returns false when the block was deferred (DEFER) and left untouched.
template <int CPT, bool FULL, bool ALIGNED, bool EF, bool DEFER = false, int QMODE = kQBlock>
__device__ __forceinline__ bool compress_block(const CompressArgs &A, CompressSmem<CPT> &sm, int64_t j,
                                               int64_t s, int L, int64_t off, int kb,
                                               FullBlockStage<CPT> *st, const FullBlockInputs<CPT> *raw,
                                               uint32_t *lds_row = nullptr, uint32_t *lds_hash = nullptr,
                                               const FusedBits *fb = nullptr) {
  // The thread index is passed through an empty asm statement so that, inside
  // the persistent loop, values derived from it are recomputed per block
  // instead of being hoisted out of the loop and held in (spilled) registers.
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  __builtin_assume(tid >= 0 && tid < kThreads);
  // the wave index is uniform: a scalar register
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------- ef_dequant_accumulate: a = f32(g) + fmaf(code, step, delta)
  float lo = 0.f, step = 0.f;
  if (EF) {
    lo = (FULL && ALIGNED) ? raw->lo : A.stats[2 * j];
    const float hi = (FULL && ALIGNED) ? raw->hi : A.stats[2 * j + 1];
    step = (hi - lo) / 15.0f;
  }
  float a[CPT][kChunk];
  uint32_t oldc[CPT];
  if (FULL && ALIGNED) {
    wait_vm_all();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const uint32_t cwc = EF ? st->ef[c][tid] : 0u;
      const u32x4 gvc = st->g[c][tid];
      oldc[c] = cwc;
      const uint32_t gw[4] = {gvc.x, gvc.y, gvc.z, gvc.w};
      // even / odd codes as bytes; the empty asm keeps the masks, so each
      // code converts with one byte-select conversion
      uint32_t ce = cwc & 0x0f0f0f0fu, co = (cwc >> 4) & 0x0f0f0f0fu;
      asm volatile("" : "+v"(ce), "+v"(co));
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const float gf = (e & 1) ? u2f(gw[e >> 1] & 0xffff0000u) : u2f(gw[e >> 1] << 16);
        if (EF) {
          const uint32_t cb = (e & 1) ? co : ce;
          const float code = (float)((cb >> (8 * (e >> 1))) & 0xffu);
          a[c][e] = gf + fmaf(code, step, lo);
        } else {
          a[c][e] = gf;
        }
      }
    }
    // the fused bitmap's words alias the staged codes (word w is code word
    // w mod 512 of chunk w / 512, which only thread w mod 512 reads, above):
    // each thread clears its own words (ordered before the bitmap's use by the
    // selection's barriers)
    if (fb)
      for (int w = tid; w < CPT * kChunkSpan / 32; w += kThreads) fb->bits[w] = 0u;
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i0 = c * kChunkSpan + tid * kChunk;
      uint32_t cw = 0;
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = i0 + e;
        float v = 0.f;
        if (i < L) {
          const int64_t gi = s + i;
          const float gf = bf16_bits_to_f32(A.g[gi]);
          if (EF) {
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
#define MA_VALID(i) (FULL || (i) < L)

  // ---------------- block_topk: the k_b largest keys (topk_key: the 31-bit
  // pattern of |a|, NaN canonical), ties to the lower index.  For finite
  // thresholds the key order is the order of |a| as floats, so the passes over
  // all elements compare |a| (a free source modifier), written so that a NaN
  // compares above every finite threshold.  Result: threshold key T and
  // idx_last, the index of the last selected element with key T; an element is
  // selected iff key > T, or key == T and index <= idx_last.  exact: every
  // element with key T is selected (then "key >= T" alone decides).
  uint32_t T = 0x7f800000u;   // k_b = 0: the key of +inf, above every finite |a|
  int idx_last = -1;
  bool exact = true;
  bool hashed = false;         // lds_hash holds the block's random words
  if (QMODE == kQGlobal2) {
    T = A.selinfo[2 * j];
    idx_last = (int)A.selinfo[2 * j + 1];
    exact = idx_last == 0x7fffffff;
  } else if (kb > 0) {
    bool done = false;
    const int q = (kb + kWaves - 1) / kWaves;
    if (q <= 64 && kb < L) {
      // (1) candidate threshold tau with at least k_b keys >= tau: each wave
      // finds a value reached by q of its lane maxima; tau = their minimum, so
      // at least kWaves * q >= k_b distinct elements reach it.
      // For finite values the 31-bit key order is the order of |a| as floats,
      // so the streaming passes compare |a| (a free source modifier) instead of
      // materialising keys.  The lane maxima skip NaN (fmaxf), so tau is
      // reached by real elements; every NaN is a candidate below.
      float lanemax_f = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
          if (MA_VALID(c * kChunkSpan + tid * kChunk + e)) lanemax_f = fmaxf(lanemax_f, fabsf(a[c][e]));
      const uint32_t lanemax = f2u(lanemax_f);
      uint32_t P = 0;
      for (int b = 30; b >= kCoarseLowBit; --b) {
        const uint32_t cand = P | (1u << b);
        if ((int)__popcll(__ballot(lanemax >= cand)) >= q) P = cand;
      }
      if (lane == 0) sm.red[wv] = P;
      __syncthreads();
      uint32_t tau = sm.red[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) tau = min(tau, sm.red[w]);
      const float tau_f = u2f(tau);
      // (2) gather the candidates (key >= tau: !(|a| < tau), which NaN
      // passes) into LDS in index order
      uint32_t cnt[CPT], pos[CPT], C;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
          n += (MA_VALID(c * kChunkSpan + tid * kChunk + e) && !(fabsf(a[c][e]) < tau_f)) ? 1u : 0u;
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, C, sm.cnt);
      if (C <= (uint32_t)kCandMax) {
        // the counting pass's test, recomputed rather than kept (32 lane
        // masks held across the scan would spill): against a copy of tau the
        // compiler cannot see through
        float tau_g = tau_f;
        asm volatile("" : "+v"(tau_g));
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          uint32_t p = pos[c];
#pragma unroll
          for (int e = 0; e < kChunk; ++e) {
            const int i = c * kChunkSpan + tid * kChunk + e;
            const bool cd = MA_VALID(i) && !(fabsf(a[c][e]) < tau_g);
            // (a wave with no candidate at this element skips it: a third
            // of the waves at k = d/100)
            if (__builtin_amdgcn_ballot_w64(cd)) {
              if (cd) sm.cand[p] = make_uint2(f2u(a[c][e]), (uint32_t)i);
              p += cd ? 1u : 0u;
            }
          }
        }
        __syncthreads();
        // (3) one wave: the exact k_b-th largest key by MSB-first bit search,
        // the tie cut in index order, and the ordered write of (I, bf16(V))
        // into the window row (ring_write).
        if (wv == 0) {
          // the serial part of the block: ahead of the other waves on its SIMD
          __builtin_amdgcn_s_setprio(3);
          const int R = ((int)C + 63) >> 6;
          uint32_t ck[kCandMax / 64];
          uint32_t kmax = 0;
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r) {
            const int ci = r * 64 + lane;
            ck[r] = (r < R && ci < (int)C) ? topk_key(u2f(sm.cand[ci].x)) : 0u;
            kmax = max(kmax, ck[r]);
          }
          kmax = wave_minmax_u32<true>(kmax);
          // T lies in [tau, kmax], so it shares their common leading bits;
          // search the rest MSB first.  Invariant: count(key >= Pk) >= k_b.
          // Padding lanes hold key 0 and never reach a candidate value >= 1.
          const uint32_t diff = tau ^ kmax;
          const int hb = diff ? 31 - __clz(diff) : -1;
          uint32_t Pk = diff ? (tau & ~((2u << hb) - 1u)) : tau;
          bool cut = (diff == 0);   // all candidates share one key: T = tau, every tie taken
          for (int b = hb; b >= 0 && !cut; --b) {
            const uint32_t cand = Pk | (1u << b);
            int n = 0;
#pragma unroll
            for (int r = 0; r < kCandMax / 64; ++r)
              if (r < R) n += (int)__popcll(__ballot(ck[r] >= cand));
            if (n >= kb) {
              Pk = cand;
              if (n == kb) {
                // exactly k_b keys reach cand: they are the selection and T is
                // their smallest key (no key equal to it is left out)
                uint32_t mn = 0xffffffffu;
#pragma unroll
                for (int r = 0; r < kCandMax / 64; ++r)
                  if (r < R && ck[r] >= cand) mn = min(mn, ck[r]);
                Pk = wave_minmax_u32<false>(mn);
                cut = true;
              }
            }
          }
          int last = 0x7fffffff;   // with a clean cut every key == T is selected
          int ntie = 0, need = 0;
          if (!cut) {
            int ngt = 0;
#pragma unroll
            for (int r = 0; r < kCandMax / 64; ++r)
              if (r < R) {
                ngt += (int)__popcll(__ballot(r * 64 + lane < (int)C && ck[r] > Pk));
                ntie += (int)__popcll(__ballot(r * 64 + lane < (int)C && ck[r] == Pk));
              }
            need = kb - ngt;   // >= 1 elements with key Pk are taken, lowest index first
            if (ntie != need) {
              int run = 0;
              last = -1;
#pragma unroll
              for (int r = 0; r < kCandMax / 64; ++r) {
                if (r < R && last < 0) {
                  const bool tie = r * 64 + lane < (int)C && ck[r] == Pk;
                  const uint64_t m = __ballot(tie);
                  const int pc = (int)__popcll(m);
                  if (run + pc >= need) {
                    const bool hit = tie && (int)lanes_below(m) == need - run - 1;
                    const int src = __ffsll((long long)__ballot(hit)) - 1;
                    last = __shfl((int)sm.cand[r * 64 + lane].y, src, 64);
                  }
                  run += pc;
                }
              }
            }
          }
          // ring_write: the selected candidates, already in index order
          uint32_t *dst = A.G + A.row_base + off;
          int wrote = 0;
#pragma unroll
          for (int r = 0; r < kCandMax / 64; ++r) {
            if (r < R) {
              const int ci = r * 64 + lane;
              const bool in = ci < (int)C;
              const int idx = in ? (int)sm.cand[ci].y : 0;
              const bool sel = in && (ck[r] > Pk || (ck[r] == Pk && idx <= last));
              const uint64_t m = __ballot(sel);
              if (sel) {
                const uint32_t ent = (uint32_t)idx | (window_bf16(sm.cand[ci].x, ck[r]) << 16);
                dst[wrote + (int)lanes_below(m)] = ent;
                if (lds_row) lds_row[wrote + (int)lanes_below(m)] = ent;
                if (fb && (ent & 0x7fff0000u)) atomicOr(&fb->bits[idx >> 5], 1u << (idx & 31));
              }
              wrote += (int)__popcll(m);
            }
          }
          if (lane == 0) {
            // a non-finite threshold key is handed on as "every key >= +Inf's"
            // (only non-finite values are selected, and all of them become 0)
            sm.sel[0] = min(Pk, kKeyInf);
            sm.sel[1] = (uint32_t)last;
            sm.sel[2] = (cut || ntie == need || Pk >= kKeyInf) ? 1u : 0u;
          }
          __builtin_amdgcn_s_setprio(0);
        } else {
          // the other waves, meanwhile: the quantizer's random words and the
          // bitmap of the window's other rows
          const int t7 = tid - 64;
          if (EF && QMODE == kQBlock && lds_hash) {
            // four consecutive words (one 16-byte LDS store) per thread and turn
            constexpr int kStride = kThreads - 64;
            uint32_t st = pcg_state(philox_block_key(A.seed, A.t, j) + 4u * (uint32_t)t7);
            for (int q = t7; q < L / 8; q += kStride, st += 4u * (uint32_t)kStride * kPcgMul) {
              u32x4 v;
              v.x = pcg_out(st);
              v.y = pcg_out(st + kPcgMul);
              v.z = pcg_out(st + 2u * kPcgMul);
              v.w = pcg_out(st + 3u * kPcgMul);
              reinterpret_cast<u32x4 *>(lds_hash)[q] = v;
            }
          }
          if (fb) {
            for (int i = 0; i < fb->M; ++i) {
              if (i == fb->tm) continue;
              for (int q = t7; q < kb; q += kThreads - 64) {
                const uint32_t e = fb->ent[i * fb->es + q];
                if ((e & 0x7fff0000u) && (int)(e & 0xffffu) < L)
                  atomicOr(&fb->bits[(e & 0xffffu) >> 5], 1u << (e & 31u));
              }
            }
          }
        }
        __syncthreads();
        hashed = EF && QMODE == kQBlock && lds_hash != nullptr;
        T = sm.sel[0];
        idx_last = (int)sm.sel[1];
        exact = sm.sel[2] != 0;
        done = true;
      }
    }
    if (DEFER && !done) {
      if (tid == 0) A.deferred[atomicAdd(A.n_deferred, 1u)] = j;
      return false;
    }
    if (!DEFER && !done) {
      // General path (k_b > 512, k_b == L, or too many candidates): exact
      // MSB-first bit search over the whole block with workgroup counts, on
      // the keys themselves (any key, NaN and +-Inf included).
      uint32_t P = 0;
      for (int b = 30; b >= 0; --b) {
        const uint32_t cand = P | (1u << b);
        uint32_t n = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
          for (int e = 0; e < kChunk; ++e)
            n += (MA_VALID(c * kChunkSpan + tid * kChunk + e) && topk_key(a[c][e]) >= cand) ? 1u : 0u;
        if ((int)block_sum(n, sm.red) >= kb) P = cand;
      }
      uint32_t ngt = 0;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
          ngt += (MA_VALID(c * kChunkSpan + tid * kChunk + e) && topk_key(a[c][e]) > P) ? 1u : 0u;
      const int need = kb - (int)block_sum(ngt, sm.red);
      uint32_t cnt[CPT], pos[CPT], tot;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
          n += (MA_VALID(c * kChunkSpan + tid * kChunk + e) && topk_key(a[c][e]) == P) ? 1u : 0u;
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, tot, sm.cnt);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t p = pos[c];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          if (MA_VALID(i) && topk_key(a[c][e]) == P) {
            if ((int)p == need - 1) sm.sel[1] = (uint32_t)i;
            ++p;
          }
        }
      }
      __syncthreads();
      T = P;
      idx_last = (int)sm.sel[1];
      exact = ((int)tot == need);
      // ring_write of every selected element, in index order
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t n = 0;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          const uint32_t x = topk_key(a[c][e]);
          n += (MA_VALID(i) && (x > T || (x == T && i <= idx_last))) ? 1u : 0u;
        }
        cnt[c] = n;
      }
      ordered_offsets<CPT>(cnt, pos, tot, sm.cnt);
      uint32_t *dst = A.G + A.row_base + off;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint32_t p = pos[c];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int i = c * kChunkSpan + tid * kChunk + e;
          const uint32_t x = topk_key(a[c][e]);
          if (MA_VALID(i) && (x > T || (x == T && i <= idx_last))) {
            const uint32_t ent = (uint32_t)i | (window_bf16(f2u(a[c][e]), x) << 16);
            dst[p] = ent;
            if (lds_row) lds_row[p] = ent;
            ++p;
          }
        }
      }
      // as in the candidate path, a non-finite threshold key is handed on to
      // the zeroing as +Inf's, exact
      if (T >= kKeyInf) {
        T = kKeyInf;
        exact = true;
      }
    }
  }

  if (!EF) return true;   // no error feedback: codes and statistics are left as they are

  // ---------------- zero the selected entries; block min / max of the residual.
  // A non-finite value left after the selection (more than k_b of them in the
  // block) is dropped from the error feedback: it becomes +0 like a selected
  // one.  With a finite threshold every non-finite value is selected, and the
  // float tests below (NaN fails every ordered compare) decide alone; with a
  // non-finite threshold key only non-finite values are selected and all of
  // them become 0 either way, which is the exact test against +Inf (the
  // selection hands such a cut on as T = +Inf's key, exact).
  float mn = __int_as_float(0x7f800000), mx = -__int_as_float(0x7f800000);
  if (exact) {
    // selected (or dropped) <=> key >= T <=> !(|a| < T)
    const float T_f = u2f(T);
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = c * kChunkSpan + tid * kChunk + e;
        a[c][e] = (fabsf(a[c][e]) < T_f) ? a[c][e] : 0.0f;
        if (MA_VALID(i)) {
          mn = fminf(mn, a[c][e]);
          mx = fmaxf(mx, a[c][e]);
        }
      }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = c * kChunkSpan + tid * kChunk + e;
        const float x = fabsf(a[c][e]);
        const bool sel = !(x <= u2f(T)) || (x == u2f(T) && i <= idx_last);
        a[c][e] = sel ? 0.0f : a[c][e];
        if (MA_VALID(i)) {
          mn = fminf(mn, a[c][e]);
          mx = fmaxf(mx, a[c][e]);
        }
      }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { sm.redf[wv] = mn; sm.redf[kWaves + wv] = mx; }   // uniform values
  __syncthreads();
  mn = sm.redf[0];
  mx = sm.redf[kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    mn = fminf(mn, sm.redf[w]);
    mx = fmaxf(mx, sm.redf[kWaves + w]);
  }
  mn = mn + 0.0f;   // a zero extreme is stored as +0
  mx = mx + 0.0f;
  // a range with no finite fp32 value (both signs near the fp32 limit) resets
  // the block's error feedback: delta = Delta = 0, every code 0 (for the
  // global pair this is decided on the pair, in global_minmax_kernel)
  if (QMODE == kQBlock && !(mx - mn <= 3.402823466e38f)) {
    mn = 0.0f;
    mx = 0.0f;
  }
  if (QMODE == kQGlobal1) {
    if (tid == 0) {
      A.blkmm[2 * j] = mn;
      A.blkmm[2 * j + 1] = mx;
      A.selinfo[2 * j] = T;
      A.selinfo[2 * j + 1] = exact ? 0x7fffffffu : (uint32_t)idx_last;
    }
    return true;
  }
  if (QMODE == kQGlobal2) {
    mn = A.gmm[0];
    mx = A.gmm[1];
  }

  // ---------------- ef_requant: unbiased stochastic 4-bit rounding.  A
  // constant block, or one whose scale 15/(Delta - delta) overflows fp32,
  // gets code 0 everywhere.
  const float inv = (mx == mn) ? 0.f : 15.0f / (mx - mn);
  const bool flat = (mx == mn) || !(inv <= 3.402823466e38f);
  const uint32_t bkey = hashed ? 0u : philox_block_key(A.seed, A.t, j);
  // the thread's LDS address, derived afresh: the one of the staged inputs'
  // reads would otherwise be held across the selection (a spilled register)
  int tq = (int)threadIdx.x;
  asm volatile("" : "+v"(tq));
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    // keep the scheduler from interleaving chunks (register pressure)
    __builtin_amdgcn_sched_barrier(0);
    const int i0 = c * kChunkSpan + tid * kChunk;
    uint32_t packed = 0;
    if (!flat) {
      // even elements' codes go to the bytes of ev, odd ones to od (the
      // byte conversion saturates, so -0 becomes 0), then nibbles interleave
      uint32_t ev = 0, od = 0;
      uint32_t hw[kChunk / 2] = {0u, 0u, 0u, 0u};
      if (FULL && hashed) {
        const u32x4 hv = reinterpret_cast<const u32x4 *>(lds_hash)[c * kThreads + tq];
        hw[0] = hv.x; hw[1] = hv.y; hw[2] = hv.z; hw[3] = hv.w;
      }
#pragma unroll
      for (int pr = 0; pr < kChunk / 2; ++pr) {
        const uint32_t h = (FULL && hashed) ? hw[pr] : pcg_out(pcg_state(bkey + (uint32_t)(i0 >> 1)) + (uint32_t)pr * kPcgMul);
        ev = __builtin_amdgcn_cvt_pk_u8_f32(quant_code_f(a[c][2 * pr], mn, inv, h & 0xffffu), pr, ev);
        od = __builtin_amdgcn_cvt_pk_u8_f32(quant_code_f(a[c][2 * pr + 1], mn, inv, h >> 16), pr, od);
      }
      packed = ev | (od << 4);
    }
    if (!FULL) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e)
        if (i0 + e >= L) packed &= ~(15u << (4 * e));
    }
    if (ALIGNED) {
      // element s + i0 starts code word (s + i0) / 8 of the block's aligned run
      // a streaming store (non-temporal): nothing reads the codes again this
      // step, and L2 keeps the lines the update will write instead
      if (FULL || i0 < L)
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(A.ef + (s >> 1)) + c * kThreads + tid);
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
#undef MA_VALID
  return true;
}

// The compressor kernels: one workgroup per block.  compress_full_kernel
// serves blocks whose every element exists and is aligned (B_d = CPT * 4096,
// 16-byte aligned gradients): blocks first_block .. first_block + grid - 1.
// compress_kernel serves the rest with bounds tests, over the same kind of
// range.  A block the full kernel defers is appended to A.deferred (whose
// count is *A.n_deferred) and finished by compress_deferred_kernel.
template <int CPT, bool EF, int QMODE = kQBlock>
__global__ __launch_bounds__(kThreads, MA_FULL_WAVES) void compress_full_kernel(CompressArgs A, int64_t first_block) {
  __shared__ CompressSmem<CPT> sm;
  __shared__ FullBlockStage<CPT> st;
  const int64_t j = first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  FullBlockInputs<CPT> in;
  stage_full_block<CPT, EF>(A, j, st, in);
  compress_block<CPT, true, true, EF, QMODE != kQGlobal2, QMODE>(A, sm, j, j * (int64_t)A.B, CPT * kChunkSpan, in.off,
                                                               in.kb, &st, &in, nullptr,
                                                               reinterpret_cast<uint32_t *>(&st));
}

template <int CPT, bool EF, int QMODE = kQBlock>
__global__ __launch_bounds__(kThreads) void compress_deferred_kernel(CompressArgs A) {
  __shared__ CompressSmem<CPT> sm;
  __shared__ FullBlockStage<CPT> st;
  const unsigned int n = *A.n_deferred;
  for (unsigned int q = blockIdx.x; q < n; q += gridDim.x) {
    const int64_t j = A.deferred[q];
    FullBlockInputs<CPT> in;
    stage_full_block<CPT, EF>(A, j, st, in);
    compress_block<CPT, true, true, EF, false, QMODE>(A, sm, j, j * (int64_t)A.B, CPT * kChunkSpan, in.off, in.kb,
                                                      &st, &in, nullptr, reinterpret_cast<uint32_t *>(&st));
    __syncthreads();
  }
}

__global__ void zero_u32_kernel(unsigned int *p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

template <int CPT, bool ALIGNED, bool EF, int QMODE = kQBlock>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs A, int64_t first_block) {
  __shared__ CompressSmem<CPT> sm;
  const int64_t j = first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  const int64_t s = j * (int64_t)A.B;
  const int L = (int)((A.d - s) < (int64_t)A.B ? (A.d - s) : (int64_t)A.B);
  const int64_t off = A.off_tab[j];
  const int kb = (int)(A.off_tab[j + 1] - off);
  compress_block<CPT, false, ALIGNED, EF, false, QMODE>(A, sm, j, s, L, off, kb, nullptr, nullptr);
}

// The global residual min / max from the blocks' (pass 1 to pass 2 of the
// global quantizer): one workgroup; min and max are exact, so the order of
// reduction does not matter; a zero extreme is stored as +0.
__global__ __launch_bounds__(kThreads) void global_minmax_kernel(const float *blkmm, int64_t n_b, float *gmm) {
  __shared__ float red[2 * kWaves];
  float mn = __int_as_float(0x7f800000), mx = -__int_as_float(0x7f800000);
  for (int64_t j = threadIdx.x; j < n_b; j += kThreads) {
    mn = fminf(mn, blkmm[2 * j]);
    mx = fmaxf(mx, blkmm[2 * j + 1]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int wv = (int)(threadIdx.x >> 6);
  if (lane_id() == 0) { red[wv] = mn; red[kWaves + wv] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) {
      mn = fminf(mn, red[w]);
      mx = fmaxf(mx, red[kWaves + w]);
    }
    mn = fminf(mn, red[0]);
    mx = fmaxf(mx, red[kWaves]);
    if (!(mx - mn <= 3.402823466e38f)) {   // no finite range: the error feedback is reset
      mn = 0.0f;
      mx = 0.0f;
    }
    gmm[0] = mn + 0.0f;
    gmm[1] = mx + 0.0f;
  }
}

// ------------------------------------------------------------------ adamstats_apply

struct ApplyArgs {
  float *theta;             // fp32 parameters [d] (MODE 0, 1)
  uint16_t *theta16;        // or bfloat16 parameters [d] (the BF variants)
  const uint32_t *G;        // window [m][k]
  const int64_t *off_tab;   // [n_b + 1]
  const float *betapow;     // [2m]: beta1^r, then beta2^r, r = 0..m-1
  float *mhat, *vhat;       // MODE 2 outputs [nblocks][B]
  const int64_t *blocks;    // MODE 2 block list; the deferred-block list of apply_list_kernel
  const unsigned int *n_list;   // apply_list_kernel: number of blocks in `blocks`
  unsigned long long *touched;   // optional: kTouchedSlots partial sums of touched positions
  int64_t d, k, n_b;
  int64_t first_block;      // MODE 0, 1: blocks first_block .. first_block + grid - 1
  int32_t B, m, tm, cap;    // tm = t mod m; cap = LDS slots per pass
  int32_t ent_cap;          // window entries the LDS copy holds (m*k_b must fit to use it)
  int32_t csu_slots;        // column-sorted update: slot words (min(B_d, m * max k_b))
  int32_t fused_union_words;  // step_csu_kernel: LDS words shared by its two phases
  int32_t thl_off, thl_n;   // step_csu_kernel, THL: LDS word offset and length (floats) of the parameter chunk
  float c1, c2, lr, eps, decay;
};

enum { kModeSparse = 0, kModeDense = 1, kModeMoments = 2 };

// Parameter access for fp32 (BF false) or bfloat16 (BF true) parameters.  A
// bfloat16 parameter is widened exactly, updated in fp32 like an fp32 one, and
// the result rounded to nearest even once.
template <bool BF>
__device__ __forceinline__ float ld_param(const ApplyArgs &A, int64_t i) {
  return BF ? bf16_bits_to_f32(A.theta16[i]) : A.theta[i];
}
template <bool BF>
__device__ __forceinline__ void st_param(const ApplyArgs &A, int64_t i, float v) {
  // streaming stores: nothing reads the parameters again this step
  if (BF)
    __builtin_nontemporal_store((uint16_t)f32_to_bf16_rne(v), A.theta16 + i);
  else
    __builtin_nontemporal_store(v, A.theta + i);
}
constexpr int kThetaPerThread = 8;   // parameters a thread holds in flight in the sparse update
constexpr int kMaxWindow = 1024;     // window rows the update kernels take (their factors sit in LDS)
constexpr int kFusedBeta = 64;       // decay factors the fused kernel holds (2m, so m <= 32)
constexpr int kTouchedSlots = 1024;  // counters the touched-parameter sum is spread over

// LDS of the update: bitmap of touched positions (W words), per-word slot
// base (W words), the block's window entries (row i at ent + i * ent_stride,
// when in_lds), and per slot z1, z2 (fp32) and its position (u16), cap slots
// per pass; cnt holds kWaves + 1 words.
struct ApplySmem {
  uint32_t *bits, *wbase, *ent;
  float *beta;   // the 2m decay factors, staged in LDS
  float *z1, *z2;
  uint16_t *pos;
  uint32_t *cnt;
  int cap, ent_stride;
  bool in_lds;
  int64_t off;   // PRELOADED: the block's window offset and k_b, already known
  int kb;
};

// A decay factor from the LDS table, read through an LDS-typed pointer (a
// generic load would be counted with vector memory, and waiting for it would
// also wait for the parameter loads in flight).
typedef __attribute__((address_space(3))) float lds_float_t;
__device__ __forceinline__ float decay_factor(const float *beta, int idx) {
  return ((const lds_float_t *)beta)[idx];
}

// Issues the LDS-DMA of the 2m decay factors into beta.  The caller waits for
// its vector memory and a barrier before the table is read.
__device__ __forceinline__ void stage_beta(const ApplyArgs &A, float *beta, int tid) {
  const int n = 2 * A.m;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int w0 = wv * 64; w0 < n; w0 += kThreads)
    if (w0 + lane < n)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(A.betapow + w0 + lane),
                                       (lds_void_t *)(beta + w0), 4, 0, 0);
}

// sqrtf(x), correctly rounded, for every active lane.  Where every active
// lane's x is finite and at least 2^-96: the hardware estimate (within one
// ulp) replaced by a neighbour when the residual x - n * s of that neighbour
// n says it is nearer (the correction sqrtf itself applies; its scaling of
// small inputs and its special cases are not needed in that range).  For any
// other wave, sqrtf.  Correct rounding makes the two agree bit for bit.
__device__ __forceinline__ float sqrt_rn(float x) {
  // x in [2^-96, FLT_MAX] (not negative, not NaN): one unsigned compare
  const bool wide = f2u(x) - 0x0f800000u <= 0x7f7fffffu - 0x0f800000u;
  if (__builtin_amdgcn_ballot_w64(wide) == __builtin_amdgcn_read_exec()) {
    const float s = __builtin_amdgcn_sqrtf(x);
    const float lo = u2f(f2u(s) - 1u), hi = u2f(f2u(s) + 1u);
    const float r = (fmaf(-lo, s, x) <= 0.0f) ? lo : s;
    return (fmaf(-hi, s, x) > 0.0f) ? hi : r;
  }
  return sqrtf(x);
}

// The same factors by physical window row: beta[i] = beta1^r and
// beta[m + i] = beta2^r, r = (tm - i) mod m the age of row i this step (the
// column sums look them up by a key's row).
__device__ __forceinline__ void stage_beta_rows(const ApplyArgs &A, float *beta, int tid) {
  const int n = 2 * A.m;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int w0 = wv * 64; w0 < n; w0 += kThreads) {
    const int i = w0 + lane;
    if (i < n) {
      const int half = i >= A.m ? A.m : 0;
      int r = A.tm - (i - half);
      if (r < 0) r += A.m;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(A.betapow + half + r),
                                       (lds_void_t *)(beta + w0), 4, 0, 0);
    }
  }
}

// The update of block j.
// MODE 0: only touched parameters are read and written (decay must be 1).
// MODE 1: the block's parameters are streamed through registers; decoupled
//         decay on all, the Adam step on the touched ones.
// MODE 2: write m_hat and v_hat of the block to row out_row of the outputs;
//         parameters untouched.
// PRELOADED: the block's window entries are already in sm.ent.
template <int CPT, int MODE, bool ALIGNED, bool PRELOADED, bool BF = false>
__device__ __forceinline__ void apply_block(const ApplyArgs &A, int64_t j, int64_t out_row, const ApplySmem &sm) {
  constexpr int W = CPT * kChunkSpan / 32;          // bitmap words
  constexpr int WPT = (W + kThreads - 1) / kThreads;
  uint32_t *s_bits = sm.bits;
  uint32_t *s_wbase = sm.wbase;
  uint32_t *s_ent = sm.ent;
  float *s_z1 = sm.z1;
  float *s_z2 = sm.z2;
  uint16_t *s_pos = sm.pos;
  uint32_t *s_cnt = sm.cnt;

  // thread-derived addresses are recomputed here rather than carried over
  // (in registers, or spilled) from the compressor of the fused kernel
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  __builtin_assume(tid >= 0 && tid < kThreads);
  const int64_t s = j * (int64_t)A.B;
  const int L = (int)((A.d - s) < (int64_t)A.B ? (A.d - s) : (int64_t)A.B);
  const int64_t off = PRELOADED ? sm.off : A.off_tab[j];
  const int kb = PRELOADED ? sm.kb : (int)(A.off_tab[j + 1] - off);
  const int M = A.m;
  const bool in_lds = PRELOADED || sm.in_lds;
  const int es = PRELOADED ? sm.ent_stride : kb;   // LDS row stride of the entries

  if (!PRELOADED) {
    for (int w = tid; w < W; w += kThreads) s_bits[w] = 0;
    __syncthreads();
  }

  // ---------------- the block's window entries and their union bitmap.  A
  // zero value adds nothing (unwritten rows are all zero); an index outside
  // the block (only possible in an imported state) is ignored.
  // (PRELOADED: the entries and the bitmap are already complete)
  // Entries that fit in LDS: every thread DMAs its share of the m * k_b
  // entries straight to LDS, all in flight at once (one memory round trip),
  // then the bitmap is built from LDS.  Otherwise one pass over global memory
  // with 8 rows in flight per thread builds the bitmap, and the rows are read
  // again from global memory when they are added.
  if (!PRELOADED) stage_beta(A, sm.beta, tid);
  const bool win_dma = !PRELOADED && in_lds;
  if (win_dma) {
    const int tot = M * kb;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int x0 = wv * 64; x0 < tot; x0 += kThreads) {
      const int x = x0 + lane;
      if (x < tot) {
        const int i = x / kb, q = x - i * kb;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(A.G + (int64_t)i * A.k + off + q),
                                         (lds_void_t *)(&s_ent[x0]), 4, 0, kCacheStream);
      }
    }
    wait_vm_all();
    __syncthreads();
    for (int x = tid; x < tot; x += kThreads) {
      const uint32_t e = s_ent[x];
      if ((e & 0x7fff0000u) && (int)(e & 0xffffu) < L)
        atomicOr(&s_bits[(e & 0xffffu) >> 5], 1u << (e & 31u));
    }
  }
  for (int i0 = 0; !PRELOADED && !win_dma && i0 < M; i0 += 8) {
    for (int q = tid; q < kb; q += kThreads) {
      uint32_t e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        e[u] = (i0 + u < M) ? A.G[(int64_t)(i0 + u) * A.k + off + q] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (i0 + u < M) {
          if (in_lds) s_ent[(i0 + u) * es + q] = e[u];
          if ((e[u] & 0x7fff0000u) && (int)(e[u] & 0xffffu) < L)
            atomicOr(&s_bits[(e[u] & 0xffffu) >> 5], 1u << (e[u] & 31u));
        }
      }
    }
  }
  if (!PRELOADED) {
    wait_vm_all();   // the decay factors' DMA (the window DMA is waited for above)
    __syncthreads();
  }

  // ---------------- compact slots: slot(p) = number of touched positions below p
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

  if (MODE == kModeMoments) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = c * kChunkSpan + tid * kChunk + e;
        if (i < L) {
          A.mhat[out_row * A.B + i] = 0.f;
          A.vhat[out_row * A.B + i] = 0.f;
        }
      }
  }
  // sparse update: slots per pass limited by what the threads hold in flight
  const uint32_t pass = (MODE == kModeSparse) ? min((uint32_t)sm.cap, (uint32_t)(kThreads * kThetaPerThread))
                                              : (uint32_t)sm.cap;
  __syncthreads();

  for (uint32_t s0 = 0; s0 < U; s0 += pass) {
    const uint32_t n = min(pass, U - s0);
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
    // the touched parameters of this pass, loaded before the row scatter so
    // their latency overlaps it
    // (Every load is issued, lanes past the pass re-loading its last slot,
    // and every loaded value is used: a register cleared instead, or a load
    // waited for on one path only, makes the compiler wait for all vector
    // memory, the compressor's stores included, at the next pass.)
    float thv[kThetaPerThread];
    if (MODE == kModeSparse) {
#pragma unroll
      for (int u = 0; u < kThetaPerThread; ++u) {
        const uint32_t x = min((uint32_t)tid + (uint32_t)(u * kThreads), n - 1u);
        thv[u] = ld_param<BF>(A, s + s_pos[x]);
      }
    }
    // dense: the thread's 8 consecutive parameters of each chunk, streamed
    // when any of them is touched (or all of them in the decay pass)
    const bool decay_pass = (MODE == kModeDense) && s0 == 0 && A.decay != 1.0f;
    float th[CPT][kChunk];
    uint32_t tb[CPT];
    // (fp32 parameters in the fused kernel: the dense loads wait until after
    // the row sums, the block's parameters would otherwise stay in registers
    // across them; measured faster for fp32 and slower for bf16, whose
    // parameters take half the registers)
    constexpr bool kLateTheta = MODE == kModeDense && PRELOADED && !BF;
    auto load_theta = [&]() {
      if (MODE == kModeDense) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int i0 = c * kChunkSpan + tid * kChunk;
          tb[c] = (i0 < L) ? (s_bits[i0 >> 5] >> (i0 & 31)) & 0xffu : 0u;
          tb[c] |= tb[c] ? 0x100u : 0u;   // bit 8: the thread's 8 parameters are streamed
          if ((tb[c] >> 8) || (decay_pass && i0 < L)) {
            if (ALIGNED && BF && i0 + kChunk <= L) {
              const u32x4 w = *reinterpret_cast<const u32x4 *>(A.theta16 + s + i0);
              const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
              for (int e = 0; e < kChunk; ++e)
                th[c][e] = (e & 1) ? u2f(ww[e >> 1] & 0xffff0000u) : u2f(ww[e >> 1] << 16);
            } else if (ALIGNED && i0 + kChunk <= L) {
              const float4 v0 = *reinterpret_cast<const float4 *>(A.theta + s + i0);
              const float4 v1 = *reinterpret_cast<const float4 *>(A.theta + s + i0 + 4);
              th[c][0] = v0.x; th[c][1] = v0.y; th[c][2] = v0.z; th[c][3] = v0.w;
              th[c][4] = v1.x; th[c][5] = v1.y; th[c][6] = v1.z; th[c][7] = v1.w;
            } else {
#pragma unroll
              for (int e = 0; e < kChunk; ++e) th[c][e] = (i0 + e < L) ? ld_param<BF>(A, s + i0 + e) : 0.f;
            }
          } else {
#pragma unroll
            for (int e = 0; e < kChunk; ++e) th[c][e] = 0.f;
          }
        }
      }
    };
    if (!kLateTheta) load_theta();
    // AdamStats: z[I] += beta^r V, rows in physical order, one row at a time.
    // Entries in LDS with at most one per thread and row: the thread's
    // entries of 8 rows at a time are looked up (slot, V) before the rows are
    // added, so each row costs one read-add-write of z and a barrier.
    if (in_lds && kb <= kThreads) {
      for (int i0 = 0; i0 < M; i0 += 8) {
        uint32_t slv[8];
        float vv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          slv[u] = 0xffffffffu;
          vv[u] = 0.f;
          if (i0 + u < M && tid < kb) {
            const uint32_t e = s_ent[(i0 + u) * es + tid];
            const uint32_t I = e & 0xffffu;
            if ((e & 0x7fff0000u) && (int)I < L) {
              slv[u] = s_wbase[I >> 5] + (uint32_t)__popc(s_bits[I >> 5] & ((1u << (I & 31u)) - 1u)) - s0;
              vv[u] = bf16_bits_to_f32(e >> 16);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u;
          if (i < M) {
            int r = A.tm - i;
            if (r < 0) r += M;
            const float f1 = decay_factor(sm.beta, r), f2 = decay_factor(sm.beta, M + r);
            if (slv[u] < n) {
              // both read before either is written: one LDS round trip, not two
              const float a1 = s_z1[slv[u]], a2 = s_z2[slv[u]];
              s_z1[slv[u]] = a1 + f1 * vv[u];
              s_z2[slv[u]] = a2 + f2 * (vv[u] * vv[u]);
            }
            __syncthreads();
          }
        }
      }
    }
    for (int i = 0; !(in_lds && kb <= kThreads) && i < M; ++i) {
      int r = A.tm - i;
      if (r < 0) r += M;
      const float f1 = decay_factor(sm.beta, r), f2 = decay_factor(sm.beta, M + r);
      for (int q = tid; q < kb; q += kThreads) {
        const uint32_t e = in_lds ? s_ent[i * es + q] : A.G[(int64_t)i * A.k + off + q];
        const uint32_t I = e & 0xffffu;
        if (!(e & 0x7fff0000u) || (int)I >= L) continue;
        const float V = bf16_bits_to_f32(e >> 16);
        const uint32_t sl = s_wbase[I >> 5] + (uint32_t)__popc(s_bits[I >> 5] & ((1u << (I & 31u)) - 1u)) - s0;
        if (sl < n) {
          const float a1 = s_z1[sl], a2 = s_z2[sl];
          s_z1[sl] = a1 + f1 * V;
          s_z2[sl] = a2 + f2 * (V * V);
        }
      }
      __syncthreads();
    }
    if (kLateTheta) load_theta();
    // m_hat = c1 z1, v_hat = c2 z2; theta -= lr * m_hat / (sqrt(v_hat) + eps)
    if (MODE == kModeSparse) {
#pragma unroll
      for (int u = 0; u < kThetaPerThread; ++u) {
        const uint32_t x = (uint32_t)tid + (uint32_t)(u * kThreads);
        const float th = thv[u];
        asm volatile("" ::"v"(th));   // the wait for the load, on every path
        if (x < n) {
          const float mh = A.c1 * s_z1[x];
          const float vh = A.c2 * s_z2[x];
          st_param<BF>(A, s + s_pos[x], th - A.lr * (mh / (sqrt_rn(vh) + A.eps)));
        }
      }
    } else if (MODE == kModeDense) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int i0 = c * kChunkSpan + tid * kChunk;
        if ((tb[c] >> 8) || (decay_pass && i0 < L)) {
          const uint32_t word = s_bits[i0 >> 5];
          const uint32_t base = s_wbase[i0 >> 5];
#pragma unroll
          for (int e = 0; e < kChunk; ++e) {
            if (decay_pass) th[c][e] = th[c][e] * A.decay;
            if ((tb[c] >> e) & 1u) {   // e < 8: the position's own bit
              const int bit = (i0 & 31) + e;
              const uint32_t sl = base + (uint32_t)__popc(word & ((1u << bit) - 1u)) - s0;
              if (sl < n) {
                const float mh = A.c1 * s_z1[sl];
                const float vh = A.c2 * s_z2[sl];
                th[c][e] = th[c][e] - A.lr * (mh / (sqrt_rn(vh) + A.eps));
              }
            }
          }
          if (ALIGNED && BF && i0 + kChunk <= L) {
            u32x4 w;
            w.x = f32_to_bf16_rne(th[c][0]) | (f32_to_bf16_rne(th[c][1]) << 16);
            w.y = f32_to_bf16_rne(th[c][2]) | (f32_to_bf16_rne(th[c][3]) << 16);
            w.z = f32_to_bf16_rne(th[c][4]) | (f32_to_bf16_rne(th[c][5]) << 16);
            w.w = f32_to_bf16_rne(th[c][6]) | (f32_to_bf16_rne(th[c][7]) << 16);
            *reinterpret_cast<u32x4 *>(A.theta16 + s + i0) = w;
          } else if (ALIGNED && i0 + kChunk <= L) {
            *reinterpret_cast<float4 *>(A.theta + s + i0) = make_float4(th[c][0], th[c][1], th[c][2], th[c][3]);
            *reinterpret_cast<float4 *>(A.theta + s + i0 + 4) = make_float4(th[c][4], th[c][5], th[c][6], th[c][7]);
          } else {
#pragma unroll
            for (int e = 0; e < kChunk; ++e)
              if (i0 + e < L) st_param<BF>(A, s + i0 + e, th[c][e]);
          }
        }
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
                A.mhat[out_row * A.B + i] = A.c1 * s_z1[sl];
                A.vhat[out_row * A.B + i] = A.c2 * s_z2[sl];
              }
            }
          }
        }
    }
    // the next pass reuses the slot arrays; after the last pass no barrier
    // (it would wait for the parameter stores to complete)
    if (s0 + pass < U) __syncthreads();
  }
  if (MODE == kModeDense && U == 0 && A.decay != 1.0f) {
    // nothing touched: the decay alone
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int i0 = c * kChunkSpan + tid * kChunk;
#pragma unroll
      for (int e = 0; e < kChunk; ++e)
        if (i0 + e < L) st_param<BF>(A, s + i0 + e, ld_param<BF>(A, s + i0 + e) * A.decay);
    }
  }
  // the touched count, spread over kTouchedSlots counters so the blocks do
  // not contend; issued after the block's last barrier, which would
  // otherwise wait for the atomic to complete
  if (MODE != kModeMoments && A.touched && tid == 0)
    atomicAdd(A.touched + (j & (kTouchedSlots - 1)), (unsigned long long)U);
}

// ------------------------------------------------------------------ column-sorted update

// The update of one block with its window transposed into columns, one per
// touched position.  A counting sort by slot in LDS (count with atomics,
// prefix in slot order, scatter) puts each window entry into its position's
// column as the key row << 16 | bf16 bits of V; each column (a few entries) is
// then sorted by row in place and summed by one thread in physical row order,
// z1 += beta1^r V and z2 += beta2^r V^2 in fp32: the same operations in the
// same order as adding the rows one at a time, with six barriers per block
// instead of one per row.  The parameters are then read and written in
// coalesced 16-byte groups: only 32-byte sectors holding a touched position,
// or every sector with decoupled decay.
//
// LDS (dynamic, CsuSmem): the bitmap and slot bases (W words each), the 2m
// decay factors, one word per slot (count, then column start / end, then the
// slot's update value) and one word per entry (first the staged raw window
// entries, then the column keys).  A thread holds at most kCsuPerThread
// entries and slots, so the block's m * k_b must not exceed
// kThreads * kCsuPerThread (the host checks it).
constexpr int kCsuPerThread = 12;

struct CsuSmem {
  uint32_t *bits, *wbase;
  float *beta;
  uint32_t *slot;   // [min(B_d, m * k_b)]
  uint32_t *col;    // [m * k_b]
  uint32_t *cnt;    // kWaves + 1 words (scans)
};

template <int CPT>
__device__ __forceinline__ CsuSmem csu_smem(const ApplyArgs &A, uint32_t *smem, uint32_t *cnt) {
  constexpr int W = CPT * kChunkSpan / 32;
  CsuSmem sm;
  sm.bits = smem;
  sm.wbase = smem + W;
  sm.beta = reinterpret_cast<float *>(smem + 2 * W);
  sm.slot = smem + 2 * W + 2 * A.m;
  sm.col = sm.slot + A.csu_slots;
  sm.cnt = cnt;
  return sm;
}

// Row of flat entry x = i * kb + q for x < 2^16: floor((x + 1/2) / kb) in
// fp32 is exact (the error of the product, below 2^-7 / kb, is far from the
// distance 1 / (2 kb) to an integer).
__device__ __forceinline__ int csu_row(int x, float inv_kb) {
  return (int)(((float)x + 0.5f) * inv_kb);
}


// MODE as apply_block (kModeSparse, kModeDense, kModeMoments).
// newrow (optional): window row t mod m of the block, already in LDS (the
// fused kernel's compressor wrote it there beside its global copy); that row
// is then copied from LDS instead of read from global memory.  pre_kb >= 0:
// the block's window offset and quota, already known (re-reading them from
// global memory would wait for all the vector memory in flight, the
// compressor's stores included).
// EARLY (dense mode): the block's 16-byte parameter groups are loaded before
// the column sums (their latency overlaps them; 4 words per load held
// meanwhile), else after them.  The sparse mode loads each touched parameter
// before the sums in either case, one word per slot.
// THL (fp32 parameters, 16-byte aligned, full block; sparse or dense mode):
// every 128-byte line of the block's parameters is read and written whole.
// The block's 16-byte groups are loaded into registers before the column
// sums (as EARLY); after them they pass through LDS in chunks of thl_n floats
// at thl (over the dead window entries): each chunk is written to LDS, the
// slot threads update their touched positions there (theta * decay -
// update), and the chunk goes back in coalesced 16-byte stores, the
// untouched positions scaled by the decay.  Whole-line write-back costs less
// HBM time than the dirty 32-byte sectors of a scattered one, even though it
// moves every byte.
template <int CPT, int MODE, bool ALIGNED, bool BF = false, bool EARLY = true, bool THL = false>
__device__ __forceinline__ void apply_block_csu(const ApplyArgs &A, int64_t j, int64_t out_row, const CsuSmem &sm,
                                                const uint32_t *newrow = nullptr, int64_t pre_off = 0,
                                                int pre_kb = -1, float *thl = nullptr) {
  static_assert(!THL || (!BF && ALIGNED && MODE != kModeMoments), "THL: fp32, aligned parameters, an update mode");
  constexpr int W = CPT * kChunkSpan / 32;           // bitmap words
  constexpr int WPT = (W + kThreads - 1) / kThreads; // words a thread owns
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  __builtin_assume(tid >= 0 && tid < kThreads);
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t s = j * (int64_t)A.B;
  const int L = (int)((A.d - s) < (int64_t)A.B ? (A.d - s) : (int64_t)A.B);
  const int64_t off = pre_kb >= 0 ? pre_off : A.off_tab[j];
  const int kb = pre_kb >= 0 ? pre_kb : (int)(A.off_tab[j + 1] - off);
  const int M = A.m;
  const int E = M * kb;
  const float inv_kb = kb > 0 ? 1.0f / (float)kb : 0.f;

  // ---------------- the block's m * k_b window entries into LDS (col), the
  // decay factors, a cleared bitmap
  for (int w = tid; w < W; w += kThreads) sm.bits[w] = 0u;
  stage_beta_rows(A, sm.beta, tid);
  for (int x0 = wv * 64; x0 < E; x0 += kThreads) {
    const int x = x0 + lane;
    if (x < E) {
      const int i = csu_row(x, inv_kb), q = x - i * kb;
      if (!newrow || i != A.tm)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(A.G + (int64_t)i * A.k + off + q),
                                         (lds_void_t *)(&sm.col[x0]), 4, 0, kCacheStream);
    }
  }
  if (newrow)
    for (int q = tid; q < kb; q += kThreads) sm.col[A.tm * kb + q] = newrow[q];
  wait_vm_all();
  __syncthreads();

  // ---------------- each thread's entries (x = tid + u * 512) into registers,
  // and the bitmap of the touched positions.  A zero value adds nothing
  // (unwritten rows are all zero); an index outside the block (only possible
  // in an imported state) is ignored.
  // (entries and slots per thread: nE = ceil(E / 512), uniform, so the
  // unrolled loops below skip their unused iterations with a scalar branch)
  const int nE = (E + kThreads - 1) / kThreads;
  uint32_t ent[kCsuPerThread];
#pragma unroll
  for (int u = 0; u < kCsuPerThread; ++u) {
    ent[u] = 0u;
    if (u < nE) {
      const int x = tid + u * kThreads;
      uint32_t e = (x < E) ? sm.col[x] : 0u;
      if (!(e & 0x7fff0000u) || (int)(e & 0xffffu) >= L) e = 0u;
      ent[u] = e;
      if (e) atomicOr(&sm.bits[(e & 0xffffu) >> 5], 1u << (e & 31u));
    }
  }
  __syncthreads();

  // ---------------- compact slots: slot(p) = number of touched positions below p
  uint32_t wc[WPT], mine = 0;
#pragma unroll
  for (int r = 0; r < WPT; ++r) {
    const int w = tid * WPT + r;
    wc[r] = (w < W) ? (uint32_t)__popc(sm.bits[w]) : 0u;
    mine += wc[r];
  }
  uint32_t cnt1[1] = {mine}, pos1[1], U;
  ordered_offsets<1>(cnt1, pos1, U, sm.cnt);
  {
    uint32_t b = pos1[0];
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = tid * WPT + r;
      if (w < W) sm.wbase[w] = b;
      b += wc[r];
    }
  }
  for (uint32_t x = (uint32_t)tid; x < U; x += kThreads) sm.slot[x] = 0u;
  __syncthreads();

  // ---------------- counting sort by slot: counts ...
  uint32_t sl[kCsuPerThread];
#pragma unroll
  for (int u = 0; u < kCsuPerThread; ++u) {
    sl[u] = 0xffffffffu;
    if (u < nE) {
      const uint32_t e = ent[u], I = e & 0xffffu;
      sl[u] = e ? sm.wbase[I >> 5] + (uint32_t)__popc(sm.bits[I >> 5] & ((1u << (I & 31u)) - 1u)) : 0xffffffffu;
      if (e) atomicAdd(&sm.slot[sl[u]], 1u);
    }
  }
  __syncthreads();
  // ... column starts, an exclusive prefix in slot order (a thread's words
  // hold a contiguous run of slots) ...
  const int w0 = tid * WPT;
  const uint32_t s_lo = (w0 < W) ? sm.wbase[w0] : U;
  const uint32_t s_hi = (w0 + WPT < W) ? sm.wbase[w0 + WPT] : U;
  uint32_t csum = 0;
  for (uint32_t x = s_lo; x < s_hi; ++x) csum += sm.slot[x];
  // (a slot word is then position << 16 | column start: the thread walks the
  // set bits of its words, which are its slots in order; E < 2^16)
  {
    uint32_t c1v[1] = {csum}, p1v[1], tot;
    ordered_offsets<1>(c1v, p1v, tot, sm.cnt);
    uint32_t run = p1v[0], x = s_lo;
#pragma unroll
    for (int r = 0; r < WPT; ++r) {
      const int w = w0 + r;
      uint32_t bits = (w < W) ? sm.bits[w] : 0u;
      while (bits) {
        const uint32_t c = sm.slot[x];
        sm.slot[x] = ((uint32_t)(w * 32 + __ffs(bits) - 1) << 16) | run;
        run += c;
        ++x;
        bits &= bits - 1u;
      }
    }
  }
  __syncthreads();
  // ... scatter of the keys (row << 16 | V bits): a slot's low half then ends
  // at the column's end
#pragma unroll
  for (int u = 0; u < kCsuPerThread; ++u) {
    if (u < nE && ent[u]) {
      const uint32_t p = atomicAdd(&sm.slot[sl[u]], 1u) & 0xffffu;
      sm.col[p] = ((uint32_t)csu_row(tid + u * kThreads, inv_kb) << 16) | (ent[u] >> 16);
    }
  }
  __syncthreads();

  // ---------------- dense mode: the parameters' loads, all issued at once
  // (before the column sums with EARLY, so that their latency overlaps them).
  // Consecutive threads take consecutive 16-byte groups (4 fp32 or 8 bf16
  // parameters): every access is coalesced across the wave.
  constexpr int G = BF ? 8 : 4;                      // parameters per 16-byte group
  constexpr int NG = CPT * kChunkSpan / G;           // groups per block
  constexpr int NIT = NG / kThreads;                 // groups per thread
  // every group whole and aligned (uniform over the block): 16-byte loads and
  // stores; otherwise element by element at the end
  const bool vec_all = ALIGNED && (L % G) == 0;
  u32x4 raw[(MODE == kModeDense || THL) ? NIT : 1];
  auto issue_loads = [&]() {
    if (MODE == kModeDense || THL) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i0 = (it * kThreads + tid) * G;
        raw[it] = u32x4{0u, 0u, 0u, 0u};
        if (vec_all && i0 < L)
          raw[it] = BF ? *reinterpret_cast<const u32x4 *>(A.theta16 + s + i0)
                       : *reinterpret_cast<const u32x4 *>(A.theta + s + i0);
      }
    }
  };
  if (EARLY || THL) issue_loads();

  // ---------------- each slot's column: sorted by row, summed in row order
  // (slots tid, tid + 512, ...).  Sparse mode: the thread that sums a slot
  // updates its parameter, whose load it issued first; every lane loads
  // (lanes past the last slot re-load its parameter) and every loaded value
  // is used, or the compiler would wait for all vector memory (in the fused
  // kernel, the compressor's stores included).  Dense mode: the update value
  // replaces the slot word, so each slot's column start and end are read
  // first, before a barrier.
  const int nU = (int)((U + kThreads - 1) / kThreads);   // slots per thread, uniform
  constexpr bool kDenseSlots = MODE == kModeDense && !THL;   // update values replace the slot words
  constexpr bool kGather = MODE == kModeSparse && !THL;      // touched parameters gathered by slot
  uint32_t cst[kDenseSlots ? kCsuPerThread : 1], cen[kDenseSlots ? kCsuPerThread : 1];
  float thv[kGather ? kCsuPerThread : 1];
  float thu[THL ? kCsuPerThread : 1];        // THL: each slot's update value and position
  uint32_t thp[THL ? kCsuPerThread : 1];
  if (kDenseSlots) {
#pragma unroll
    for (int u = 0; u < kCsuPerThread; ++u) {
      cst[u] = cen[u] = 0u;
      if (u < nU) {
        const uint32_t x = (uint32_t)tid + (uint32_t)(u * kThreads);
        cst[u] = (x < U && x > 0) ? sm.slot[x - 1] & 0xffffu : 0u;
        cen[u] = (x < U) ? sm.slot[x] & 0xffffu : 0u;
      }
    }
    __syncthreads();
  } else if (kGather) {
    if (U == 0) return;
    // (all of them, unconditionally: a scalar branch between a load and its
    // use makes the compiler wait for all vector memory there)
#pragma unroll
    for (int u = 0; u < kCsuPerThread; ++u) {
      const uint32_t x = min((uint32_t)tid + (uint32_t)(u * kThreads), U - 1u);
      thv[u] = ld_param<BF>(A, s + (sm.slot[x] >> 16));
    }
  }
#pragma unroll
  for (int u = 0; u < kCsuPerThread; ++u) {
    const uint32_t x = (uint32_t)tid + (uint32_t)(u * kThreads);
    if (THL) {
      thu[u] = 0.f;
      thp[u] = 0xffffffffu;
    }
    if (kGather || u < nU) {
      float th = 0.f;
      if (kGather) {
        th = thv[u];
        asm volatile("" ::"v"(th));   // the wait for the load, on every path
      }
      if (x < U) {
        const uint32_t sx = sm.slot[x];
        const uint32_t c0 = kDenseSlots ? cst[u] : (x > 0 ? sm.slot[x - 1] & 0xffffu : 0u);
        const uint32_t c1 = kDenseSlots ? cen[u] : sx & 0xffffu;
        float z1 = 0.f, z2 = 0.f;
        auto add = [&](uint32_t key) {   // the factors of the key's row (staged by row)
          const int row = (int)(key >> 16);
          const float V = bf16_bits_to_f32(key & 0xffffu);
          z1 = z1 + decay_factor(sm.beta, row) * V;
          z2 = z2 + decay_factor(sm.beta, M + row) * (V * V);
        };
        if (c1 - c0 <= 3u) {
          // one to three keys (almost every column): a three-key sorting
          // network in registers; absent keys are all ones, above every key
          // (rows < 65535) and never added
          const uint32_t n = c1 - c0;
          const uint32_t k0 = sm.col[c0];
          const uint32_t k1 = n >= 2u ? sm.col[c0 + 1] : 0xffffffffu;
          const uint32_t k2 = n >= 3u ? sm.col[c0 + 2] : 0xffffffffu;
          const uint32_t a = min(k0, k1), b = max(k0, k1);
          const uint32_t t = max(a, k2);
          add(min(a, k2));
          if (n >= 2u) add(min(b, t));
          if (n >= 3u) add(max(b, t));
        } else {
          for (uint32_t a = c0 + 1; a < c1; ++a) {   // insertion sort of a few keys
            const uint32_t key = sm.col[a];
            uint32_t b = a;
            while (b > c0 && sm.col[b - 1] > key) {
              sm.col[b] = sm.col[b - 1];
              --b;
            }
            sm.col[b] = key;
          }
          for (uint32_t a = c0; a < c1; ++a) add(sm.col[a]);
        }
        const float mh = A.c1 * z1;
        const float vh = A.c2 * z2;
        if (THL) {
          thu[u] = A.lr * (mh / (sqrt_rn(vh) + A.eps));
          thp[u] = sx >> 16;
        } else if (MODE == kModeMoments) {
          const int p = (int)(sx >> 16);
          A.mhat[out_row * A.B + p] = mh;
          A.vhat[out_row * A.B + p] = vh;
        } else if (MODE == kModeSparse) {
          st_param<BF>(A, s + (sx >> 16), th - A.lr * (mh / (sqrt_rn(vh) + A.eps)));
        } else {
          sm.slot[x] = f2u(A.lr * (mh / (sqrt_rn(vh) + A.eps)));
        }
      }
    }
  }
  if (THL) {
    // ---------------- the parameters through LDS, chunk by chunk: thread t's
    // groups it (elements 4 (it * 512 + t) ..) go to the chunk's LDS; after
    // a barrier the slot threads update their positions of the chunk; after
    // another the chunk is stored.  (it is unrolled: raw[] is indexed by
    // constants; a chunk holds itc of each thread's groups.)
    // (THL runs for full, aligned blocks only, so vec_all holds and every
    // group was loaded; the host sizes thl_n as a power-of-two part of the
    // block of at least G * kThreads elements, so itc >= 1)
    const bool decays = A.decay != 1.0f;
    const int cn = A.thl_n;
    const int itc = cn / (G * kThreads);   // a power of two
    u32x4 *R4 = reinterpret_cast<u32x4 *>(thl);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int li = it & (itc - 1);
      if (li == 0) __syncthreads();   // the LDS chunk is free: entries summed, previous chunk stored
      R4[li * kThreads + tid] = raw[it];
      if (li == itc - 1) {
        const int c0 = (it - li) * G * kThreads;   // the chunk's first element
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kCsuPerThread; ++u) {
          if (u < nU) {
            const uint32_t q = thp[u] - (uint32_t)c0;
            if (q < (uint32_t)cn) {
              float th = thl[q];
              if (decays) th = th * A.decay;
              thl[q] = th - thu[u];
            }
          }
        }
        __syncthreads();
        for (int r = 0; r < itc; ++r) {
          const int q = r * kThreads + tid;
          u32x4 v = R4[q];
          if (decays) {
            const int i0 = c0 + G * q;
            const uint32_t gb = (sm.bits[i0 >> 5] >> (i0 & 31)) & 15u;   // touched ones are already done
            if (!(gb & 1u)) v.x = f2u(u2f(v.x) * A.decay);
            if (!(gb & 2u)) v.y = f2u(u2f(v.y) * A.decay);
            if (!(gb & 4u)) v.z = f2u(u2f(v.z) * A.decay);
            if (!(gb & 8u)) v.w = f2u(u2f(v.w) * A.decay);
          }
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(A.theta + s + c0) + q);
        }
      }
    }
    if (A.touched && tid == 0) atomicAdd(A.touched + (j & (kTouchedSlots - 1)), (unsigned long long)U);
    return;
  }
  if (MODE == kModeMoments) {
    // positions without an entry: 0
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int i = c * kChunkSpan + tid * kChunk + e;
        if (i < L && !((sm.bits[i >> 5] >> (i & 31)) & 1u)) {
          A.mhat[out_row * A.B + i] = 0.f;
          A.vhat[out_row * A.B + i] = 0.f;
        }
      }
    return;
  }
  if (MODE == kModeSparse) {
    if (A.touched && tid == 0) atomicAdd(A.touched + (j & (kTouchedSlots - 1)), (unsigned long long)U);
    return;
  }
  __syncthreads();

  // ---------------- dense mode: theta = theta * decay - update on touched positions
  if (!EARLY) issue_loads();
  // (without decay, the factor 1 is not applied: the stored value is the
  // loaded one, as in the sparse mode)
  const bool decays = A.decay != 1.0f;
  if (vec_all) {
    // no loads here: the stores need no waits
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = (it * kThreads + tid) * G;
      if (i0 >= L) continue;
      const int w = i0 >> 5;
      const uint32_t word = sm.bits[w];
      const uint32_t gb = (word >> (i0 & 31)) & ((1u << G) - 1u);   // this group's touched bits
      const uint32_t base = sm.wbase[w] + (uint32_t)__popc(word & ((1u << (i0 & 31)) - 1u));
      float th[G];
      const uint32_t vv[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
#pragma unroll
      for (int e = 0; e < G; ++e)
        th[e] = BF ? ((e & 1) ? u2f(vv[e >> 1] & 0xffff0000u) : u2f(vv[e >> 1] << 16)) : u2f(vv[e]);
#pragma unroll
      for (int e = 0; e < G; ++e) {
        if (decays) th[e] = th[e] * A.decay;
        if ((gb >> e) & 1u) th[e] = th[e] - u2f(sm.slot[base + (uint32_t)__popc(gb & ((1u << e) - 1u))]);
      }
      if (BF) {
        u32x4 v;
        v.x = f32_to_bf16_rne(th[0]) | (f32_to_bf16_rne(th[1]) << 16);
        v.y = f32_to_bf16_rne(th[2]) | (f32_to_bf16_rne(th[3]) << 16);
        v.z = f32_to_bf16_rne(th[4]) | (f32_to_bf16_rne(th[5]) << 16);
        v.w = f32_to_bf16_rne(th[6]) | (f32_to_bf16_rne(th[7]) << 16);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(A.theta16 + s + i0));
      } else {
        const u32x4 v0 = {f2u(th[0]), f2u(th[1]), f2u(th[2]), f2u(th[3])};
        __builtin_nontemporal_store(v0, reinterpret_cast<u32x4 *>(A.theta + s + i0));
      }
    }
  } else {
    // unaligned parameters or a partial group: element by element
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = (it * kThreads + tid) * G;
      if (i0 >= L) continue;
      const int w = i0 >> 5;
      const uint32_t word = sm.bits[w];
      const uint32_t gb = (word >> (i0 & 31)) & ((1u << G) - 1u);
      const uint32_t base = sm.wbase[w] + (uint32_t)__popc(word & ((1u << (i0 & 31)) - 1u));
#pragma unroll
      for (int e = 0; e < G; ++e) {
        if (i0 + e < L) {
          float th = ld_param<BF>(A, s + i0 + e) * A.decay;
          if ((gb >> e) & 1u) th = th - u2f(sm.slot[base + (uint32_t)__popc(gb & ((1u << e) - 1u))]);
          st_param<BF>(A, s + i0 + e, th);
        }
      }
    }
  }
  if (A.touched && tid == 0) atomicAdd(A.touched + (j & (kTouchedSlots - 1)), (unsigned long long)U);
}

// One workgroup per block (blocks first_block .. first_block + grid - 1, or
// the listed ones in MODE 2), column-sorted update.
template <int CPT, int MODE, bool ALIGNED, bool BF = false>
__global__ __launch_bounds__(kThreads) void apply_csu_kernel(ApplyArgs A) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_cnt[kWaves + 1];
  const int64_t j = (MODE == kModeMoments) ? A.blocks[blockIdx.x]
                                           : A.first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  apply_block_csu<CPT, MODE, ALIGNED, BF>(A, j, (int64_t)blockIdx.x, csu_smem<CPT>(A, smem, s_cnt));
}

// The column-sorted update of the blocks in the device list A.blocks[0 .. *A.n_list).
template <int CPT, bool BF = false, int MODE = kModeSparse>
__global__ __launch_bounds__(kThreads) void apply_csu_list_kernel(ApplyArgs A) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_cnt[kWaves + 1];
  const unsigned int n = *A.n_list;
  for (unsigned int q = blockIdx.x; q < n; q += gridDim.x) {
    apply_block_csu<CPT, MODE, false, BF>(A, A.blocks[q], 0, csu_smem<CPT>(A, smem, s_cnt));
    __syncthreads();
  }
}

// LDS of the standalone update: dynamic, laid out as in ApplySmem.
template <int CPT>
__device__ __forceinline__ ApplySmem apply_smem(const ApplyArgs &A, uint32_t *smem, uint32_t *cnt, int64_t j) {
  constexpr int W = CPT * kChunkSpan / 32;
  ApplySmem sm;
  sm.bits = smem;
  sm.wbase = smem + W;
  sm.beta = reinterpret_cast<float *>(smem + 2 * W);
  sm.ent = smem + 2 * W + 2 * A.m;
  sm.z1 = reinterpret_cast<float *>(sm.ent + A.ent_cap);
  sm.z2 = sm.z1 + A.cap;
  sm.pos = reinterpret_cast<uint16_t *>(sm.z2 + A.cap);
  sm.cnt = cnt;
  sm.cap = A.cap;
  sm.ent_stride = 0;
  sm.in_lds = A.m * (A.off_tab[j + 1] - A.off_tab[j]) <= A.ent_cap;
  return sm;
}

// One workgroup per block: blocks first_block .. first_block + grid - 1
// (MODE 0, 1) or the listed blocks (MODE 2).
template <int CPT, int MODE, bool ALIGNED, bool BF = false>
__global__ __launch_bounds__(kThreads) void apply_kernel(ApplyArgs A) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_cnt[kWaves + 1];
  const int64_t j = (MODE == kModeMoments) ? A.blocks[blockIdx.x]
                                           : A.first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  apply_block<CPT, MODE, ALIGNED, false, BF>(A, j, (int64_t)blockIdx.x, apply_smem<CPT>(A, smem, s_cnt, j));
}

// The update (MODE 0 or 1) of the blocks in the device list
// A.blocks[0 .. *A.n_list).
template <int CPT, bool BF = false, int MODE = kModeSparse>
__global__ __launch_bounds__(kThreads) void apply_list_kernel(ApplyArgs A) {
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t s_cnt[kWaves + 1];
  const unsigned int n = *A.n_list;
  for (unsigned int q = blockIdx.x; q < n; q += gridDim.x) {
    const int64_t j = A.blocks[q];
    apply_block<CPT, MODE, false, false, BF>(A, j, 0, apply_smem<CPT>(A, smem, s_cnt, j));
    __syncthreads();
  }
}

// ------------------------------------------------------------------ fused step

// Window entries the fused kernel holds in LDS: m rows of k_b entries, each
// row padded to whole waves (64 entries).  Sized so that three workgroups of
// the four-chunk kernel fit the 160 KiB of LDS of a CU.
constexpr int kFusedEnt = 1984;

// The whole step of one full, aligned block in one workgroup: compress (rows
// a1-a5) and then, with the block's window in LDS, the sparse update (a6-a7).
// The window rows the step does not write are copied to LDS by LDS-DMA while
// the block's gradients and codes are staged; the compressor's new row goes to
// LDS beside its global copy.  Co-resident workgroups are in different
// phases, so the VALU-bound compressor and the memory-bound update share each
// CU.  A block the compressor defers is left entirely (compress and update)
// to compress_deferred_kernel and apply_list_kernel.  QMODE kQGlobal1: the
// global quantizer's first pass (selection, window row, the block's min / max
// and cut) with the update; the codes are left to the second pass.  MODE:
// the update's mode (kModeDense with decoupled decay), PAL: 16-byte aligned
// parameters (required by the dense mode here; in the sparse mode only the
// column-sorted update uses it).
template <int CPT, bool EF, bool BF = false, int QMODE = kQBlock, int MODE = kModeSparse, bool PAL = false>
__global__ __launch_bounds__(kThreads, MA_FULL_WAVES) void step_full_kernel(CompressArgs C, ApplyArgs A,
                                                                             int64_t first_block) {
  static_assert(QMODE == kQBlock || (QMODE == kQGlobal1 && EF), "the fused kernel runs a step or a first pass");
  static_assert(MODE == kModeSparse || (MODE == kModeDense && PAL), "dense updates in the fused kernel are aligned");
  __shared__ CompressSmem<CPT> sm;
  __shared__ FullBlockStage<CPT> st;
  __shared__ uint32_t ent[kFusedEnt];
  __shared__ float s_beta[kFusedBeta];
  static_assert(2 * (kFusedEnt / 64) <= kFusedBeta, "the fused kernel's decay factors fit");
  static_assert(sizeof(FullBlockStage<CPT>) >= 4u * (CPT * kChunkSpan / 2) + 8u * (CPT * kChunkSpan / 32),
                "random words, bitmap and slot bases fit the staging space");
  const int64_t j = first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  FullBlockInputs<CPT> in;
  stage_full_block<CPT, EF>(C, j, st, in);

  // window rows other than row t mod m, into ent[i * es ..] (whole waves; the
  // lanes past k_b re-read the segment's last entry into the row's padding);
  // streaming loads, measured slightly faster
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int es = (in.kb + 63) & ~63;
  if (in.kb > 0) {
    const int wpr = es >> 6;   // wave loads per row
    for (int w = tid >> 6; w < A.m * wpr; w += kWaves) {
      const int i = w / wpr, q0 = (w - i * wpr) << 6;
      if (i == A.tm) continue;
      const int q = min(q0 + (tid & 63), in.kb - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(A.G + (int64_t)i * A.k + in.off + q),
                                       (lds_void_t *)(&ent[i * es + q0]), 4, 0, kCacheStream);
    }
  }
  // the decay factors, waited for with the staged inputs
  stage_beta(A, s_beta, tid);
  // LDS of the staged inputs, once they are consumed: the quantizer's random
  // words (L/2 words), then the bitmap and slot bases; the update's per-slot
  // arrays later reuse the random words' space
  constexpr int W = CPT * kChunkSpan / 32;
  uint32_t *st_words = reinterpret_cast<uint32_t *>(&st);
  FusedBits fbits;
  // (the bitmap's words are the staged codes, from st.ef[0][0] on: the
  // compressor clears each once its only reader has read it)
  fbits.bits = &st.ef[0][0];
  fbits.ent = ent;
  fbits.es = es;
  fbits.M = A.m;
  fbits.tm = A.tm;
  const bool done = compress_block<CPT, true, true, EF, true, QMODE>(C, sm, j, j * (int64_t)C.B, CPT * kChunkSpan, in.off,
                                                              in.kb, &st, &in, &ent[A.tm * es], st_words, &fbits);
  if (!done) return;
  __syncthreads();

  ApplySmem as;
  as.bits = fbits.bits;
  as.wbase = as.bits + W;
  as.ent = ent;
  as.z1 = reinterpret_cast<float *>(st_words);
  as.cap = (int)((4u * (CPT * kChunkSpan / 2)) / 10u);
  as.z2 = as.z1 + as.cap;
  as.pos = reinterpret_cast<uint16_t *>(as.z2 + as.cap);
  as.cnt = sm.cnt;
  as.ent_stride = es;
  as.in_lds = true;
  as.beta = s_beta;
  as.off = in.off;
  as.kb = in.kb;
  apply_block<CPT, MODE, PAL, true, BF>(A, j, 0, as);
}

// The whole step of one full, aligned block in one workgroup with the
// column-sorted update: the compressor (rows a1-a5), then the update (a6-a7)
// reading the block's m window rows after the compressor has finished.  One
// static LDS buffer of kFusedCsuWords (a third of a CU's LDS: three
// workgroups per CU) serves both phases, the compressor's CompressSmem and
// staging first and the update's CsuSmem after (A.fused_union_words words);
// the new window row is kept apart, behind it, where the compressor writes it
// beside its global copy.  Co-resident workgroups are in different phases, so
// the arithmetic-bound compressor and the memory-bound update share each CU.
// Blocks the compressor defers are left to compress_deferred_kernel and
// apply_csu_list_kernel, as in step_full_kernel.  THL: the update writes every
// parameter line whole, through an LDS chunk at A.thl_off words (behind the
// update's slot words, over its dead window entries; apply_block_csu).
// (A static buffer: with a dynamic one the compressor's addresses are formed
// at run time and its registers spill.)  Three workgroups fit a CU's 160 KiB
// when each takes at most 53,760 bytes (LDS is allocated in 1,280-byte
// granules), the scan words included.
constexpr int kFusedCsuWords = (53760 - 64) / 4;

template <int CPT, bool EF, bool BF = false, int QMODE = kQBlock, int MODE = kModeSparse, bool PAL = false,
          bool THL = false>
__global__ __launch_bounds__(kThreads, MA_FULL_WAVES) void step_csu_kernel(CompressArgs C, ApplyArgs A,
                                                                            int64_t first_block) {
  static_assert(QMODE == kQBlock || (QMODE == kQGlobal1 && EF), "the fused kernel runs a step or a first pass");
  static_assert(MODE == kModeSparse || (MODE == kModeDense && PAL), "dense updates in the fused kernel are aligned");
  static_assert(sizeof(FullBlockStage<CPT>) >= 4u * (CPT * kChunkSpan / 2), "the random words fit the staging space");
  __shared__ __attribute__((aligned(16))) uint32_t lds[kFusedCsuWords];
  __shared__ uint32_t s_cnt[kWaves + 1];
  constexpr int kSmWords = (int)((sizeof(CompressSmem<CPT>) + 15) / 16 * 4);
  CompressSmem<CPT> &sm = *reinterpret_cast<CompressSmem<CPT> *>(lds);
  FullBlockStage<CPT> *st = reinterpret_cast<FullBlockStage<CPT> *>(lds + kSmWords);
  uint32_t *newrow = lds + A.fused_union_words;
  const int64_t j = first_block + xcd_block((int64_t)blockIdx.x, (int64_t)gridDim.x);
  FullBlockInputs<CPT> in;
  stage_full_block<CPT, EF>(C, j, *st, in);
  const bool done = compress_block<CPT, true, true, EF, true, QMODE>(C, sm, j, j * (int64_t)C.B, CPT * kChunkSpan,
                                                                   in.off, in.kb, st, &in, newrow,
                                                                   reinterpret_cast<uint32_t *>(st), nullptr);
  if (!done) return;
  __syncthreads();
  apply_block_csu<CPT, MODE, PAL, BF, MODE == kModeDense, THL>(A, j, 0, csu_smem<CPT>(A, lds, s_cnt), newrow, in.off,
                                                                in.kb, reinterpret_cast<float *>(lds + A.thl_off));
}

}  // namespace microadam
