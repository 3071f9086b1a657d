/*
 * MicroAdam CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C implementation of one MicroAdam optimizer
 * step, written from the page "MicroAdam (Sparse-Gradient Adaptive
 * Optimization with Quantized Error Feedback)".  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant generator with the GPU library; the two are
 * compared element by element.
 *
 * Arithmetic: every floating-point value the step stores (EF statistics, the
 * accumulator, the moments, the parameters) is IEEE fp32, each operation
 * rounded to nearest even, no contraction (the file is built with
 * -ffp-contract=off); the one intended fused operation is an explicit fmaf.
 * Host constants (beta powers, bias corrections, decay) are computed in double
 * and rounded once to fp32.  Integer decisions (the Top-k set, the 4-bit codes)
 * are taken in that fp32 arithmetic.
 *
 * Parity status of each function is stated next to it; "pinned" means a CPU
 * test checks it against something other than itself (a library routine,
 * published known-answer vectors, a closed form, an invariant, brute force).
 */
#ifndef MICROADAM_ORACLE_H
#define MICROADAM_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_FLAG_NO_EF 1u         /* a_t = g_t: the stored error is neither read nor rewritten */
#define ORC_FLAG_GLOBAL_QUANT 2u  /* one (delta, Delta) pair over all d (the literal scalar form) */

typedef struct {
    int64_t d;        /* flat parameter count */
    int32_t B;        /* block length B_d, 1 <= B < 2^15 - 1 */
    int32_t m;        /* window rows */
    int64_t k;        /* total Top-k budget per step, 0 <= k <= d */
    int32_t b;        /* quantizer bits; only 4 is defined */
    float beta1, beta2, eps, lr, wd;
    uint64_t seed;
    uint32_t flags;
} orc_cfg;

/* ---- elementary pieces (pinned individually) ---- */
uint16_t orc_bf16_rne(float x);            /* pinned: torch CPU float->bfloat16 */
float    orc_bf16_to_f32(uint16_t h);      /* pinned: torch CPU bfloat16->float */
void     orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]); /* pinned: Random123 KAT */
uint32_t orc_pcg_hash(uint32_t x);         /* pinned: bijection + uniformity (statistical) */
uint32_t orc_block_key(uint64_t seed, int64_t t, int64_t j);
uint32_t orc_xi16(uint64_t seed, int64_t t, int64_t j, int64_t local);

int64_t  orc_floor_mul_div(int64_t k, int64_t x, int64_t d);   /* floor(k*x/d), exact */
void     orc_block_range(const orc_cfg *c, int64_t j, int64_t *start, int64_t *len);
void     orc_block_quota(const orc_cfg *c, int64_t j, int64_t *off, int64_t *kb);
int64_t  orc_num_blocks(const orc_cfg *c);

void     orc_step_constants(const orc_cfg *c, int64_t t, float *fac1, float *fac2,
                            float *c1, float *c2, float *decay);

/* Top-k of |a| over n values: writes the kb selected positions in ascending
 * order.  Order: key = bits(|a|) descending, ties to the lower position. */
void     orc_topk(const float *a, int64_t n, int64_t kb, int32_t *sel_out);

/* 4-bit stochastic quantizer of one group (a block, or all of d) */
void     orc_quant_group(const float *x, int64_t n, uint64_t seed, int64_t t, int64_t j,
                         int64_t local0, float lo, float hi, uint8_t *codes_out);
void     orc_group_minmax(const float *x, int64_t n, float *lo, float *hi);
/* a range hi - lo that is not finite resets the pair to (0, 0) */
void     orc_range_reset(float *lo, float *hi);
void     orc_dequant_group(const uint8_t *codes, int64_t n, float lo, float hi, float *out);

/* nibble access: element i of a packed array lives in byte i/2, low nibble for even i */
uint8_t  orc_get_nibble(const uint8_t *bytes, int64_t i);
void     orc_set_nibble(uint8_t *bytes, int64_t i, uint8_t v);

/* ---- one block of one step ----
 * theta, g: the block's L parameters and gradients.
 * ef: packed codes; element i of the block is nibble (nib0 + i) of ef.
 * stats: {delta, Delta} of the block.
 * gseg: this block's segment of each window row, row i at gseg + i*gstride,
 *       k_b entries each; entry = index | bf16(V) << 16.
 * mhat, vhat: optional (may be NULL) per-position moments, length L.
 * Returns 0, or a negative value for an unsupported configuration. */
int orc_block_step(const orc_cfg *c, int64_t t, int64_t j,
                   float *theta, const uint16_t *g,
                   uint8_t *ef, int64_t nib0, float *stats,
                   uint32_t *gseg, int64_t gstride,
                   float *mhat, float *vhat);

/* ---- one full step over all d ----
 * ef: ceil(d/2) bytes, stats: 2*n_b floats (or 2 with ORC_FLAG_GLOBAL_QUANT),
 * G: m*k entries.  t is the new step number (1-based). */
int orc_step(const orc_cfg *c, int64_t t, float *theta, const uint16_t *g,
             uint8_t *ef, float *stats, uint32_t *G, float *mhat, float *vhat);

/* ---- comparison baseline: fp32 AdamW (the second paragraph's 8d-byte
 * optimizer), one step t (1-based) over n elements, in place.  Per element,
 * each operation rounded once in fp32:
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *   theta = theta*decay - lr*((m*r1) / (sqrtf(v*r2) + eps))
 * with g the bf16 gradient widened, (1-b), decay = 1 - lr*wd and the bias
 * factors r = 1/(1 - b^t) computed in double and rounded to fp32. */
void orc_adamw_step(int64_t n, int64_t t, float b1, float b2, float eps, float lr, float wd,
                    float *theta, const uint16_t *g, float *m, float *v);

/* ---- comparison baseline: 8-bit block-quantized AdamW (the second
 * paragraph's 2d-byte optimizer).  Reading (the page fixes no 8-bit scheme):
 * blocks of ORC_Q8_BLOCK elements, each with two fp32 scales; m as int8 codes
 * c = rint(m * (127/sm)) with sm = max|m| of the block, m~ = c * (sm/127); v as
 * uint8 codes of sqrt(v): c = rint(sqrt(v) * (255/sr)) with sr = max sqrt(v),
 * v~ = (c * (sr/255))^2.  One step: dequantize, the AdamW recurrence and
 * parameter update of orc_adamw_step on the dequantized moments, then
 * requantize the new moments with the block's new scales (a zero block gets
 * scale 0 and codes 0).  cm: int8[n], cv: uint8[n], sm, sr: float[ceil(n/B)]. */
#define ORC_Q8_BLOCK 256
void orc_adamw8_step(int64_t n, int64_t t, float b1, float b2, float eps, float lr, float wd,
                     float *theta, const uint16_t *g, int8_t *cm, uint8_t *cv, float *sm, float *sr);

/* array helpers */
void orc_bf16_rne_array(const float *x, int64_t n, uint16_t *out);
void orc_pcg_hash_array(const uint32_t *x, int64_t n, uint32_t *out);
void orc_xi16_array(uint64_t seed, int64_t t, int64_t j, int64_t local0, int64_t n, uint32_t *out);

/* state size the memory paragraph counts: 0.5d (rounded up to bytes) + 4mk */
uint64_t orc_state_bytes(const orc_cfg *c);

#ifdef __cplusplus
}
#endif
#endif
