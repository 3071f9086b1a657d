/*
 * MicroAdam CPU oracle -- TEST INFRASTRUCTURE ONLY (see microadam_oracle.h).
 *
 * Source of the method: the page "MicroAdam (Sparse-Gradient Adaptive
 * Optimization with Quantized Error Feedback)":
 *   - first paragraph (the per-step algorithm): a_t = g_t + Q^{-1}(e_t, delta_t,
 *     Delta_t); (I_t, V_t) = T_k(|a_t|) with block-relative int16 indices in
 *     blocks B_d < 2^15 - 1; zero those entries of a_t; e_{t+1} = Q(a_t,
 *     delta_{t+1}, Delta_{t+1}) with b = 4 bits; (I_t, V_t) goes to row t mod m
 *     of the circular window G; m_hat = AdamStats(beta1, G), v_hat =
 *     AdamStats(beta2, G^2) by the unrolled decay z[I_i] += beta^r V_i;
 *   - second paragraph (memory): 0.5d bytes of codes + 4mk bytes of window;
 *   - third paragraph (theory): Q is unbiased (Lemma 1 gives its omega);
 *   - last paragraph: the update u_t is sparse.
 * Readings of what the page leaves open are stated where they are used.
 *
 * Built with: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math (see build.py).
 */
#include "microadam_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bfloat16                                                             */
/* ------------------------------------------------------------------ */

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bfloat16 keeps the top 16 bits of an fp32; round to nearest, ties to even.
 * (The page stores window values as bfloat16.)  NaN stays a quiet NaN. */
uint16_t orc_bf16_rne(float x)
{
    uint32_t u = f2u(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

float orc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* ------------------------------------------------------------------ */
/* Counter-based random numbers (keyed on seed, step, element)          */
/* ------------------------------------------------------------------ */

/* Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): each round multiplies
 * words 0 and 2 by two fixed odd constants, and the new state is built from the
 * high and low product halves xor-ed with the other two words and the key; the
 * key is bumped by two Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The "pcg_hash" of Jarzynski and Olano, "Hash Functions for GPU Rendering"
 * (JCGT 2020): one step of the 32-bit PCG linear congruential generator
 * followed by PCG's RXS-M-XS output permutation. */
uint32_t orc_pcg_hash(uint32_t x)
{
    uint32_t state = x * 747796405u + 2891336453u;
    uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

/* Per-(seed, step, block) key: the first Philox output word for counter
 * (j low, j high, t low, t high) under key (seed low, seed high). */
uint32_t orc_block_key(uint64_t seed, int64_t t, int64_t j)
{
    uint32_t ctr[4] = { (uint32_t)(uint64_t)j, (uint32_t)((uint64_t)j >> 32),
                        (uint32_t)(uint64_t)t, (uint32_t)((uint64_t)t >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[0];
}

/* 16-bit uniform for element `local` of block j at step t: the low half of
 * pcg_hash(key + local/2) for even local, the high half for odd. */
uint32_t orc_xi16(uint64_t seed, int64_t t, int64_t j, int64_t local)
{
    uint32_t h = orc_pcg_hash(orc_block_key(seed, t, j) + (uint32_t)(local >> 1));
    return (local & 1) ? (h >> 16) : (h & 0xffffu);
}

/* ------------------------------------------------------------------ */
/* Blocks and per-block Top-k quota                                     */
/* ------------------------------------------------------------------ */

int64_t orc_floor_mul_div(int64_t k, int64_t x, int64_t d)
{
    unsigned __int128 p = (unsigned __int128)(uint64_t)k * (unsigned __int128)(uint64_t)x;
    return (int64_t)(p / (unsigned __int128)(uint64_t)d);
}

int64_t orc_num_blocks(const orc_cfg *c) { return (c->d + c->B - 1) / c->B; }

void orc_block_range(const orc_cfg *c, int64_t j, int64_t *start, int64_t *len)
{
    int64_t s = j * (int64_t)c->B;
    int64_t e = s + c->B;
    if (e > c->d) e = c->d;
    *start = s;
    *len = e - s;
}

/* The page fixes k = d/100 over all of d and block-relative indices, but not
 * how k is split over blocks.  Reading: block j = [s, e) gets
 * floor(k*e/d) - floor(k*s/d) entries, placed at offset floor(k*s/d) of every
 * window row.  The quotas add up to exactly k, so a row holds k entries. */
void orc_block_quota(const orc_cfg *c, int64_t j, int64_t *off, int64_t *kb)
{
    int64_t s, len;
    orc_block_range(c, j, &s, &len);
    int64_t lo = orc_floor_mul_div(c->k, s, c->d);
    int64_t hi = orc_floor_mul_div(c->k, s + len, c->d);
    *off = lo;
    *kb = hi - lo;
}

/* ------------------------------------------------------------------ */
/* Step constants                                                       */
/* ------------------------------------------------------------------ */

/* Physical window row i was written at the step whose number is congruent to
 * i mod m, so at step t its age is r = (t - i) mod m and its weight beta^r.
 * The page leaves the normalisation of AdamStats open; reading: Adam's bias
 * correction c = (1 - beta)/(1 - beta^t), so that t = 1 gives m_hat = V and
 * v_hat = V^2.  All computed in double from the fp32 hyperparameters, then
 * rounded once to fp32. */
void orc_step_constants(const orc_cfg *c, int64_t t, float *fac1, float *fac2,
                        float *c1, float *c2, float *decay)
{
    double b1 = (double)c->beta1, b2 = (double)c->beta2;
    int64_t tm = t % c->m;
    for (int32_t i = 0; i < c->m; ++i) {
        int64_t r = (tm - i + c->m) % c->m;
        fac1[i] = (float)pow(b1, (double)r);
        fac2[i] = (float)pow(b2, (double)r);
    }
    *c1 = (float)((1.0 - b1) / (1.0 - pow(b1, (double)t)));
    *c2 = (float)((1.0 - b2) / (1.0 - pow(b2, (double)t)));
    *decay = (float)(1.0 - (double)c->lr * (double)c->wd);
}

/* ------------------------------------------------------------------ */
/* Top-k by magnitude                                                   */
/* ------------------------------------------------------------------ */

typedef struct { uint32_t key; int32_t pos; } orc_kp;

static int cmp_key_desc_pos_asc(const void *pa, const void *pb)
{
    const orc_kp *a = (const orc_kp *)pa, *b = (const orc_kp *)pb;
    if (a->key != b->key) return a->key > b->key ? -1 : 1;
    return a->pos < b->pos ? -1 : (a->pos > b->pos ? 1 : 0);
}

static int cmp_int32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* T_k(|a|): the page ranks by magnitude.  Reading: the key is the fp32 |a| taken
 * as its 31-bit pattern (monotone in |a| for finite values; +-Inf above every
 * finite value and NaN above that), larger first, and equal keys go to the
 * lower position.  Written as a full sort, then the first
 * kb positions re-sorted ascending (the order window entries are stored in). */
void orc_topk(const float *a, int64_t n, int64_t kb, int32_t *sel_out)
{
    if (kb <= 0) return;
    orc_kp *v = (orc_kp *)malloc((size_t)n * sizeof(orc_kp));
    for (int64_t i = 0; i < n; ++i) {
        v[i].key = f2u(a[i]) & 0x7fffffffu;
        v[i].pos = (int32_t)i;
    }
    qsort(v, (size_t)n, sizeof(orc_kp), cmp_key_desc_pos_asc);
    for (int64_t q = 0; q < kb; ++q) sel_out[q] = v[q].pos;
    qsort(sel_out, (size_t)kb, sizeof(int32_t), cmp_int32);
    free(v);
}

/* ------------------------------------------------------------------ */
/* 4-bit quantizer                                                      */
/* ------------------------------------------------------------------ */

uint8_t orc_get_nibble(const uint8_t *bytes, int64_t i)
{
    uint8_t b = bytes[i >> 1];
    return (i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0f);
}

void orc_set_nibble(uint8_t *bytes, int64_t i, uint8_t v)
{
    uint8_t *b = &bytes[i >> 1];
    if (i & 1) *b = (uint8_t)((*b & 0x0f) | (uint8_t)(v << 4));
    else       *b = (uint8_t)((*b & 0xf0) | (v & 0x0f));
}

/* delta = min x, Delta = max x.  A zero result is stored as +0 so the stored
 * statistics do not depend on which signed zero won. */
void orc_group_minmax(const float *x, int64_t n, float *lo, float *hi)
{
    float mn = x[0], mx = x[0];
    for (int64_t i = 1; i < n; ++i) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    *lo = mn + 0.0f;
    *hi = mx + 0.0f;
}

/* Q(x, delta, Delta) with b = 4: levels delta + c*s, c = 0..15, s = (Delta -
 * delta)/15.  Unbiased stochastic rounding (third paragraph): with y = (x -
 * delta)*15/(Delta - delta), take floor(y) and add one when a uniform xi falls
 * below the fractional part, so E[code] = y.  xi is a 16-bit uniform u/2^16
 * from the counter-based generator; the comparison xi < frac is done exactly
 * as u < frac*2^16 in fp32.  A constant group quantizes to code 0. */
void orc_quant_group(const float *x, int64_t n, uint64_t seed, int64_t t, int64_t j,
                     int64_t local0, float lo, float hi, uint8_t *codes_out)
{
    /* Reading: when 15/(Delta - delta) has no finite fp32 value (a range below
     * about 4.4e-38) the group is treated like a constant one. */
    float inv = (hi == lo) ? 0.0f : 15.0f / (hi - lo);
    if (hi == lo || !(inv <= FLT_MAX)) {
        for (int64_t i = 0; i < n; ++i) codes_out[i] = 0;
        return;
    }
    for (int64_t i = 0; i < n; ++i) {
        float y = (x[i] - lo) * inv;
        /* The step only passes finite values in [lo, hi] (it drops non-finite
         * residual entries and resets a group whose range is not finite), so
         * y lies in [0, 15] up to rounding.  Outside that, no float-to-int
         * conversion is left undefined: y >= 15 gives 15 (as the cap below
         * would), y < 0 or NaN gives 0. */
        if (!(y >= 0.0f)) {
            codes_out[i] = 0;
            continue;
        }
        if (y >= 15.0f) {
            codes_out[i] = 15;
            continue;
        }
        float f = floorf(y);
        float frac = y - f;
        uint32_t u = orc_xi16(seed, t, j, local0 + i);
        int code = (int)f + (((float)u < frac * 65536.0f) ? 1 : 0);
        if (code > 15) code = 15;
        codes_out[i] = (uint8_t)code;
    }
}

/* Reading for a residual whose range Delta - delta is not a finite fp32 value
 * (values of both signs near the fp32 limit): the levels would be infinitely
 * far apart and the dequantizer would produce NaN, so the group's error
 * feedback is reset: delta = Delta = 0, hence every code 0. */
void orc_range_reset(float *lo, float *hi)
{
    if (!(*hi - *lo <= FLT_MAX)) {
        *lo = 0.0f;
        *hi = 0.0f;
    }
}

/* Q^{-1}: x_hat = fmaf(code, s, delta) with s = (Delta - delta)/15. */
void orc_dequant_group(const uint8_t *codes, int64_t n, float lo, float hi, float *out)
{
    float s = (hi - lo) / 15.0f;
    for (int64_t i = 0; i < n; ++i) out[i] = fmaf((float)codes[i], s, lo);
}

/* ------------------------------------------------------------------ */
/* One block                                                            */
/* ------------------------------------------------------------------ */

static int cfg_supported(const orc_cfg *c)
{
    if (c->d < 1 || c->B < 1 || c->B >= 32767 || c->m < 1 || c->k < 0 || c->k > c->d) return 0;
    if (c->b != 4) return 0;
    return 1;
}

/* Steps 1-3 of a block: accumulator, Top-k, zeroing; writes the window row.
 * a_out receives the zeroed residual. */
static void block_compress(const orc_cfg *c, int64_t t, int64_t j,
                           const uint16_t *g, const uint8_t *ef, int64_t nib0,
                           const float *stats, uint32_t *gseg, int64_t gstride,
                           float *a_out)
{
    int64_t s, len, off, kb;
    orc_block_range(c, j, &s, &len);
    orc_block_quota(c, j, &off, &kb);
    (void)off;

    /* a_t = g_t + Q^{-1}(e_t, delta_t, Delta_t), in fp32 */
    if (c->flags & ORC_FLAG_NO_EF) {
        for (int64_t i = 0; i < len; ++i) a_out[i] = orc_bf16_to_f32(g[i]);
    } else {
        uint8_t *codes = (uint8_t *)malloc((size_t)len);
        float *xh = (float *)malloc((size_t)len * sizeof(float));
        for (int64_t i = 0; i < len; ++i) codes[i] = orc_get_nibble(ef, nib0 + i);
        orc_dequant_group(codes, len, stats[0], stats[1], xh);
        for (int64_t i = 0; i < len; ++i) a_out[i] = orc_bf16_to_f32(g[i]) + xh[i];
        free(codes);
        free(xh);
    }
    /* Reading for non-finite values (the page assumes finite gradients): a NaN
     * of the accumulator stands for the canonical quiet NaN, whatever payload
     * or sign the arithmetic left on it, so its Top-k key is 0x7fc00000 and
     * its window value the bfloat16 0x7fc0. */
    for (int64_t i = 0; i < len; ++i)
        if (isnan(a_out[i])) a_out[i] = u2f(0x7fc00000u);

    /* (I_t, V_t) = T_k(|a_t|); V is the signed a rounded to bfloat16 */
    int64_t row = t % c->m;
    uint32_t *dst = gseg + row * gstride;
    if (kb > 0) {
        int32_t *sel = (int32_t *)malloc((size_t)kb * sizeof(int32_t));
        orc_topk(a_out, len, kb, sel);
        for (int64_t q = 0; q < kb; ++q) {
            uint32_t idx = (uint32_t)sel[q];
            uint32_t vb = orc_bf16_rne(a_out[sel[q]]);
            dst[q] = idx | (vb << 16);
        }
        /* zero the selected entries of a_t (the bf16 rounding error is dropped) */
        for (int64_t q = 0; q < kb; ++q) a_out[sel[q]] = 0.0f;
        free(sel);
    }
    /* Reading: the keys of NaN and +-Inf are above every finite key, so they
     * are selected first; any left over (more than kb in the block) are
     * dropped from the error feedback, which stays finite. */
    for (int64_t i = 0; i < len; ++i)
        if (!isfinite(a_out[i])) a_out[i] = 0.0f;
}

/* Steps 6-7 of a block: AdamStats over the window, then the AdamW update. */
static void block_apply(const orc_cfg *c, int64_t t, int64_t j, float *theta,
                        const uint32_t *gseg, int64_t gstride, float *mhat, float *vhat)
{
    int64_t s, len, off, kb;
    orc_block_range(c, j, &s, &len);
    orc_block_quota(c, j, &off, &kb);
    (void)off; (void)s;

    float *fac1 = (float *)malloc((size_t)c->m * sizeof(float));
    float *fac2 = (float *)malloc((size_t)c->m * sizeof(float));
    float c1, c2, decay;
    orc_step_constants(c, t, fac1, fac2, &c1, &c2, &decay);

    /* z[I_i] += beta^r V_i, row by row in physical order 0..m-1 */
    float *z1 = (float *)calloc((size_t)len, sizeof(float));
    float *z2 = (float *)calloc((size_t)len, sizeof(float));
    for (int32_t i = 0; i < c->m; ++i) {
        const uint32_t *row = gseg + (int64_t)i * gstride;
        for (int64_t q = 0; q < kb; ++q) {
            uint32_t e = row[q];
            uint32_t I = e & 0xffffu;
            float V = orc_bf16_to_f32((uint16_t)(e >> 16));
            z1[I] = z1[I] + fac1[i] * V;
            z2[I] = z2[I] + fac2[i] * (V * V);
        }
    }

    /* AdamW: decoupled decay first, then theta -= lr * m_hat/(sqrt(v_hat)+eps) */
    for (int64_t i = 0; i < len; ++i) {
        float mh = c1 * z1[i];
        float vh = c2 * z2[i];
        if (mhat) mhat[i] = mh;
        if (vhat) vhat[i] = vh;
        float th = theta[i] * decay;
        float den = sqrtf(vh) + c->eps;
        float upd = c->lr * (mh / den);
        theta[i] = th - upd;
    }
    free(z1); free(z2); free(fac1); free(fac2);
}

int orc_block_step(const orc_cfg *c, int64_t t, int64_t j,
                   float *theta, const uint16_t *g,
                   uint8_t *ef, int64_t nib0, float *stats,
                   uint32_t *gseg, int64_t gstride,
                   float *mhat, float *vhat)
{
    if (!cfg_supported(c) || (c->flags & ORC_FLAG_GLOBAL_QUANT)) return -1;
    int64_t s, len;
    orc_block_range(c, j, &s, &len);
    float *a = (float *)malloc((size_t)len * sizeof(float));
    block_compress(c, t, j, g, ef, nib0, stats, gseg, gstride, a);

    /* e_{t+1} = Q(a_t, delta_{t+1}, Delta_{t+1}); reading: one (delta, Delta)
     * pair per block */
    if (!(c->flags & ORC_FLAG_NO_EF)) {
        float lo, hi;
        uint8_t *codes = (uint8_t *)malloc((size_t)len);
        orc_group_minmax(a, len, &lo, &hi);
        orc_range_reset(&lo, &hi);
        orc_quant_group(a, len, c->seed, t, j, 0, lo, hi, codes);
        for (int64_t i = 0; i < len; ++i) orc_set_nibble(ef, nib0 + i, codes[i]);
        stats[0] = lo;
        stats[1] = hi;
        free(codes);
    }
    free(a);
    block_apply(c, t, j, theta, gseg, gstride, mhat, vhat);
    return 0;
}

int orc_step(const orc_cfg *c, int64_t t, float *theta, const uint16_t *g,
             uint8_t *ef, float *stats, uint32_t *G, float *mhat, float *vhat)
{
    if (!cfg_supported(c)) return -1;
    int64_t nb = orc_num_blocks(c);
    if (!(c->flags & ORC_FLAG_GLOBAL_QUANT)) {
        for (int64_t j = 0; j < nb; ++j) {
            int64_t s, len, off, kb;
            orc_block_range(c, j, &s, &len);
            orc_block_quota(c, j, &off, &kb);
            int rc = orc_block_step(c, t, j, theta + s, g + s, ef, s, stats + 2 * j,
                                    G + off, c->k, mhat ? mhat + s : NULL, vhat ? vhat + s : NULL);
            if (rc) return rc;
        }
        return 0;
    }
    /* The literal form of the first paragraph: scalar delta, Delta over all d.
     * The accumulator needs the whole vector before the quantizer runs. */
    float *a = (float *)malloc((size_t)c->d * sizeof(float));
    for (int64_t j = 0; j < nb; ++j) {
        int64_t s, len, off, kb;
        orc_block_range(c, j, &s, &len);
        orc_block_quota(c, j, &off, &kb);
        block_compress(c, t, j, g + s, ef, s, stats, G + off, c->k, a + s);
    }
    if (!(c->flags & ORC_FLAG_NO_EF)) {
        float lo, hi;
        orc_group_minmax(a, c->d, &lo, &hi);
        orc_range_reset(&lo, &hi);
        uint8_t *codes = (uint8_t *)malloc((size_t)c->B);
        for (int64_t j = 0; j < nb; ++j) {
            int64_t s, len;
            orc_block_range(c, j, &s, &len);
            orc_quant_group(a + s, len, c->seed, t, j, 0, lo, hi, codes);
            for (int64_t i = 0; i < len; ++i) orc_set_nibble(ef, s + i, codes[i]);
        }
        free(codes);
        stats[0] = lo;
        stats[1] = hi;
    }
    free(a);
    for (int64_t j = 0; j < nb; ++j) {
        int64_t s, len, off, kb;
        orc_block_range(c, j, &s, &len);
        orc_block_quota(c, j, &off, &kb);
        block_apply(c, t, j, theta + s, G + off, c->k, mhat ? mhat + s : NULL, vhat ? vhat + s : NULL);
    }
    return 0;
}

/* The baseline AdamW of the comparison in the second paragraph (fp32 m and v,
 * 8 bytes of state per parameter), in the decoupled-decay form used above. */
void orc_adamw_step(int64_t n, int64_t t, float b1, float b2, float eps, float lr, float wd,
                    float *theta, const uint16_t *g, float *m, float *v)
{
    const float omb1 = (float)(1.0 - (double)b1);
    const float omb2 = (float)(1.0 - (double)b2);
    const float r1 = (float)(1.0 / (1.0 - pow((double)b1, (double)t)));
    const float r2 = (float)(1.0 / (1.0 - pow((double)b2, (double)t)));
    const float decay = (float)(1.0 - (double)lr * (double)wd);
    for (int64_t i = 0; i < n; ++i) {
        float gi = orc_bf16_to_f32(g[i]);
        m[i] = b1 * m[i] + omb1 * gi;
        v[i] = b2 * v[i] + omb2 * (gi * gi);
        float mh = m[i] * r1;
        float vh = v[i] * r2;
        theta[i] = theta[i] * decay - lr * (mh / (sqrtf(vh) + eps));
    }
}

/* The 8-bit comparison optimizer (see the header for the reading). */
void orc_adamw8_step(int64_t n, int64_t t, float b1, float b2, float eps, float lr, float wd,
                     float *theta, const uint16_t *g, int8_t *cm, uint8_t *cv, float *sm, float *sr)
{
    const float omb1 = (float)(1.0 - (double)b1);
    const float omb2 = (float)(1.0 - (double)b2);
    const float r1 = (float)(1.0 / (1.0 - pow((double)b1, (double)t)));
    const float r2 = (float)(1.0 / (1.0 - pow((double)b2, (double)t)));
    const float decay = (float)(1.0 - (double)lr * (double)wd);
    float m[ORC_Q8_BLOCK], v[ORC_Q8_BLOCK];
    for (int64_t b0 = 0; b0 < n; b0 += ORC_Q8_BLOCK) {
        const int64_t q = b0 / ORC_Q8_BLOCK;
        const int64_t len = (n - b0 < ORC_Q8_BLOCK) ? n - b0 : ORC_Q8_BLOCK;
        const float qm = sm[q] / 127.0f, qr = sr[q] / 255.0f;
        float amax = 0.0f, rmax = 0.0f;
        for (int64_t i = 0; i < len; ++i) {
            const float mo = (float)cm[b0 + i] * qm;
            const float ro = (float)cv[b0 + i] * qr;
            const float vo = ro * ro;
            const float gi = orc_bf16_to_f32(g[b0 + i]);
            m[i] = b1 * mo + omb1 * gi;
            v[i] = b2 * vo + omb2 * (gi * gi);
            const float mh = m[i] * r1;
            const float vh = v[i] * r2;
            theta[b0 + i] = theta[b0 + i] * decay - lr * (mh / (sqrtf(vh) + eps));
            if (fabsf(m[i]) > amax) amax = fabsf(m[i]);
            if (sqrtf(v[i]) > rmax) rmax = sqrtf(v[i]);
        }
        sm[q] = amax;
        sr[q] = rmax;
        const float im = (amax > 0.0f) ? 127.0f / amax : 0.0f;
        const float ir = (rmax > 0.0f) ? 255.0f / rmax : 0.0f;
        for (int64_t i = 0; i < len; ++i) {
            float c = rintf(m[i] * im);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            cm[b0 + i] = (int8_t)c;
            float d = rintf(sqrtf(v[i]) * ir);
            if (d > 255.0f) d = 255.0f;
            cv[b0 + i] = (uint8_t)d;
        }
    }
}

uint64_t orc_state_bytes(const orc_cfg *c)
{
    return (uint64_t)((c->d + 1) / 2) + 4ull * (uint64_t)c->m * (uint64_t)c->k;
}

/* ------------------------------------------------------------------ */
/* Array helpers for the Python side (plain loops over the above)        */
/* ------------------------------------------------------------------ */

void orc_bf16_rne_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

void orc_pcg_hash_array(const uint32_t *x, int64_t n, uint32_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_pcg_hash(x[i]);
}

void orc_xi16_array(uint64_t seed, int64_t t, int64_t j, int64_t local0, int64_t n, uint32_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_xi16(seed, t, j, local0 + i);
}
