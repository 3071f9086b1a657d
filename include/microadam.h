/*
 * libmicroadam -- the MicroAdam optimizer step on AMD Instinct MI355X (gfx950).
 *
 * The method is the one on the page "MicroAdam (Sparse-Gradient Adaptive
 * Optimization with Quantized Error Feedback)".  Its first paragraph defines
 * one step t over a flat parameter vector of length d:
 *
 *   a_t = g_t + Q^{-1}(e_t, delta_t, Delta_t)     accumulate the 4-bit error
 *   (I_t, V_t) = T_k(|a_t|)                       block-wise Top-k, k = d/100,
 *                                                 int16 indices relative to
 *                                                 blocks of B_d < 2^15 - 1
 *   a_t[I_t] = 0;  e_{t+1} = Q(a_t, ...)          requantize the residual, b = 4
 *   G[t mod m] = (I_t, V_t)                       circular window of m rows
 *   m_hat = AdamStats(beta1, G), v_hat = AdamStats(beta2, G^2)
 *                                                 z[I_i] += beta^r V_i
 * and the parameters take an AdamW step with (m_hat, v_hat).  Its second
 * paragraph counts the state: 0.5d bytes of codes and 4mk bytes of window.
 *
 * Layouts (device memory, all owned by the library unless stated):
 *   codes   u8[ceil(d/2)]  element i in byte i/2, low nibble for even i
 *   stats   f32[2*n_b]     per block j: {delta_j, Delta_j} (min and max of the
 *                          block's residual; one pair per block)
 *   window  u32[m][k]      row r holds k entries; block j's k_b(j) entries start
 *                          at offset floor(k*s_j/d) of every row, ascending in
 *                          index; entry = index | bf16_bits(V) << 16
 * with n_b = ceil(d/B_d), block j = [s_j, e_j) = [j*B_d, min((j+1)*B_d, d)) and
 * k_b(j) = floor(k*e_j/d) - floor(k*s_j/d).
 *
 * Errors: functions return 0 or a negative MA_E* code (pointer-returning ones
 * return NULL).  The code and a message are kept per calling thread
 * (ma_last_error, ma_last_error_message).  Nothing here prints or aborts.
 *
 * Streams: ma_step only enqueues work on the stream given and never
 * synchronizes.  The debug calls (ma_debug_moments, ma_debug_residual) run on
 * the stream given and synchronize it before returning.  The state/accessor
 * calls marked "synchronous" wait for the whole device.  Calls on one handle
 * must not overlap.
 */
#ifndef MICROADAM_H
#define MICROADAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ma_ctx ma_ctx;

enum {
    MA_OK = 0,
    MA_EINVAL = -1,         /* bad argument: null or misaligned pointer, out-of-range value */
    MA_EUNSUPPORTED = -2,   /* valid for the method but not built here (b != 4) */
    MA_ENOMEM = -3,         /* device allocation failed; nothing is leaked */
    MA_EHIP = -4,           /* a HIP call or kernel launch failed */
};

/* Flags for ma_set_flags. */
#define MA_FLAG_NO_EF 1u        /* a_t = g_t: stored error neither read nor rewritten */
#define MA_FLAG_FORCE_DENSE 4u  /* stream the parameters through registers in the update
                                   (same results) */
#define MA_FLAG_FORCE_SPARSE 8u /* gather only touched parameters (same results; ignored
                                   when weight decay makes every parameter change) */
/* Without either flag, full blocks of 16-byte aligned fp32 parameters with a
 * short window (m * k_b up to 2048 entries: m <= 12 at k = d/100 and
 * B_d = 16384) are loaded whole into registers and merged through LDS in
 * chunks: the touched positions are updated there and every parameter line is
 * written back whole.  Elsewhere the touched parameters are gathered (no
 * decay) or all of them streamed (decay).  Every form gives the same bits. */
#define MA_FLAG_UNFUSED 16u     /* run compress and update as two kernels even where the
                                   fused per-block kernel applies (same results) */
#define MA_FLAG_ROW_SUMS 64u     /* AdamStats by adding the window rows one at a time into
                                   per-slot sums (a barrier per row) wherever the library would
                                   otherwise sort the window by position and sum each column
                                   (its choice per step: longer windows, decay, fp32 parameters
                                   from 10 rows; same results either way) */
#define MA_FLAG_GLOBAL_QUANT 32u /* one (delta, Delta) pair over all d, the literal scalar form
                                   of the first paragraph (default: one pair per B_d block).
                                   Costs a second pass over gradients and codes.  The pair is
                                   stored as every block's statistics.  Ignored with NO_EF. */

/* State buffers for ma_read_state / ma_write_state. */
#define MA_STATE_CODES 0
#define MA_STATE_STATS 1
#define MA_STATE_WINDOW 2

/*
 * Creates an optimizer for d parameters (first paragraph of the MicroAdam
 * page: blocks of B_d < 2^15 - 1, Top-k budget k per step, window of m rows,
 * b-bit error quantizer; AdamW hyperparameters beta1, beta2, eps, lr, wd;
 * seed keys the quantizer's counter-based random numbers on (seed, step,
 * element)).  Requires d >= 1, 1 <= B_d <= 32766, 0 <= k <= d, m >= 1,
 * 0 <= beta < 1, eps > 0, finite lr and wd >= 0; b must be 4 and m at
 * most 1024 (MA_EUNSUPPORTED otherwise: the update keeps the window's decay
 * factors in LDS).  Allocates and zero-fills all state on the
 * current HIP device (so e_1 = 0 and unwritten window rows add nothing);
 * step count t = 0.  Returns NULL on error.
 */
ma_ctx *ma_create(int64_t d, int32_t B_d, int64_t k, int32_t m, int32_t b, float beta1,
                  float beta2, float eps, float lr, float wd, uint64_t seed);

/*
 * One MicroAdam step (t -> t+1).  params: caller-owned device f32[d], updated
 * in place.  grads: caller-owned device bf16[d] (raw bits), read only.  Both
 * must be element-aligned and live on the handle's device.  Enqueued on
 * `stream`, asynchronous.  Returns MA_OK, MA_EINVAL (null/misaligned pointer)
 * or MA_EHIP (launch error); t advances only on success.  After MA_EHIP some
 * of the step's kernels may already be enqueued, so the state can be partly
 * advanced: restore a saved state (ma_write_state, ma_set_step) or destroy
 * the handle.
 */
int ma_step(ma_ctx *h, float *params, const uint16_t *grads, hipStream_t stream);

/*
 * The same step for bfloat16 parameters (the regime of the fourth paragraph's
 * full fine-tuning of LLaMA-2 7B on one 40 GB GPU: bf16 parameters and
 * gradients plus 0.9d of state).  params: caller-owned device bf16[d] (raw
 * bits), 2-byte aligned, updated in place: each changed parameter is widened
 * exactly to fp32, updated as ma_step updates an fp32 parameter (decay, then
 * the Adam step), and rounded to nearest even once.  Parameters no window
 * entry touches are unchanged when wd = 0.  Errors as ma_step.
 */
int ma_step_bf16(ma_ctx *h, uint16_t *params, const uint16_t *grads, hipStream_t stream);

/*
 * For callers that cannot allocate: code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc.  The same step as ma_step (same
 * arguments, results and errors), with nothing allocated or created per call:
 * every launch goes to `stream` (no side stream, no timing events), and the
 * step's scratch (the deferred-block list and its counters, the global
 * quantizer's per-block min / max and cut) lives in one static device array of
 * 24 MiB that each device the library runs on holds until the process ends,
 * instead of the handle's buffers.  Handles of more than 2^20 blocks are
 * rejected with MA_EUNSUPPORTED before anything is launched; MA_EHIP if the
 * array's device address could not be looked up when the handle was created.
 * Every call on one device shares that array and leaves its contents behind
 * (the step clears what must start at zero), so ma_step_noalloc calls that
 * overlap on one device race, even on different handles and streams.
 */
int ma_step_noalloc(ma_ctx *h, float *params, const uint16_t *grads, hipStream_t stream);

/*
 * Comparison baseline: one fp32 AdamW step (the 8d-byte optimizer the second
 * paragraph compares against), stateless, on caller-owned device arrays of n
 * elements: theta, m, v fp32 (updated in place), grads bf16 (raw bits).  Step t
 * is 1-based; with m = v = 0 before step 1.  Per element, each operation
 * rounded once in fp32: m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*g*g;
 * theta = theta*decay - lr*((m*r1)/(sqrtf(v*r2) + eps)), where (1-b),
 * decay = 1 - lr*wd and r = 1/(1 - b^t) are computed in double and rounded to
 * fp32.  Enqueued on `stream`.  MA_EINVAL for n < 0, t < 1, a null or
 * misaligned pointer (4 bytes for fp32, 2 for bf16); MA_OK for n = 0.
 */
int ma_adamw_step(int64_t n, int64_t t, float beta1, float beta2, float eps, float lr, float wd, float *theta,
                  const uint16_t *grads, float *m, float *v, hipStream_t stream);

/*
 * Comparison baseline: one 8-bit block-quantized AdamW step (the 2d-byte
 * optimizer the second paragraph compares against).  The page fixes no 8-bit
 * scheme; this one: blocks of 256 elements, each with scales sm = max|m| and
 * sr = max sqrt(v); cm: int8 codes rint(m * (127/sm)); cv: uint8 codes
 * rint(sqrt(v) * (255/sr)) (round to nearest even; a zero block has scale 0
 * and codes 0).  A step dequantizes m~ = cm * (sm/127), v~ = (cv * (sr/255))^2,
 * applies the ma_adamw_step recurrence and update to them, and requantizes the
 * new moments with the block's new scales.  Arrays caller-owned on the device:
 * theta fp32[n], grads bf16[n], cm int8[n], cv uint8[n], sm, sr fp32[ceil(n/256)]
 * (all zero before step 1).  Errors as ma_adamw_step.
 */
int ma_adamw8_step(int64_t n, int64_t t, float beta1, float beta2, float eps, float lr, float wd, float *theta,
                   const uint16_t *grads, int8_t *cm, uint8_t *cv, float *sm, float *sr, hipStream_t stream);

/* Optimizer-state bytes the second paragraph of the MicroAdam page counts:
 * ceil(d/2) + 4*m*k (0.9d at m = 10, k = d/100).  0 for NULL. */
size_t ma_state_bytes(const ma_ctx *h);

/* Everything else the library holds on the device: per-block statistics
 * (8*n_b), the block offset table (8*(n_b+1)), the beta-power table (8*m),
 * the code buffer's tail padding, the touched-parameter counters (8 KiB), the
 * compressor's deferred-block list (8*n_b + 256) and the global quantizer's
 * per-block min / max and cut (16*n_b + 8).
 * 0 for NULL. */
size_t ma_aux_bytes(const ma_ctx *h);

/* Frees every device buffer of the handle; NULL is accepted. */
void ma_destroy(ma_ctx *h);

/* Last error code / message of the calling thread (MA_OK / "" if none). */
int ma_last_error(void);
const char *ma_last_error_message(void);

/* Accessors. */
int64_t ma_get_step(const ma_ctx *h);       /* t: number of completed steps */
int64_t ma_num_blocks(const ma_ctx *h);     /* n_b */

/* Sets the step counter (used when importing a saved state). t >= 0. */
int ma_set_step(ma_ctx *h, int64_t t);
/* Sets MA_FLAG_* bits (replaces the previous set). */
int ma_set_flags(ma_ctx *h, uint32_t flags);
/* Changes the learning rate used by later steps (finite). */
int ma_set_lr(ma_ctx *h, float lr);

/*
 * Copies nbytes at byte_offset of state buffer `which` (MA_STATE_*) to or from
 * host memory.  Synchronous (waits for the device first).  MA_EINVAL when the
 * range is outside the buffer (codes: ceil(d/2) bytes, stats: 8*n_b, window:
 * 4*m*k) or a pointer is NULL.  Together with ma_set_step this exports and
 * imports the complete state: the random numbers are keyed on (seed, step,
 * element) and carry no hidden state.
 */
int ma_read_state(const ma_ctx *h, int which, uint64_t byte_offset, uint64_t nbytes, void *host_dst);
int ma_write_state(ma_ctx *h, int which, uint64_t byte_offset, uint64_t nbytes, const void *host_src);

/*
 * The whole optimizer state in one call, for checkpoint and exact resume (the
 * state the second paragraph of the MicroAdam page counts, plus the block
 * statistics and the step count; the quantizer's random numbers are keyed on
 * (seed, step, element), so these determine every later step).  Host buffers
 * the caller owns: codes ceil(d/2) bytes (element i in nibble i), stats 8*n_b
 * bytes (fp32 delta, Delta per block), window 4*m*k bytes (row-major m x k
 * entries, int16 index | bf16 value << 16); t the number of completed steps.
 * window may be NULL when m*k = 0.  Synchronous: waits for the device first.
 * MA_EINVAL for a null handle or buffer, or t < 0 on import; MA_EHIP if a copy
 * fails, after which an imported state is incomplete and must be imported
 * again before the next step.
 */
int ma_export_state(const ma_ctx *h, void *codes, void *stats, void *window, int64_t *t);
int ma_import_state(ma_ctx *h, const void *codes, const void *stats, const void *window, int64_t t);

/*
 * m_hat and v_hat of the last completed step (AdamStats of the first
 * paragraph, bias-corrected) for nblocks chosen blocks.  blocks: host array of
 * block numbers.  mhat_out, vhat_out: device f32[nblocks * B_d]; row q holds
 * block blocks[q], its first len_j entries valid (0 where the window has no
 * entry).  Runs on `stream` and synchronizes it before returning.  MA_EINVAL
 * before the first step or for a block number out of range.
 */
int ma_debug_moments(ma_ctx *h, const int64_t *blocks, int64_t nblocks, float *mhat_out,
                     float *vhat_out, hipStream_t stream);

/*
 * The accumulator of the first line of the step (first paragraph of the
 * MicroAdam page), a_t = g_t + Q^-1(e_t, delta_t, Delta_t), for nblocks chosen
 * blocks, computed from the current codes and statistics (the state the next
 * ma_step would start from) and the given gradients, with the step's own
 * arithmetic (fp32: f32(g) + fmaf(code, (Delta - delta)/15, delta); with
 * MA_FLAG_NO_EF, f32(g)).  The state is not changed.  grads: device bf16[d].
 * blocks: host array of block numbers.  a_out: device f32[nblocks * B_d]; row q
 * holds block blocks[q], 0 past the block's end.  Runs on `stream` and
 * synchronizes it before returning.  MA_EINVAL for a NULL pointer or a block
 * number out of range; MA_ENOMEM if the temporary block list cannot be
 * allocated.
 */
int ma_debug_residual(ma_ctx *h, const uint16_t *grads, const int64_t *blocks, int64_t nblocks,
                      float *a_out, hipStream_t stream);

/*
 * Per-kernel timing with HIP events recorded around each launch, on the stream
 * the kernel runs on.  ma_set_timing(h, 1) clears and starts collecting;
 * ma_kernel_times waits for the recorded events and returns, for nk <= 3
 * kernels (0: compress, 1: adamstats_apply, 2: the fused step of full blocks,
 * with the pass over the blocks it deferred), the summed milliseconds and
 * launch counts.  The fused step's own launches are not counted under 0 or 1.
 */
int ma_set_timing(ma_ctx *h, int on);
int ma_kernel_times(ma_ctx *h, double *ms_out, int64_t *launches_out, int nk);

/*
 * Overlap inside one step.  The blocks are cut into `chunks` contiguous ranges
 * (1 <= chunks <= 64, at most n_b are used); the update of range i runs on a
 * stream the handle owns (default priority), after the compressor of range i
 * and concurrently with the compressor of range i+1, which stays on the
 * caller's stream.  Ranges share no state, so results do not depend on
 * `chunks`.  The caller's stream waits for the handle's stream before ma_step
 * returns, so the step remains ordered on `stream` as one unit.  Default: 8
 * when n_b >= 8192, else 1.  With timing on, the per-kernel times then include
 * the time the two kernels spend sharing the device.
 */
int ma_set_pipeline(ma_ctx *h, int chunks);
/* Number of block ranges ma_step uses (min(chunks, n_b)); -1 for NULL. */
int ma_get_pipeline(const ma_ctx *h);

/* Counting of touched parameters (positions present in the window, i.e. the
 * parameters an update reads and writes), summed over blocks and steps.
 * ma_set_count_touched(h, 1) zeroes the counter (synchronous) and makes every
 * later step add its count on the device; ma_touched_count waits for the
 * device and returns the sum, or -1 when counting is off. */
int ma_set_count_touched(ma_ctx *h, int on);
int64_t ma_touched_count(ma_ctx *h);

#ifdef __cplusplus
}
#endif
#endif
