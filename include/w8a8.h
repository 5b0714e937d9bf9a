/*
 * w8a8.h -- C ABI of the deterministic W8A8 int8 linear layer for MI355X (gfx950).
 *
 * The layer is the one described on the review page "StartLux-Prism: Fast,
 * exact inference for StartLux-Decision models on NVIDIA GPUs".  Weights are
 * int8 with one fp32 scale per output channel.  Activations are divided by a
 * SmoothQuant per-channel vector and quantised to int8 per token (section
 * "Compute shared evidence once").  The int8 products accumulate exactly in
 * int32.  Split-K partial sums stay integers.  A fixed sequence of binary32
 * operations then applies the scales and the residual (section "Bitwise
 * consistency is not lossless quantization").  Running the same projection
 * as a read-out over a few candidate vocabulary rows follows the dsiab.com
 * post on moving decision models from vLLM to Prism, section "方案": scoring
 * only the candidates, then normalising among them, equals the
 * full-vocabulary softmax renormalised over those candidates.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device.  Host pointers are marked "host".
 *   - Matrices are row-major.  int8 operands are K-contiguous: the
 *     activation is [M,K] and the weight is [N,K].
 *   - `stream` is a hipStream_t passed as void*.  NULL means the default
 *     stream.  Every compute call is asynchronous on `stream`; no call
 *     synchronises.
 *   - The caller owns every buffer, including the split-K workspace.  The
 *     library allocates no device memory and keeps no per-call state.
 *   - Host-checkable errors return a negative w8a8_status before anything
 *     is launched, and leave every output untouched.
 *   - Determinism: output row m depends only on row m of the inputs and on
 *     the weights and scales.  It does not depend on M, the row's position,
 *     other rows, padding, the split-K factor, the kernel or tile the
 *     library picks, the stream, or the run.  Results are bit-identical to
 *     the plain definitions written next to each call.
 *   - Weights must lie in [-127, 127] (the symmetric range), and K <= 133120.
 *     Then |sum_k q*w| <= K * 127^2 < 2^31, so int32 accumulation is exact.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARG = -1,        /* null pointer, negative size, bad leading dimension */
    W8A8_ERR_SHAPE = -2,              /* K not a positive multiple of 64, or a size limit */
    W8A8_ERR_ALIGN = -3,              /* a pointer or stride breaks the stated alignment */
    W8A8_ERR_WORKSPACE = -4,          /* split-K workspace missing or too small */
    W8A8_ERR_K_BOUND = -5,            /* K above W8A8_MAX_K: int32 accumulation could overflow */
    W8A8_ERR_TOO_MANY_CANDIDATES = -6,/* C above W8A8_MAX_CANDIDATES: use the full-vocabulary GEMM */
    W8A8_ERR_HIP = -7                 /* a HIP launch or runtime call failed */
} w8a8_status;

/* Largest multiple of 64 with K * 127^2 < 2^31 (the bound is K <= 133144). */
#define W8A8_MAX_K 133120
/* Hard cap on candidates per row.  The dsiab.com post (section "复盘", its
 * closing list of improvements) asks for a cap on the candidate count, with
 * fallback to the general path above it.  The number 64 is this library's
 * choice. */
#define W8A8_MAX_CANDIDATES 64
/* Largest split-K factor accepted. */
#define W8A8_MAX_SPLITK 64
/* Most rows per call of the entry points that work row by row: the
 * quantisations and row maxima (M), the candidate read-out, softmax and
 * answer head (M) and the requantisation (N).  Above it they return
 * W8A8_ERR_SHAPE.  (Each such row takes one workgroup; the limit keeps a
 * launch below 2^32 work-items.) */
#define W8A8_MAX_ROWS 4194303

/* Human-readable name of a status code (host; never NULL). */
const char* w8a8_status_string(int status);

/* Version of this ABI: major*10000 + minor*100 + patch (host). */
int w8a8_abi_version(void);

/*
 * w8a8_quantize_act -- per-token int8 quantisation after a per-channel
 * smoothing divide (review page, section "Compute shared evidence once").
 *
 * For each output row m, with source row i = row_idx ? row_idx[m] : m, and
 * fl() meaning one correctly rounded binary32 operation:
 *     x'[k]  = fl(x[i,k] / smooth[k])                (true IEEE division)
 *     a      = max_k |x'[k]|
 *     sx[m]  = fl(a / 127)
 *     xq[m,k]= clamp(round_half_even(fl(x'[k] / sx[m])), -127, 127),
 *              or 0 for every k when sx[m] == 0.
 *
 * x        device, fp32; row i starts at x + i*ldx; x_rows rows are readable.
 * ldx      elements between rows, >= K and a multiple of 4.
 * x_rows   rows of x that may be read; every row_idx entry must lie in [0, x_rows).
 * row_idx  device int32 [M] or NULL.  NULL requires M <= x_rows.  An entry
 *          outside [0, x_rows) yields xq[m,:] = 0 and sx[m] = quiet NaN,
 *          with no out-of-bounds read.
 * smooth   device fp32 [K], every entry > 0 and finite.
 * M, K     M >= 0 (M == 0 is a no-op); K a positive multiple of 64, K <= W8A8_MAX_K.
 * xq       device int8 [M,K] row-major, 16-byte aligned.
 * sx       device fp32 [M].
 * Alignment: x and smooth 16-byte aligned.
 * Non-finite values: a row whose smoothed values x' include a NaN or an
 * infinity (from x itself, or from x/smooth overflowing) has no finite
 * maximum and so no scale.  It is treated like a row that cannot be read:
 * sx[m] = quiet NaN and xq[m,:] = 0 (its GEMM outputs are then NaN).  Other
 * rows are not affected.
 */
int w8a8_quantize_act(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                      const float* smooth, int64_t M, int64_t K,
                      int8_t* xq, float* sx, void* stream);

/*
 * w8a8_gemm -- int8 x int8 GEMM with exact int32 accumulation and the fixed
 * binary32 epilogue (review page, section "Bitwise consistency is not
 * lossless quantization"):
 *     acc[m,n] = sum_k xq[m,k] * w[n,k]                         (exact, int32)
 *     y[m,n]   = fl(fl(fl(float(acc)) * sx[m]) * sw[n])          (+ residual:)
 *     y[m,n]   = fl(that + residual[m,n])
 * Each step rounds once (ties to even).  No fused multiply-add is used.
 * float(acc) is the int32 -> binary32 conversion, ties to even.
 *
 * xq        device int8 [M,K], 16-byte aligned (from w8a8_quantize_act).
 * sx        device fp32 [M].
 * w         device int8 [N,K], 16-byte aligned, entries in [-127, 127].
 * sw        device fp32 [N].
 * residual  device fp32 [M,N] or NULL.  It may be the same pointer as y
 *           (in-place update of the residual stream), but must not
 *           otherwise overlap y.
 * y         device fp32 [M,N], 4-byte aligned.
 * M, N      >= 0 (an empty output is a no-op).
 * K         positive multiple of 64, <= W8A8_MAX_K.
 */
int w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
              const float* residual, float* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w8a8_gemm_splitk_workspace_bytes -- bytes of device workspace that
 * w8a8_gemm_splitk needs for this shape and split factor (host; no GPU
 * call).  Returns 0 when splitk == 1 or the output is empty, and
 * (size_t)-1 for invalid arguments.
 */
size_t w8a8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splitk);

/*
 * w8a8_gemm_splitk -- the same result as w8a8_gemm, with K cut into at
 * most `splitk` contiguous chunks (review page, section "Bitwise
 * consistency is not lossless quantization": split-K partial sums stay
 * integers).  With S chunks (S = splitk on the tiled kernel; the column-panel
 * kernel, which runs most products of up to 1536 rows, picks S <= splitk for
 * speed; w8a8_gemm_plan reports which):
 *     chunk c covers k in [c*Kc, min((c+1)*Kc, K)), Kc = ceil(K/S)
 *     rounded up to a multiple of 64 (of 128 on the panel kernel);
 *     P_c[m,n] = sum over chunk c of xq[m,k]*w[n,k]      (int32)
 *     acc      = P_0 + P_1 + ... + P_{S-1}                (int32)
 * followed by the same epilogue as w8a8_gemm.  No floating-point atomic is
 * used anywhere.  Each chunk writes P_c as int32 to its own slice of the
 * workspace; a second kernel on the same stream adds the slices in chunk
 * order and runs the epilogue.  Integer addition is exact and associative,
 * so neither that order nor S can change a bit: the output is
 * bit-identical to w8a8_gemm.
 *
 * splitk     1 <= splitk <= W8A8_MAX_SPLITK.
 * workspace  device, 256-byte aligned, at least
 *            w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk) bytes
 *            (splitk * M * N int32 partials).  Its contents on entry do not
 *            matter and are overwritten; calls that share one workspace
 *            must not overlap in time.  Ignored when splitk == 1.
 * Other arguments as for w8a8_gemm.
 */
int w8a8_gemm_splitk(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                     const float* residual, float* y, int64_t M, int64_t N, int64_t K,
                     int splitk, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's own split-K scratch (64 MiB per GPU), the most
 * w8a8_gemm_splitk_noalloc accepts. */
#define W8A8_NOALLOC_SCRATCH_BYTES 67108864

/*
 * w8a8_gemm_splitk_noalloc -- w8a8_gemm_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and result bits as
 * w8a8_gemm_splitk, without the workspace: the int32 partials go to a
 * scratch array of W8A8_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends.  The call allocates nothing.
 * Its first call on a device looks up that device's array (a runtime
 * symbol query, no allocation); later calls do no host-side set-up.
 *
 * Returns W8A8_ERR_WORKSPACE when
 * w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk) exceeds
 * W8A8_NOALLOC_SCRATCH_BYTES (e.g. 256 x 5120 at splitk 8 is 42 MB and fits;
 * 8192 x 5120 at splitk 2 is 336 MB and does not: use w8a8_gemm_splitk).
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (nothing in it needs clearing: each chunk overwrites
 * its whole slice).  Calls that overlap in time on one GPU (on different
 * streams, or from several host threads) therefore race and must be
 * serialised by the caller.
 */
int w8a8_gemm_splitk_noalloc(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                             const float* residual, float* y, int64_t M, int64_t N, int64_t K,
                             int splitk, void* stream);

/*
 * w8a8_readout_candidates -- candidate-only lm_head read-out.  The review
 * page, section "Compute shared evidence once", keeps the read-out to the
 * answer positions.  The dsiab.com post, section "方案", scores only the
 * candidate tokens.
 *     logits[m,c] = fl(fl(float(sum_k xq[m,k]*w_vocab[cand[m,c],k]) * sx[m]) * sw_vocab[cand[m,c]])
 * This is bit-identical to column cand[m,c] of
 * w8a8_gemm(xq, sx, w_vocab, sw_vocab, NULL, ...) (no residual).  For
 * K <= 18432 one workgroup per row computes its C dot products (the answer
 * head's code); for larger K the skinny-GEMM kernel runs, with the weight
 * rows gathered through `cand`.
 *
 * xq, sx      device int8 [M,K] (16-byte aligned) and fp32 [M]; usually the
 *             answer rows, picked with w8a8_quantize_act's row_idx.
 * w_vocab     device int8 [V,K], 16-byte aligned; sw_vocab device fp32 [V].
 * cand        device int32 [M,C]: vocabulary ids, one set per row.  A shared
 *             set is the same row repeated.
 * C           0 <= C <= W8A8_MAX_CANDIDATES (above it: W8A8_ERR_TOO_MANY_CANDIDATES,
 *             use w8a8_gemm over the whole vocabulary instead).
 * logits      device fp32 [M,C].
 * err_flag    device int32 or NULL.  An id outside [0,V) makes its logit a
 *             quiet NaN.  If err_flag is given, bit 0 of *err_flag is set
 *             (bitwise OR; the library never clears it).
 */
int w8a8_readout_candidates(const int8_t* xq, const float* sx, int64_t M, int64_t K,
                            const int8_t* w_vocab, const float* sw_vocab, int64_t V,
                            const int32_t* cand, int64_t C, float* logits, int32_t* err_flag,
                            void* stream);

/*
 * w8a8_requantize_q8_0 -- startup requantisation of Q8_0 weights with
 * SmoothQuant (review page, section "Compute shared evidence once": the
 * Q8_0 weights are requantised with SmoothQuant at startup).  Q8_0 keeps
 * blocks of 32 int8 codes along a weight row, each block with one binary16
 * scale: w = d * q.  With the smoothing vector that divides the
 * activations (x' = x / s), per output channel n:
 *     w'[n,k] = fl(fl(d[n, k/32] * q[n,k]) * smooth[k])
 *     sw[n]   = fl(max_k |w'[n,k]| / 127)
 *     w[n,k]  = clamp(rne(fl(w'[n,k] / sw[n])), -127, 127)   (0 if sw[n] = 0)
 * The result feeds w8a8_gemm as (w, sw).  The smoothing vector comes from
 * calibration (not done here).  A row whose w' holds a NaN or an infinity
 * (a non-finite block scale or smoothing value, or an overflow) gets
 * sw[n] = NaN and all codes 0, as an activation row that cannot be quantised
 * does; a non-finite smoothing value therefore leaves every row so.
 *
 * q       device int8 [N,K] Q8_0 codes, 16-byte aligned; K a multiple of 64.
 * d       device uint16 [N,K/32]: the binary16 bit patterns of the block
 *         scales (2-byte aligned).
 * smooth  device fp32 [K], 16-byte aligned.
 * w, sw   device int8 [N,K] (16-byte aligned; may be q itself, else must not
 *         overlap it) and fp32 [N].
 */
int w8a8_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N, int64_t K,
                         int8_t* w, float* sw, void* stream);

/*
 * Tensor-parallel row-parallel layers.  The review page, section "Bitwise
 * consistency is not lossless quantization", combines the integer partial
 * sums of the ranks before scaling.  A rank holds a K-slice of the
 * activations and of the weight; for its int32 partials to be added before
 * scaling, every rank quantises with one per-token scale, taken from the
 * exact MAX of the ranks' slice maxima.  One rank's steps:
 *   w8a8_row_absmax         slice maximum (then MAX across ranks)
 *   w8a8_quantize_act_amax  quantise the slice with the global maximum
 *   w8a8_gemm_int32         int32 partials of the slice (then SUM across ranks)
 *   w8a8_epilogue_int32     the fixed epilogue of the added partials
 * With the collectives done exactly (MAX of floats, SUM of int32), the
 * output is bit-identical to the single-device w8a8_quantize_act + w8a8_gemm
 * for any number of ranks and any slicing into multiples of 64.
 */

/*
 * w8a8_row_absmax -- amax[m] = max_k |fl(x[row m, k] / smooth[k])| over this
 * K-slice, exact (every element divided).  accumulate != 0: amax[m] =
 * fmax(amax[m], that value), so successive calls over the slices of one
 * device give the global maximum.  A slice holding a NaN or infinite
 * smoothed value gives +Inf (so the global maximum marks the row invalid on
 * every rank, as w8a8_quantize_act does on one device).  A row index
 * outside [0, x_rows) writes NaN.  Arguments as for w8a8_quantize_act; amax
 * device fp32 [M].
 */
int w8a8_row_absmax(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                    const float* smooth, int64_t M, int64_t K, int accumulate, float* amax,
                    void* stream);

/*
 * w8a8_quantize_act_amax -- w8a8_quantize_act with the per-token maximum
 * given: sx[m] = fl(amax[m] / 127), q = clamp(rne(fl(fl(x/s)/sx)), -127, 127)
 * (q = 0 when sx = 0).  With amax[m] the row's own maximum this is exactly
 * w8a8_quantize_act.  amax: device fp32 [M], 4-byte aligned; a NaN,
 * negative or infinite entry (or a bad row index) gives sx = NaN and zero
 * codes.  With a finite maximum that does not bound the row, an element
 * whose quotient is NaN gets code 0 and an infinite one +-127.
 */
int w8a8_quantize_act_amax(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                           const float* smooth, const float* amax, int64_t M, int64_t K, int8_t* xq,
                           float* sx, void* stream);

/*
 * w8a8_gemm_int32 -- the exact int32 accumulators, no epilogue:
 *     acc[m,n] = sum_k xq[m,k] * w[n,k]            (row-major [M,N])
 * xq, w as for w8a8_gemm; acc device int32 [M,N], 16-byte aligned.
 */
int w8a8_gemm_int32(const int8_t* xq, const int8_t* w, int64_t M, int64_t N, int64_t K, int32_t* acc,
                    void* stream);

/*
 * w8a8_epilogue_int32 -- y = epilogue(P_0 + P_1 + ... + P_{S-1}) for S
 * int32 slices parts [S,M,N] (row-major, slice s at parts + s*M*N), added
 * in slice order, then the fixed epilogue of w8a8_gemm with sx [M], sw [N]
 * and the optional residual (may equal y).  The sum must fit int32, which
 * holds for the partials of one contraction with K <= W8A8_MAX_K.
 * 1 <= S <= W8A8_MAX_SPLITK; parts must not overlap y.
 */
int w8a8_epilogue_int32(const int32_t* parts, int S, const float* sx, const float* sw,
                        const float* residual, float* y, int64_t M, int64_t N, void* stream);

/*
 * w8a8_candidate_softmax -- the probabilities over each row's candidates.
 * The dsiab.com post, section "方案", normalises the candidate scores
 * within the candidate set (equal to the full-vocabulary softmax
 * renormalised over the candidates); the review page says the decision
 * model returns probabilities for the options.  One fixed sequence of
 * binary64 operations, identical on every run and for any batch:
 *     mx = max_c (double)logits[m,c];  e_c = exp(logits[m,c] - mx)
 *     S  = (((e_0 + e_1) + e_2) + ...) + e_{C-1}   (candidate order)
 *     probs[m,c] = e_c / S
 * exp is the library's own (Cody-Waite reduction, degree-13 Taylor
 * polynomial with fused multiply-adds); the relative error of a
 * probability is at most about (C + 6) binary64 units in the last place.
 * A row with a non-finite logit (NaN from a bad candidate id) gets NaN for
 * every candidate.
 *
 * logits   device fp32 [M,C], 4-byte aligned.
 * probs    device fp64 [M,C], 8-byte aligned, not overlapping logits.
 * C        0 <= C <= W8A8_MAX_CANDIDATES (else W8A8_ERR_TOO_MANY_CANDIDATES).
 */
int w8a8_candidate_softmax(const float* logits, int64_t M, int64_t C, double* probs, void* stream);

/*
 * w8a8_answer_head -- the answer read-out end to end on `stream`:
 * w8a8_quantize_act of the hidden rows answer_rows[0..M) of h (the answer
 * positions; review page, section "Compute shared evidence once"),
 * w8a8_readout_candidates on them, and w8a8_candidate_softmax.  For
 * K <= 18432 the three steps run as one kernel (one workgroup per answer
 * row); above it, as the three launches.  Every result is bit-identical to
 * calling those three entry points in turn with the same arguments.  All
 * arguments are checked before the first launch; a rejected call writes
 * nothing.
 *
 * h, ldh, h_rows   device fp32 hidden states [h_rows, ldh] (as x of
 *                  w8a8_quantize_act); answer_rows device int32 [M], required.
 * smooth, K        the lm_head's smoothing vector [K] (as in w8a8_quantize_act).
 * w_vocab, sw_vocab, V, cand, C, err_flag   as in w8a8_readout_candidates.
 * xq, sx           device scratch owned by the caller: int8 [M,K] (16-byte
 *                  aligned) and fp32 [M]; they hold the quantised rows after
 *                  the call.
 * logits           device fp32 [M,C]; probs device fp64 [M,C].
 */
int w8a8_answer_head(const float* h, int64_t ldh, int64_t h_rows, const int32_t* answer_rows,
                     int64_t M, const float* smooth, int64_t K, const int8_t* w_vocab,
                     const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C, int8_t* xq,
                     float* sx, float* logits, double* probs, int32_t* err_flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
