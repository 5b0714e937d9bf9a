/*
 * CPU oracle for the deterministic W8A8 int8 linear layer and the
 * candidate-only lm_head read-out.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg load this file's library.  The GPU
 * product path never calls it, links it or shares code with it.
 *
 * What is computed comes from the StartLux-Prism review page ("StartLux-Prism:
 * Fast, exact inference for StartLux-Decision models on NVIDIA GPUs"):
 *   - section "Compute shared evidence once": Q8_0 weights are requantised
 *     with SmoothQuant and activations are quantised per token for W8A8
 *     execution;
 *   - section "Bitwise consistency is not lossless quantization": the int8
 *     products accumulate exactly in int32, are then scaled and added to the
 *     residual with a fixed rounding sequence, split-K partial sums stay
 *     integers, and the scaling, addition and read-out paths are fixed;
 *   - section "Compute shared evidence once": in the last layer the read-out
 *     is limited to the answer positions;
 * and from the dsiab.com post on moving decision models from vLLM to Prism,
 * section "方案" (the approach): only the candidate tokens are scored, which
 * equals a full-vocabulary softmax renormalised over the candidates.
 *
 * Where those pages leave a step open, the plainest reading is taken:
 *   smoothing is a true IEEE division x/s (not a multiply by 1/s);
 *   the range is symmetric [-127, 127];
 *   the per-token scale is sx = fl(amax/127) and q = rne(fl(x'/sx));
 *   rounding is round-half-to-even;
 *   a row whose sx is 0 (all zero, or amax/127 underflowing) quantises to 0;
 *   a row whose smoothed values include a NaN or an infinity (from the
 *   input, or from x/s overflowing) has no finite maximum and no scale: it
 *   gets sx = NaN and all codes 0, as a row that cannot be read;
 *   the epilogue is y = fl(fl(fl((float)acc * sx) * sw) + r), left to right,
 *   with no fused multiply-add anywhere.
 *
 * Arithmetic: scalar loops, int64 accumulation, binary32 for the epilogue.
 * Build with -O2 -ffp-contract=off -fno-fast-math so that the compiler keeps
 * every binary32 operation separate and correctly rounded.  Rows are spread
 * over OpenMP threads; each output element is computed by exactly one thread
 * in the same scalar order, so the thread count never changes a bit.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_OVERFLOW (-2)

/* |acc| must stay below 2^31 for int32 accumulation to be exact. */
static const int64_t ORACLE_INT32_MAX = 2147483647LL;

/* Absolute value for the row maximum, with NaN taken as +infinity, so that a
 * row holding any non-finite smoothed value has an infinite maximum. */
static float oracle_abs_for_max(float v) {
    float a = fabsf(v);
    if (a != a) return INFINITY;
    return a;
}

/* A per-token maximum that yields a scale: not NaN, not negative, finite. */
static int oracle_usable_max(float a) { return a >= 0.0f && a <= FLT_MAX; }

/* Round the quotient t = fl(x'/sx) to a code: round half to even, clamp to
 * [-127, 127].  A NaN quotient (only possible when a given maximum does not
 * bound the row) gives 0; an infinite one clamps. */
static int8_t oracle_code(float t);

/* Round half to even, written out: floor, then compare the fraction with 1/2.
 * For |t| < 2^23 the subtraction t - floor(t) is exact in binary32. */
static float oracle_round_half_even(float t) {
    float f = floorf(t);
    float d = t - f;
    if (d > 0.5f) return f + 1.0f;
    if (d < 0.5f) return f;
    /* exact tie: pick the even neighbour */
    return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

static int8_t oracle_code(float t) {
    if (t != t) return 0;
    if (t >= 127.0f) return 127;
    if (t <= -127.0f) return -127;
    float r = oracle_round_half_even(t);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)(int)r;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (the results never depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Per-token quantisation after the SmoothQuant per-channel divide.
 *   x        fp32, row r starts at x + r*ldx
 *   row_idx  optional [M]: output row m reads input row row_idx[m]
 *   smooth   fp32 [K], > 0
 *   xq       int8 [M,K] row-major, sx fp32 [M]
 */
int oracle_quantize_act(const float* x, int64_t ldx, const int32_t* row_idx,
                        const float* smooth, int64_t M, int64_t K,
                        int8_t* xq, float* sx) {
    if (!x || !smooth || !xq || !sx || M < 0 || K <= 0 || ldx < K) return ORACLE_ERR_ARG;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const int64_t src = row_idx ? (int64_t)row_idx[m] : m;
        const float* xr = x + src * ldx;
        /* step 1+2: smoothed value and its absolute maximum */
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float xs = xr[k] / smooth[k];
            float ab = oracle_abs_for_max(xs);
            if (ab > amax) amax = ab;
        }
        /* a non-finite smoothed value: no scale, all codes 0 */
        if (!oracle_usable_max(amax)) {
            sx[m] = NAN;
            for (int64_t k = 0; k < K; ++k) xq[m * K + k] = 0;
            continue;
        }
        /* step 3: per-token scale */
        float s = amax / 127.0f;
        sx[m] = s;
        /* step 4: quantise */
        for (int64_t k = 0; k < K; ++k) {
            int8_t q = 0;
            if (s != 0.0f) {
                float xs = xr[k] / smooth[k];
                float t = xs / s;
                q = oracle_code(t);
            }
            xq[m * K + k] = q;
        }
    }
    return ORACLE_OK;
}

/* Tensor-parallel row-parallel layers (review page, section "Bitwise
 * consistency is not lossless quantization": tensor parallelism combines
 * integer partial sums before scaling).  A rank holds a K-slice of the
 * activations.  For the integer partials of the ranks to be added before
 * scaling they must share one per-token scale, so the plainest reading is:
 * each rank takes the maximum of its smoothed slice, the maxima are combined
 * by an exact MAX across ranks, and every rank quantises its slice with the
 * token scale of that global maximum.  The two steps of oracle_quantize_act
 * are therefore also given separately. */

/* Steps 1+2 only: amax[m] = max_k |fl(x[m,k] / smooth[k])| over this slice;
 * +infinity when the slice holds a NaN or infinite smoothed value. */
int oracle_row_absmax(const float* x, int64_t ldx, const int32_t* row_idx,
                      const float* smooth, int64_t M, int64_t K, float* amax_out) {
    if (!x || !smooth || !amax_out || M < 0 || K <= 0 || ldx < K) return ORACLE_ERR_ARG;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const int64_t src = row_idx ? (int64_t)row_idx[m] : m;
        const float* xr = x + src * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float ab = oracle_abs_for_max(xr[k] / smooth[k]);
            if (ab > amax) amax = ab;
        }
        amax_out[m] = amax;
    }
    return ORACLE_OK;
}

/* Steps 3+4 with a given per-token maximum (the global one): sx = fl(amax/127)
 * and q = clamp(rne(fl(fl(x/s)/sx)), -127, 127), q = 0 when sx = 0.  A given
 * maximum that is NaN, negative or infinite has no scale: sx = NaN and all
 * codes 0. */
int oracle_quantize_act_amax(const float* x, int64_t ldx, const int32_t* row_idx,
                             const float* smooth, const float* amax_in, int64_t M, int64_t K,
                             int8_t* xq, float* sx) {
    if (!x || !smooth || !amax_in || !xq || !sx || M < 0 || K <= 0 || ldx < K) return ORACLE_ERR_ARG;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const int64_t src = row_idx ? (int64_t)row_idx[m] : m;
        const float* xr = x + src * ldx;
        if (!oracle_usable_max(amax_in[m])) {
            sx[m] = NAN;
            for (int64_t k = 0; k < K; ++k) xq[m * K + k] = 0;
            continue;
        }
        float s = amax_in[m] / 127.0f;
        sx[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int8_t q = 0;
            if (s != 0.0f) {
                float xs = xr[k] / smooth[k];
                float t = xs / s;
                q = oracle_code(t);
            }
            xq[m * K + k] = q;
        }
    }
    return ORACLE_OK;
}

/* Split-K chunk c of S: [c*Kc, min((c+1)*Kc, K)) with Kc = ceil(K/S) rounded
 * up to a multiple of ktile. */
static void oracle_chunk(int64_t K, int splitk, int64_t ktile, int c, int64_t* k0, int64_t* k1) {
    int64_t kc = (K + splitk - 1) / splitk;
    kc = ((kc + ktile - 1) / ktile) * ktile;
    int64_t a = (int64_t)c * kc, b = a + kc;
    if (a > K) a = K;
    if (b > K) b = K;
    *k0 = a;
    *k1 = b;
}

/* Exact integer dot product of one activation row with one weight row,
 * accumulated chunk by chunk in the fixed order c = 0..S-1.  Each partial and
 * the total are checked against the int32 range.  Returns 0 or an error. */
static int oracle_dot(const int8_t* a, const int8_t* b, int64_t K, int splitk, int64_t ktile,
                      int64_t* out) {
    int64_t acc = 0;
    for (int c = 0; c < splitk; ++c) {
        int64_t k0, k1;
        oracle_chunk(K, splitk, ktile, c, &k0, &k1);
        int64_t part = 0;
        for (int64_t k = k0; k < k1; ++k) part += (int64_t)a[k] * (int64_t)b[k];
        if (part > ORACLE_INT32_MAX || part < -ORACLE_INT32_MAX) return ORACLE_ERR_OVERFLOW;
        acc += part;
    }
    if (acc > ORACLE_INT32_MAX || acc < -ORACLE_INT32_MAX) return ORACLE_ERR_OVERFLOW;
    *out = acc;
    return ORACLE_OK;
}

/* The fixed-order epilogue: convert, scale by the token, scale by the
 * channel, add the residual.  Each line is one correctly rounded binary32
 * operation. */
static float oracle_epilogue(int64_t acc, float sxm, float swn, const float* r) {
    float t0 = (float)(int32_t)acc;
    float t1 = t0 * sxm;
    float t2 = t1 * swn;
    if (!r) return t2;
    float y = t2 + *r;
    return y;
}

/* y[m,n] = epilogue(sum_k xq[m,k]*w[n,k]) over all M x N outputs.
 * residual may be NULL or equal to y. */
int oracle_gemm(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                const float* residual, float* y, int64_t M, int64_t N, int64_t K,
                int splitk, int64_t ktile) {
    if (!xq || !sx || !w || !sw || !y || M < 0 || N < 0 || K <= 0 || splitk < 1 || ktile < 1)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    int64_t m;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc;
            if (oracle_dot(xq + m * K, w + n * K, K, splitk, ktile, &acc) != ORACLE_OK) {
#pragma omp atomic write
                err = ORACLE_ERR_OVERFLOW;
                acc = 0;
            }
            y[m * N + n] = oracle_epilogue(acc, sx[m], sw[n], residual ? residual + m * N + n : 0);
        }
    }
    return err;
}

/* Same definition at P sampled points (mi[p], ni[p]); out[p] = y[mi, ni].
 * residual, if given, is the full [M,N] array. */
int oracle_gemm_sampled(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                        const float* residual, int64_t M, int64_t N, int64_t K, int splitk,
                        int64_t ktile, const int64_t* mi, const int64_t* ni, int64_t P, float* out) {
    if (!xq || !sx || !w || !sw || !mi || !ni || !out || K <= 0 || splitk < 1) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    int64_t p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
        int64_t m = mi[p], n = ni[p];
        if (m < 0 || m >= M || n < 0 || n >= N) {
#pragma omp atomic write
            err = ORACLE_ERR_ARG;
            out[p] = 0.0f;
            continue;
        }
        int64_t acc;
        if (oracle_dot(xq + m * K, w + n * K, K, splitk, ktile, &acc) != ORACLE_OK) {
#pragma omp atomic write
            err = ORACLE_ERR_OVERFLOW;
            acc = 0;
        }
        out[p] = oracle_epilogue(acc, sx[m], sw[n], residual ? residual + m * N + n : 0);
    }
    return err;
}

/* Exact int32 accumulators (no epilogue) for an [M,N] block; used by the
 * tests that check the integer stage on its own. */
int oracle_gemm_acc(const int8_t* xq, const int8_t* w, int64_t M, int64_t N, int64_t K,
                    int splitk, int64_t ktile, int64_t* acc_out) {
    if (!xq || !w || !acc_out || K <= 0 || splitk < 1) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            if (oracle_dot(xq + m * K, w + n * K, K, splitk, ktile, &acc) != ORACLE_OK) {
#pragma omp atomic write
                err = ORACLE_ERR_OVERFLOW;
            }
            acc_out[m * N + n] = acc;
        }
    }
    return err;
}

/* Startup requantisation of Q8_0 weights with SmoothQuant (review page,
 * section "Compute shared evidence once": the Q8_0 weights are requantised
 * with SmoothQuant at startup).  Q8_0 keeps blocks of 32 int8 codes along a
 * weight row with one binary16 scale each: w = d * q.  SmoothQuant moves the
 * activations' per-channel scale into the weights, x' = x / s and
 * w' = w * s, so x'.w'^T = x.w^T.  The pages give neither the calibration of
 * s nor the order of the operations; the plainest reading, with s given:
 *   w'[n,k] = fl(fl(d[n, k/32] * q[n,k]) * s[k])   (d*q is exact in binary32)
 *   sw[n]   = fl(max_k |w'[n,k]| / 127)
 *   wq[n,k] = clamp(rne(fl(w'[n,k] / sw[n])), -127, 127), 0 when sw[n] = 0
 * i.e. the same symmetric round-half-even rule as the activations, per
 * output channel.  d is given as binary16 bit patterns.  A row whose w'
 * holds a NaN or an infinity (a non-finite d or s, or an overflow) has no
 * scale: sw[n] = NaN and all its codes 0, the activations' rule for a row
 * that cannot be quantised (the pages say nothing of such inputs). */
static float oracle_f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    float v;
    if (e == 0) v = ldexpf((float)f, -24);                    /* subnormal or zero */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexpf((float)(f | 1024), e - 25);
    return sign ? -v : v;
}

int oracle_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N,
                           int64_t K, int8_t* wq, float* sw) {
    if (!q || !d || !smooth || !wq || !sw || N < 0 || K <= 0 || (K % 32) != 0) return ORACLE_ERR_ARG;
    const int64_t nb = K / 32;
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        float amax = 0.0f;
        int finite = 1;
        for (int64_t k = 0; k < K; ++k) {
            float w = oracle_f16_to_f32(d[n * nb + k / 32]) * (float)q[n * K + k];
            float ws = w * smooth[k];
            float ab = fabsf(ws);
            if (!isfinite(ws)) finite = 0;
            if (ab > amax) amax = ab;
        }
        if (!finite) {
            sw[n] = NAN;
            for (int64_t k = 0; k < K; ++k) wq[n * K + k] = 0;
            continue;
        }
        float s = amax / 127.0f;
        sw[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            int8_t c = 0;
            if (s != 0.0f) {
                float w = oracle_f16_to_f32(d[n * nb + k / 32]) * (float)q[n * K + k];
                float ws = w * smooth[k];
                float t = ws / s;
                float r = oracle_round_half_even(t);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                c = (int8_t)(int)r;
            }
            wq[n * K + k] = c;
        }
    }
    return ORACLE_OK;
}

/* The epilogue of given exact accumulators (the integer partials of the
 * ranks already added): y[m,n] = epilogue(acc[m,n]).  An accumulator outside
 * the int32 range is an error. */
int oracle_epilogue_acc(const int64_t* acc, const float* sx, const float* sw,
                        const float* residual, float* y, int64_t M, int64_t N) {
    if (!acc || !sx || !sw || !y || M < 0 || N < 0) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const int64_t a = acc[m * N + n];
            if (a > ORACLE_INT32_MAX || a < -ORACLE_INT32_MAX) err = ORACLE_ERR_OVERFLOW;
            y[m * N + n] = oracle_epilogue(a, sx[m], sw[n], residual ? residual + m * N + n : 0);
        }
    }
    return err;
}

/* Candidate-only read-out: logits[m,c] is the epilogue (no residual) of the
 * exact dot of row m with vocabulary row cand[m,c].  An id outside [0,V)
 * gives a quiet NaN and bit 0 of *err_flag. */
int oracle_readout_candidates(const int8_t* xq, const float* sx, int64_t M, int64_t K,
                              const int8_t* w_vocab, const float* sw_vocab, int64_t V,
                              const int32_t* cand, int64_t C, float* logits, int32_t* err_flag) {
    if (!xq || !sx || !w_vocab || !sw_vocab || !cand || !logits || M < 0 || K <= 0 || V <= 0 || C < 0)
        return ORACLE_ERR_ARG;
    int32_t flag = 0;
    int err = ORACLE_OK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < C; ++c) {
            int64_t id = cand[m * C + c];
            if (id < 0 || id >= V) {
                logits[m * C + c] = nanf("");
                flag |= 1;
                continue;
            }
            int64_t acc;
            if (oracle_dot(xq + m * K, w_vocab + id * K, K, 1, K, &acc) != ORACLE_OK) {
                err = ORACLE_ERR_OVERFLOW;
                acc = 0;
            }
            logits[m * C + c] = oracle_epilogue(acc, sx[m], sw_vocab[id], 0);
        }
    }
    if (err_flag) *err_flag |= flag;
    return err;
}
