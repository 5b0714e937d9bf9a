/*
 * The library used from plain C, with nothing but include/w8a8.h and the
 * HIP runtime: the startup requantisation of Q8_0 weights, one linear layer
 * on them (per-token quantisation, GEMM with residual, the same GEMM at
 * split-K 3) and the candidate read-out of three rows, each output compared
 * bit for bit with the CPU oracle (linked in as test infrastructure; the
 * library itself never uses it).  Exit status 0 when every output matches,
 * 1 on a mismatch, 2 on an error.
 *
 * The definitions checked are those of the review page "StartLux-Prism:
 * Fast, exact inference for StartLux-Decision models on NVIDIA GPUs",
 * sections "Compute shared evidence once" (Q8_0 weights requantised with
 * SmoothQuant at startup; per-token quantisation after the smoothing divide;
 * read-out at the answer positions) and "Bitwise
 * consistency is not lossless quantization" (exact int32 accumulation,
 * integer split-K partials, one fixed rounding sequence).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "w8a8.h"

/* the oracle's entry points (oracle/w8a8_oracle.c) */
int oracle_quantize_act(const float* x, int64_t ldx, const int32_t* row_idx, const float* smooth, int64_t M,
                        int64_t K, int8_t* xq, float* sx);
int oracle_gemm(const int8_t* xq, const float* sx, const int8_t* w, const float* sw, const float* residual,
                float* y, int64_t M, int64_t N, int64_t K, int splitk, int64_t ktile);
int oracle_readout_candidates(const int8_t* xq, const float* sx, int64_t M, int64_t K, const int8_t* w_vocab,
                              const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C, float* logits,
                              int32_t* err_flag);
int oracle_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N, int64_t K,
                           int8_t* wq, float* sw);

enum { M = 37, N = 300, K = 704, SPLITK = 3, RM = 3, C = 5 };

static uint64_t lcg_state = 12345u;
static uint32_t lcg(void) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 33);
}
static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)(lcg() % 1000000u) / 1000000.0f; }

#define HIP_OK(call)                                                             \
    do {                                                                         \
        if ((call) != hipSuccess) {                                              \
            fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);         \
            return 2;                                                            \
        }                                                                        \
    } while (0)
#define LIB_OK(call)                                                                           \
    do {                                                                                       \
        const int st_ = (call);                                                                \
        if (st_ != W8A8_OK) {                                                                  \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, w8a8_status_string(st_));       \
            return 2;                                                                          \
        }                                                                                      \
    } while (0)

static int same(const void* a, const void* b, size_t bytes, const char* what) {
    if (memcmp(a, b, bytes) == 0) return 1;
    fprintf(stderr, "%s differs from the oracle\n", what);
    return 0;
}

/* binary16 bit pattern of v for 2^-14 <= v < 2^15 (normal range, rounded toward zero) */
static uint16_t f16_bits(float v) {
    int e = 0;
    float f = v;
    while (f >= 2.0f) { f *= 0.5f; ++e; }
    while (f < 1.0f) { f *= 2.0f; --e; }
    return (uint16_t)(((e + 15) << 10) | (int)((f - 1.0f) * 1024.0f));
}

int main(void) {
    static float x[M * K], smooth[K], sw[N], r[M * N], y[M * N], y3[M * N], sx[M], logits[RM * C];
    static int8_t w[N * K], xq[M * K], q8[N * K], o_w[N * K];
    static uint16_t d8[N * (K / 32)];
    static float o_sw[N];
    static int32_t cand[RM * C];
    static float o_sx[M], o_y[M * N], o_logits[RM * C];
    static int8_t o_xq[M * K];
    for (int i = 0; i < M * K; ++i) x[i] = uniform(-1.0f, 1.0f);
    for (int m = 0; m < M; ++m) x[m * K + (int)(lcg() % K)] *= 30.0f;   /* an outlier channel per row */
    for (int k = 0; k < K; ++k) smooth[k] = uniform(0.5f, 4.0f);
    /* Q8_0 weights: codes and binary16 block scales, requantised below with the smoothing vector */
    for (int i = 0; i < N * K; ++i) q8[i] = (int8_t)((int)(lcg() % 255u) - 127);
    for (int i = 0; i < N * (K / 32); ++i) d8[i] = f16_bits(uniform(1e-3f, 1e-2f));
    for (int i = 0; i < M * N; ++i) r[i] = uniform(-2.0f, 2.0f);
    for (int i = 0; i < RM * C; ++i) cand[i] = (int32_t)(lcg() % N);

    float *d_x, *d_smooth, *d_sw, *d_r, *d_y, *d_y3, *d_sx, *d_logits;
    int8_t *d_w, *d_xq;
    int32_t *d_cand, *d_flag;
    uint16_t* d_d8;
    void* d_ws = NULL;
    HIP_OK(hipMalloc((void**)&d_x, sizeof x));
    HIP_OK(hipMalloc((void**)&d_smooth, sizeof smooth));
    HIP_OK(hipMalloc((void**)&d_sw, sizeof sw));
    HIP_OK(hipMalloc((void**)&d_r, sizeof r));
    HIP_OK(hipMalloc((void**)&d_y, sizeof y));
    HIP_OK(hipMalloc((void**)&d_y3, sizeof y3));
    HIP_OK(hipMalloc((void**)&d_sx, sizeof sx));
    HIP_OK(hipMalloc((void**)&d_logits, sizeof logits));
    HIP_OK(hipMalloc((void**)&d_w, sizeof w));
    HIP_OK(hipMalloc((void**)&d_xq, sizeof xq));
    HIP_OK(hipMalloc((void**)&d_cand, sizeof cand));
    HIP_OK(hipMalloc((void**)&d_flag, sizeof(int32_t)));
    HIP_OK(hipMalloc((void**)&d_d8, sizeof d8));
    HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_smooth, smooth, sizeof smooth, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_r, r, sizeof r, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, q8, sizeof q8, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_d8, d8, sizeof d8, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cand, cand, sizeof cand, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_flag, 0, sizeof(int32_t)));

    /* startup: the Q8_0 codes requantised in place into the layer's weights and channel scales */
    LIB_OK(w8a8_requantize_q8_0(d_w, d_d8, d_smooth, N, K, d_w, d_sw, NULL));
    /* the layer: quantise, GEMM with residual, the same at split-K 3 */
    LIB_OK(w8a8_quantize_act(d_x, K, M, NULL, d_smooth, M, K, d_xq, d_sx, NULL));
    LIB_OK(w8a8_gemm(d_xq, d_sx, d_w, d_sw, d_r, d_y, M, N, K, NULL));
    const size_t ws_bytes = w8a8_gemm_splitk_workspace_bytes(M, N, K, SPLITK);
    if (ws_bytes == (size_t)-1) return 2;
    if (ws_bytes) HIP_OK(hipMalloc(&d_ws, ws_bytes));
    LIB_OK(w8a8_gemm_splitk(d_xq, d_sx, d_w, d_sw, d_r, d_y3, M, N, K, SPLITK, d_ws, ws_bytes, NULL));
    /* the candidate read-out of the first RM rows, the weight rows as a vocabulary */
    LIB_OK(w8a8_readout_candidates(d_xq, d_sx, RM, K, d_w, d_sw, N, d_cand, C, d_logits, d_flag, NULL));
    HIP_OK(hipDeviceSynchronize());

    int32_t flag = -1;
    HIP_OK(hipMemcpy(xq, d_xq, sizeof xq, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sx, d_sx, sizeof sx, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, d_y, sizeof y, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y3, d_y3, sizeof y3, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(logits, d_logits, sizeof logits, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&flag, d_flag, sizeof flag, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(w, d_w, sizeof w, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(sw, d_sw, sizeof sw, hipMemcpyDeviceToHost));

    int32_t o_flag = 0;
    if (oracle_requantize_q8_0(q8, d8, smooth, N, K, o_w, o_sw) != 0) return 2;
    if (oracle_quantize_act(x, K, NULL, smooth, M, K, o_xq, o_sx) != 0) return 2;
    if (oracle_gemm(o_xq, o_sx, o_w, o_sw, r, o_y, M, N, K, 1, 64) != 0) return 2;
    if (oracle_readout_candidates(o_xq, o_sx, RM, K, o_w, o_sw, N, cand, C, o_logits, &o_flag) != 0) return 2;

    int ok = same(w, o_w, sizeof w, "requantised weights") & same(sw, o_sw, sizeof sw, "channel scales") &
             same(xq, o_xq, sizeof xq, "codes") & same(sx, o_sx, sizeof sx, "token scales") &
             same(y, o_y, sizeof y, "gemm") & same(y3, o_y, sizeof y3, "gemm split-K 3") &
             same(logits, o_logits, sizeof logits, "candidate logits");
    if (flag != o_flag) {
        fprintf(stderr, "err_flag %d, oracle %d\n", flag, o_flag);
        ok = 0;
    }
    void* bufs[] = {d_ws, d_x, d_smooth, d_sw, d_r, d_y, d_y3, d_sx, d_logits, d_w, d_xq, d_cand, d_flag, d_d8};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    if (!ok) return 1;
    printf("c-abi: requantize_q8_0, quantise, gemm, gemm_splitk(%d), readout_candidates bit-exact against the "
           "oracle\n", SPLITK);
    return 0;
}
