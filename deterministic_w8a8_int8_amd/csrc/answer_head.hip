// The answer head in one launch: gather the hidden row at an answer
// position, quantise it, score the candidate vocabulary rows and turn the
// scores into probabilities.
//
// The review page "StartLux-Prism: Fast, exact inference for
// StartLux-Decision models on NVIDIA GPUs", section "Compute shared evidence
// once", confines the read-out of the last layer to the answer positions;
// the dsiab.com post on moving decision models from vLLM to Prism, section
// "方案", scores only the candidate tokens and normalises among them.  Each
// step is the library's own definition, computed by the same device code as
// the separate entry points, so every result is bit-identical to calling
// w8a8_quantize_act (with row_idx), w8a8_readout_candidates and
// w8a8_candidate_softmax in turn:
//   - one workgroup per answer row holds the row in registers and quantises
//     it with quantize_rows_regs (the per-token quantisation of quantize.hip);
//   - a candidate logit is the exact int32 dot product of the row's codes
//     with the candidate's weight row (v_dot4_i32_i8, four int8 products and
//     an int32 addition, no saturation: K * 127^2 < 2^31 keeps every partial
//     sum exact), summed over the workgroup in int32 (exact, so the order
//     does not matter), then the fixed epilogue fl(fl(float(acc) * sx) * sw);
//   - an id outside [0, V) gives a quiet NaN logit and sets bit 0 of
//     err_flag, as the read-out does;
//   - wave 0 then runs candidate_softmax_wave (the softmax kernel's code) on
//     the logits.
// The weight rows of the first candidates are requested before the
// quantisation starts, so their latency overlaps the row's; the workgroup
// then walks the candidates in groups of AH_GROUP, each group's weights in
// flight while the previous group is reduced.
//
// The candidate scoring is also the candidate read-out itself
// (w8a8_readout_candidates for K <= 18432): readout_rows_kernel runs it on
// codes that are already quantised, one workgroup per row.
#include "device_common.h"
#include "launch.h"
#include "quantize_row.h"
#include "softmax_row.h"

namespace w8a8 {

namespace {

constexpr int AH_GROUP = 4;   // candidates whose weight rows are loaded together

// Candidate ids of one row: lane c of every wave holds id c (C <= 64); an id
// outside [0, V) reads row 0 and yields a NaN logit.
struct CandLane {
    int id;
    bool ok;
    float sw;   // the candidate's channel scale, requested early
};
__device__ __forceinline__ CandLane cand_lane(const int32_t* __restrict__ cand_row, int C, int64_t V,
                                              const float* __restrict__ sw, int lane) {
    const int id_raw = lane < C ? cand_row[lane] : 0;
    CandLane r;
    r.ok = id_raw >= 0 && id_raw < V;
    r.id = r.ok ? id_raw : 0;
    r.sw = lane < C ? sw[r.id] : 0.0f;
    return r;
}

// Weight words of candidates g0 .. g0 + AH_GROUP - 1: thread t's word i is
// word j = t + T*i of the row, the int8 weights of columns 4j .. 4j+3.
template <int NV, int T>
__device__ __forceinline__ void load_cand_group(uint32_t (&wv)[AH_GROUP][NV], const int8_t* __restrict__ w,
                                                int64_t K, int K4, int id_lane, int C, int g0, int t) {
#pragma unroll
    for (int c = 0; c < AH_GROUP; ++c) {
        const int id = __shfl(id_lane, min(g0 + c, 63), 64);
        const uint32_t* wr = reinterpret_cast<const uint32_t*>(w + static_cast<int64_t>(id) * K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            wv[c][i] = (j < K4 && g0 + c < C) ? wr[j] : 0u;
        }
    }
}

// The C candidate logits of one row from its codes (q[i] is word t + T*i of
// the row), AH_GROUP candidates at a time, each group's weight rows in flight
// while the previous group is reduced (wv holds group 0 on entry): exact
// int32 dot products (v_dot4_i32_i8, wave shuffles, per-wave partials through
// LDS), then the fixed epilogue.  Writes logits_row[c] and, when lg is not
// null, lg[c] (LDS); a bad id gives a quiet NaN and sets bit 0 of err_flag.
template <int NV, int T>
__device__ __forceinline__ void score_candidates(const uint32_t (&q)[NV], uint32_t (&wv)[AH_GROUP][NV],
                                                 const CandLane& cl, float sxm, const int8_t* __restrict__ w,
                                                 int64_t K, int K4, int C, int32_t (&part)[2][AH_GROUP][T / 64],
                                                 float* logits_row, float* lg, int32_t* err_flag, int t) {
    constexpr int NW = T / 64;
    const int lane = t & 63, wave = t >> 6;
    for (int g0 = 0, gi = 0; g0 < C; g0 += AH_GROUP, ++gi) {
        int32_t dot[AH_GROUP];
#pragma unroll
        for (int c = 0; c < AH_GROUP; ++c) {
            int32_t a = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                a = __builtin_amdgcn_sdot4(static_cast<int>(q[i]), static_cast<int>(wv[c][i]), a, false);
            dot[c] = a;
        }
        if (g0 + AH_GROUP < C) load_cand_group<NV, T>(wv, w, K, K4, cl.id, C, g0 + AH_GROUP, t);   // next group in flight
#pragma unroll
        for (int c = 0; c < AH_GROUP; ++c) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) dot[c] += __shfl_xor(dot[c], off, 64);
        }
        if (lane == 0) {
#pragma unroll
            for (int c = 0; c < AH_GROUP; ++c) part[gi & 1][c][wave] = dot[c];
        }
        // lane l < AH_GROUP of wave 0 finishes candidate g0 + l: its id and
        // validity, shuffled from lane g0 + l while every lane is active
        const int src_lane = min(g0 + (lane & (AH_GROUP - 1)), 63);
        const float swc = __shfl(cl.sw, src_lane, 64);
        const bool okc = __shfl(static_cast<int>(cl.ok), src_lane, 64) != 0;
        __syncthreads();
        if (wave == 0 && lane < AH_GROUP && g0 + lane < C) {
            int32_t acc = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) acc += part[gi & 1][lane][v];
            const int c = g0 + lane;
            const float l = okc ? scale_acc(acc, sxm, swc) : quiet_nan();
            if (lg) lg[c] = l;
            logits_row[c] = l;
            if (!okc && err_flag) atomicOr(err_flag, 1);
        }
    }
}

template <int NV, int T>
__global__ __launch_bounds__(T) void answer_head_kernel(
    const float* __restrict__ h, int64_t ldh, int64_t h_rows, const int32_t* __restrict__ rows,
    const float* __restrict__ smooth, int64_t K, const int8_t* __restrict__ w, const float* __restrict__ sw,
    int64_t V, const int32_t* __restrict__ cand, int C, int8_t* __restrict__ xq, float* __restrict__ sx,
    float* __restrict__ logits, double* __restrict__ probs, int32_t* __restrict__ err_flag) {
    constexpr int NW = T / 64;
    __shared__ float red[NW];
    __shared__ int32_t part[2][AH_GROUP][NW];
    __shared__ float lg[64];
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int K4 = static_cast<int>(K >> 2);

    const CandLane cl = cand_lane(cand + m * C, C, V, sw, lane);
    uint32_t wv[AH_GROUP][NV];
    if (C > 0) load_cand_group<NV, T>(wv, w, K, K4, cl.id, C, 0, t);

    // the answer row, quantised (bits of quantize_rows_reg); the smoothing
    // values stay in registers, so no exact path waits on memory
    int64_t src;
    const bool ok1[1] = {source_row(rows, m, h_rows, &src)};
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    float4 xv[1][NV];
    load_row<NV, T>(reinterpret_cast<const float4*>(h + src * ldh), K4, xv[0]);
    float4 rv[NV], sv[NV];
    bool odd_t;
    load_smoothing<NV, T, true>(s4, K4, rv, sv, odd_t);
    uint32_t q[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) q[i] = 0u;
    uint32_t* qr = reinterpret_cast<uint32_t*>(xq + m * K);
    const float no_max[1] = {0.0f};
    float scale1[1];
    bool valid1[1];
    quantize_rows_regs<NV, T, 1, false>(
        xv, [&](int i) __attribute__((always_inline)) { return rv[i]; },
        [&](int i, int) __attribute__((always_inline)) { return sv[i]; }, odd_t, K4, ok1, no_max, red,
        [&](int, int i, uint32_t packed) __attribute__((always_inline)) {
            q[i] = packed;   // kept for the candidate dot products
            qr[t + i * T] = packed;
        },
        scale1, valid1);
    const float scale = scale1[0];
    const bool valid = valid1[0];
    const float sxm = valid ? scale : quiet_nan();
    if (t == 0) sx[m] = sxm;

    // candidate logits
    score_candidates<NV, T>(q, wv, cl, sxm, w, K, K4, C, part, logits + m * C, lg, err_flag, t);
    __syncthreads();
    if (wave == 0 && C > 0) {
        const bool live = lane < C;
        const double p = candidate_softmax_wave(live ? lg[lane] : 0.0f, live, C);
        if (live) probs[m * C + lane] = p;
    }
}

// The candidate read-out on given codes: one workgroup per row loads the
// row's codes and its first candidates' weight rows together, then scores
// the candidates with the answer head's code.
template <int NV, int T>
__global__ __launch_bounds__(T) void readout_rows_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int64_t K, const int8_t* __restrict__ w,
    const float* __restrict__ sw, int64_t V, const int32_t* __restrict__ cand, int C,
    float* __restrict__ logits, int32_t* __restrict__ err_flag) {
    __shared__ int32_t part[2][AH_GROUP][T / 64];
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63;
    const int K4 = static_cast<int>(K >> 2);
    const CandLane cl = cand_lane(cand + m * C, C, V, sw, lane);
    uint32_t wv[AH_GROUP][NV];
    load_cand_group<NV, T>(wv, w, K, K4, cl.id, C, 0, t);
    const uint32_t* qr = reinterpret_cast<const uint32_t*>(xq + m * K);
    uint32_t q[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * T;
        q[i] = j < K4 ? qr[j] : 0u;
    }
    score_candidates<NV, T>(q, wv, cl, sx[m], w, K, K4, C, part, logits + m * C, nullptr, err_flag, t);
}

template <int NV, int T>
hipError_t launch_rr(const ReadoutRowsArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((readout_rows_kernel<NV, T>), dim3(static_cast<unsigned>(a.M)), dim3(T), 0, stream, a.xq,
                       a.sx, a.K, a.w, a.sw, a.V, a.cand, static_cast<int>(a.C), a.logits, a.err_flag);
    return hipGetLastError();
}

template <int NV, int T>
hipError_t launch_t(const AnswerHeadArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((answer_head_kernel<NV, T>), dim3(static_cast<unsigned>(a.M)), dim3(T), 0, stream, a.h,
                       a.ldh, a.h_rows, a.rows, a.smooth, a.K, a.w, a.sw, a.V, a.cand, static_cast<int>(a.C),
                       a.xq, a.sx, a.logits, a.probs, a.err_flag);
    return hipGetLastError();
}

}  // namespace

bool answer_head_fused_fits(int64_t K) { return K <= 18432; }

hipError_t launch_answer_head(const AnswerHeadArgs& a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    const int64_t n256 = (a.K + 1023) / 1024;   // float4 per thread with 256 threads
    const int64_t n512 = (a.K + 2047) / 2048;   // ... with 512 threads
    // Past K = 2048 a row is split over 512 threads: the head is a chain of
    // dependent phases (load, reduce, quantise, dot, reduce, softmax) on one
    // workgroup per row, and halving each thread's share shortens every
    // phase (K = 5120: 6.5 against 7.9 us back to back; 1024 threads: 6.7).
    if (n256 <= 1) return launch_t<1, 256>(a, stream);
    if (n256 <= 2) return launch_t<2, 256>(a, stream);
    if (n512 <= 2) return launch_t<2, 512>(a, stream);
    if (n512 <= 3) return launch_t<3, 512>(a, stream);
    if (n512 <= 4) return launch_t<4, 512>(a, stream);
    if (n512 <= 5) return launch_t<5, 512>(a, stream);
    if (n512 <= 6) return launch_t<6, 512>(a, stream);
    if (n512 <= 8) return launch_t<8, 512>(a, stream);
    if (n512 <= 9) return launch_t<9, 512>(a, stream);
    return hipErrorInvalidValue;
}

// The same shapes as the answer head: 256 threads per row up to K = 2048,
// 512 above, up to K = 18432.
hipError_t launch_readout_rows(const ReadoutRowsArgs& a, hipStream_t stream) {
    if (a.M == 0 || a.C == 0) return hipSuccess;
    const int64_t n256 = (a.K + 1023) / 1024;
    const int64_t n512 = (a.K + 2047) / 2048;
    if (n256 <= 1) return launch_rr<1, 256>(a, stream);
    if (n256 <= 2) return launch_rr<2, 256>(a, stream);
    if (n512 <= 2) return launch_rr<2, 512>(a, stream);
    if (n512 <= 3) return launch_rr<3, 512>(a, stream);
    if (n512 <= 4) return launch_rr<4, 512>(a, stream);
    if (n512 <= 5) return launch_rr<5, 512>(a, stream);
    if (n512 <= 6) return launch_rr<6, 512>(a, stream);
    if (n512 <= 8) return launch_rr<8, 512>(a, stream);
    if (n512 <= 9) return launch_rr<9, 512>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace w8a8
