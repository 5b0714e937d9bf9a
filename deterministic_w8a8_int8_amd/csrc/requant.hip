// Startup requantisation of Q8_0 weights with SmoothQuant.
//
// The review page "StartLux-Prism: Fast, exact inference for
// StartLux-Decision models on NVIDIA GPUs", section "Compute shared evidence
// once", requantises the released Q8_0 weights with SmoothQuant at startup,
// for W8A8 execution.  Q8_0 keeps blocks of 32 int8 codes along a weight row
// with one binary16 scale each (w = d * q); SmoothQuant multiplies weight
// column k by the smoothing value s_k that divides activation channel k.
// Per output channel n, one rounding per step:
//   w'[n,k] = fl(fl(d[n, k/32] * q[n,k]) * s[k])     (d*q exact in binary32)
//   sw[n]   = fl(max_k |w'[n,k]| / 127)
//   wq[n,k] = clamp(rne(fl(w'[n,k] / sw[n])), -127, 127), 0 when sw[n] = 0
// the same symmetric round-half-even rule as the activations; a row whose w'
// holds a NaN or an infinity gets sw[n] = NaN and all codes 0, as an
// activation row that cannot be quantised does.  The row maximum propagates
// NaNs (v_maximum3_f32, no more instructions than a plain maximum), so such a
// row shows as a maximum that is not finite.
//
// Design.  A one-off pass moving 2 bytes per weight (1 read, 1 written) plus
// 2 bytes of block scale per 32; the smoothing vector is shared by all rows
// and stays in cache.  What limits it is vector ALU work, about 10
// instructions per weight, most of them in the division; so the division
// goes through the row's reciprocal, exactly (code_of below).  Work is cut
// into 16-column chunks: one 16-byte load of codes, four float4 of
// smoothing values, one block scale (16 columns never straddle a 32-column
// block).
//  * Rows of up to 24576 columns: each lane holds its chunks of the row in
//    registers -- all loads issued before the first is used, every wave load
//    covering 1 KB of the row -- and keeps w' there from pass 1 (the exact
//    maximum: max is exact, order free) to pass 2 (the codes), so a row
//    costs one trip to memory.  Up to 6144 columns one wave takes a row, four
//    rows per workgroup, no barrier; longer rows are split over the four
//    waves of a workgroup, the maximum combined through LDS.
//  * Longer rows: one 256-thread workgroup per row, 16 columns per thread at
//    a time; pass 2 re-reads the codes (from L2).
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int RQ_THREADS = 256;   // both kernels: four waves
constexpr int RQ_WAVES = RQ_THREADS / 64;
constexpr int RQ_MAX_CPL = 6;     // chunks per lane kept in registers (16 floats of w' each)

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));   // exact widening
}

__device__ __forceinline__ float4 smoothed4(uint32_t q4, float d, float4 s) {
    // d * q is exact in binary32 (11 + 8 significant bits); then one rounding
    const float w0 = d * static_cast<float>(static_cast<int8_t>(q4 & 255u));
    const float w1 = d * static_cast<float>(static_cast<int8_t>((q4 >> 8) & 255u));
    const float w2 = d * static_cast<float>(static_cast<int8_t>((q4 >> 16) & 255u));
    const float w3 = d * static_cast<float>(static_cast<int8_t>(q4 >> 24));
    return make_float4(w0 * s.x, w1 * s.y, w2 * s.z, w3 * s.w);
}

// Maximum that propagates NaN (IEEE maximum; one v_maximum3_f32 takes two
// of them with the absolute values).
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float abs_nmax4(float m, float4 w) {
    const float t = nmax(nmax(m, fabsf(w.x)), fabsf(w.y));
    return nmax(nmax(t, fabsf(w.z)), fabsf(w.w));
}

__device__ __forceinline__ float wave_nmax(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = nmax(v, __shfl_xor(v, off, 64));
    return v;
}

// The channel scale of a row maximum m: fl(m / 127), or a NaN (no scale)
// when m is not finite.
__device__ __forceinline__ float channel_scale(float m) {
    return m <= 0x1.fffffep127f ? m / 127.0f : __builtin_nanf("");
}

// The reciprocal that code_of divides by: fl(1 / sc) for sc in [2^-120,
// 2^120], where it and every product w * (1/sc) (|w| <= 127.00001 sc) stay
// normal; a NaN otherwise, which sends every value to the true division.
__device__ __forceinline__ float recip_or_nan(float sc) {
    return (sc >= 0x1p-120f && sc <= 0x1p120f) ? 1.0f / sc : __builtin_nanf("");
}

// rne(fl(w / sc)) clamped to [-127, 127] for |w| <= max|w| = 127 sc (1 +
// 2^-24 at most), with inv = recip_or_nan(sc).  Let t = fl(w * inv): then
// |t - w/sc| <= 1.5 * 2^-23 |w/sc| (two roundings) and |fl(w/sc) - w/sc| <=
// 2^-24 |w/sc|, so t and fl(w/sc) differ by less than 3.1e-5.  When t lies
// more than 2^-12 from every half-integer, both round to the same integer r,
// and |r| <= 127 without clamping.  Otherwise -- a few values in 10^4, every
// NaN (its comparison fails) and every value when inv is a NaN -- the true
// division decides.  The branch is taken by the whole wave when any lane
// needs it (a ballot), so it jumps over the division rather than selecting
// after it, and is laid out of line.
__device__ __forceinline__ int32_t code_of(float w, float sc, float inv) {
    const float t = w * inv;
    float r = rintf(t);
    const bool exact_div = !(fabsf(t - r) < 0.5f - 0x1p-12f);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(exact_div) != 0, 0)) {
        float e = rintf(w / sc);
        e = fminf(fmaxf(e, -127.0f), 127.0f);
        r = exact_div ? e : r;
    }
    return static_cast<int32_t>(r);
}

__device__ __forceinline__ int32_t pack4(int32_t a, int32_t b, int32_t c, int32_t d) {
    return static_cast<int32_t>((static_cast<uint32_t>(a) & 255u) | ((static_cast<uint32_t>(b) & 255u) << 8) |
                                ((static_cast<uint32_t>(c) & 255u) << 16) | (static_cast<uint32_t>(d) << 24));
}

__device__ __forceinline__ int32_t code4(float4 w, float sc, float inv) {
    return pack4(code_of(w.x, sc, inv), code_of(w.y, sc, inv), code_of(w.z, sc, inv), code_of(w.w, sc, inv));
}

// The four float4 of smoothing values of chunk j.
__device__ __forceinline__ void load_s4(const float4* __restrict__ s4, int j, float4 (&sv)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = s4[4 * j + e];
}

// Rows held in registers.  WPR waves share a row (1: four rows per
// workgroup; RQ_WAVES: one row per workgroup); lane l of part p holds the
// row's chunks (c * WPR + p) * 64 + l, c < CPL.  A chunk block lying wholly
// past the row is skipped by its wave (a uniform branch); within a block, a
// lane past the row works on the row's last chunk again (repeats leave the
// maximum as it is) and stores nothing, so no load needs a guard.  q and wq
// may be the same buffer (in place): each lane loads all of its chunks
// before it stores any, and stores only those.
template <int CPL, int WPR>
__global__ __launch_bounds__(RQ_THREADS) void requantize_rows_kernel(
    const int8_t* q, const uint16_t* __restrict__ d, const float* __restrict__ smooth, int64_t N, int64_t K,
    int8_t* wq, float* __restrict__ sw) {
    static_assert(WPR == 1 || WPR == RQ_WAVES, "a row takes one wave or the whole workgroup");
    __shared__ float red[RQ_WAVES];
    const int lane = static_cast<int>(threadIdx.x & 63);
    const int wave = static_cast<int>(threadIdx.x >> 6);
    const int part = wave % WPR;
    const int64_t n = static_cast<int64_t>(blockIdx.x) * (RQ_WAVES / WPR) + wave / WPR;
    if (n >= N) return;   // WPR == 1 only (the grid has a workgroup per row otherwise): no barrier there
    const int K16 = static_cast<int>(K >> 4);
    const i32x4* qr = reinterpret_cast<const i32x4*>(q + n * K);
    const uint16_t* dr = d + n * (K >> 5);
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    auto first = [&](int c) { return (c * WPR + part) * 64; };             // the block's first chunk
    auto chunk = [&](int c) { return min(first(c) + lane, K16 - 1); };
    auto live = [&](int c) { return c + 1 < CPL || first(c) < K16; };      // wave-uniform

    i32x4 qv[CPL];
    float dv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        qv[c] = __builtin_nontemporal_load(qr + chunk(c));
        dv[c] = f16_bits_to_f32(dr[chunk(c) >> 1]);
    }

    // Pass 1.  The smoothing values are read one chunk ahead of their use,
    // so only two chunks of them (32 floats) are live; the scheduling barrier
    // after each chunk keeps the compiler from hoisting them all to the top.
    float wv[CPL][16];
    float4 sa[4], sb[4];
    load_s4(s4, chunk(0), sa);
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (c + 1 < CPL) load_s4(s4, chunk(c + 1), sb);
        if (live(c)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float4 w = smoothed4(static_cast<uint32_t>(qv[c][e]), dv[c], sa[e]);
                amax = abs_nmax4(amax, w);
                wv[c][4 * e] = w.x;
                wv[c][4 * e + 1] = w.y;
                wv[c][4 * e + 2] = w.z;
                wv[c][4 * e + 3] = w.w;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[e] = sb[e];
        __builtin_amdgcn_sched_barrier(0);
    }
    float m = wave_nmax(amax);
    if constexpr (WPR > 1) {
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int i = 1; i < WPR; ++i) m = nmax(m, red[i]);
    }
    const float sc = channel_scale(m);
    if (lane == 0 && part == 0) sw[n] = sc;

    // Pass 2 from the registers.
    i32x4* out = reinterpret_cast<i32x4*>(wq + n * K);
    const float inv = recip_or_nan(sc);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (live(c)) {
            i32x4 packed = {0, 0, 0, 0};
            if (sc > 0.0f) {   // else an all-zero row or one without a scale: every code is 0
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    packed[e] = code4(make_float4(wv[c][4 * e], wv[c][4 * e + 1], wv[c][4 * e + 2],
                                                  wv[c][4 * e + 3]),
                                      sc, inv);
            }
            if (first(c) + lane < K16) __builtin_nontemporal_store(packed, out + first(c) + lane);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int CPL, int WPR>
hipError_t launch_rows(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N, int64_t K, int8_t* wq,
                       float* sw, hipStream_t stream) {
    constexpr int rows = RQ_WAVES / WPR;
    const int64_t blocks = (N + rows - 1) / rows;
    hipLaunchKernelGGL((requantize_rows_kernel<CPL, WPR>), dim3(static_cast<unsigned>(blocks)), dim3(RQ_THREADS),
                       0, stream, q, d, smooth, N, K, wq, sw);
    return hipGetLastError();
}

// Long rows: one workgroup per row, two passes over it.
__global__ __launch_bounds__(RQ_THREADS) void requantize_q8_0_kernel(
    const int8_t* q, const uint16_t* __restrict__ d, const float* __restrict__ smooth, int64_t K, int8_t* wq,
    float* __restrict__ sw) {
    __shared__ float red[RQ_WAVES];
    const int64_t n = blockIdx.x;
    const i32x4* qr = reinterpret_cast<const i32x4*>(q + n * K);
    const uint16_t* dr = d + n * (K / 32);
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int64_t K16 = K >> 4;   // 16-column groups (K % 64 == 0)

    float amax = 0.0f;
    for (int64_t j = threadIdx.x; j < K16; j += RQ_THREADS) {
        const i32x4 q16 = qr[j];
        const float dv = f16_bits_to_f32(dr[j >> 1]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 w = smoothed4(static_cast<uint32_t>(q16[c]), dv, s4[4 * j + c]);
            amax = abs_nmax4(amax, w);
        }
    }
    amax = wave_nmax(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < RQ_WAVES; ++i) m = nmax(m, red[i]);
    const float sc = channel_scale(m);
    if (threadIdx.x == 0) sw[n] = sc;
    const float inv = recip_or_nan(sc);
    // all of the row's loads above come before any store below (the barrier),
    // so the codes may be written over q in place

    i32x4* out = reinterpret_cast<i32x4*>(wq + n * K);
    for (int64_t j = threadIdx.x; j < K16; j += RQ_THREADS) {
        i32x4 packed = {0, 0, 0, 0};
        if (sc > 0.0f) {
            const i32x4 q16 = qr[j];
            const float dv = f16_bits_to_f32(dr[j >> 1]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                packed[c] = code4(smoothed4(static_cast<uint32_t>(q16[c]), dv, s4[4 * j + c]), sc, inv);
        }
        out[j] = packed;
    }
}

}  // namespace

hipError_t launch_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N,
                                  int64_t K, int8_t* wq, float* sw, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    const int64_t k16 = K / 16;
    if (k16 <= RQ_MAX_CPL * 64) {   // a wave per row
        switch ((k16 + 63) / 64) {
            case 1: return launch_rows<1, 1>(q, d, smooth, N, K, wq, sw, stream);
            case 2: return launch_rows<2, 1>(q, d, smooth, N, K, wq, sw, stream);
            case 3: return launch_rows<3, 1>(q, d, smooth, N, K, wq, sw, stream);
            case 4: return launch_rows<4, 1>(q, d, smooth, N, K, wq, sw, stream);
            case 5: return launch_rows<5, 1>(q, d, smooth, N, K, wq, sw, stream);
            default: return launch_rows<6, 1>(q, d, smooth, N, K, wq, sw, stream);
        }
    }
    if (k16 <= RQ_MAX_CPL * RQ_THREADS) {   // a workgroup per row
        switch ((k16 + RQ_THREADS - 1) / RQ_THREADS) {
            case 2: return launch_rows<2, RQ_WAVES>(q, d, smooth, N, K, wq, sw, stream);
            case 3: return launch_rows<3, RQ_WAVES>(q, d, smooth, N, K, wq, sw, stream);
            case 4: return launch_rows<4, RQ_WAVES>(q, d, smooth, N, K, wq, sw, stream);
            case 5: return launch_rows<5, RQ_WAVES>(q, d, smooth, N, K, wq, sw, stream);
            default: return launch_rows<6, RQ_WAVES>(q, d, smooth, N, K, wq, sw, stream);
        }
    }
    hipLaunchKernelGGL(requantize_q8_0_kernel, dim3(static_cast<unsigned>(N)), dim3(RQ_THREADS), 0,
                       stream, q, d, smooth, K, wq, sw);
    return hipGetLastError();
}

}  // namespace w8a8
