// Per-row building blocks of the per-token quantisation (review page
// "StartLux-Prism: Fast, exact inference for StartLux-Decision models on
// NVIDIA GPUs", section "Compute shared evidence once": activations are
// divided by the SmoothQuant vector and quantised per token), shared by the
// quantisation kernels and the fused answer head, so that both produce the
// same bits by the same code.  The reasoning behind the fast path (exact
// results from reciprocals, proved per element) is written out at the top of
// quantize.hip.
#pragma once

#include "device_common.h"

namespace w8a8 {

__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// Clamp a rounded quotient to the code range; a NaN quotient (possible only
// with a given maximum that does not bound the row) gives code 0.
__device__ __forceinline__ int8_t to_code(float q) {
    if (!(q == q)) return 0;
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(q));
}

// Exact quantisation of one smoothed value (both true divisions done).
__device__ __forceinline__ int8_t quantize_exact(float x, float s, float scale) {
    if (scale == 0.0f) return 0;
    const float t = (x / s) / scale;
    return to_code(rintf(t));
}

// Fast quantisation with the proof described above; falls back to the exact
// divisions when the approximate quotient is near a rounding boundary.
__device__ __forceinline__ int8_t quantize_fast(float x, float r, const float4* s4, int j, int c,
                                                float scale, float inv) {
    const float t = (x * r) * inv;
    const float d = fabsf((t - floorf(t)) - 0.5f);
    float q;
    if (d > 0x1p-12f) {
        q = rintf(t);
    } else {
        const float s = reinterpret_cast<const float*>(s4)[4 * j + c];
        q = rintf((x / s) / scale);
    }
    return to_code(q);
}

// The same with the smoothing value at hand (held in a register).
__device__ __forceinline__ int8_t quantize_fast_s(float x, float r, float s, float scale, float inv) {
    const float t = (x * r) * inv;
    const float d = fabsf((t - floorf(t)) - 0.5f);
    const float q = d > 0x1p-12f ? rintf(t) : rintf((x / s) / scale);
    return to_code(q);
}

__device__ __forceinline__ float4 f4(float v) { return make_float4(v, v, v, v); }

__device__ __forceinline__ float absmax4(float m, float4 v) {
    return fmaxf(fmaxf(fmaxf(m, fabsf(v.x)), fmaxf(fabsf(v.y), fabsf(v.z))), fabsf(v.w));
}

// |v| for the exact row maximum, with NaN mapped to +Inf: a row holding a
// NaN or infinite smoothed value then has an infinite maximum (fmaxf alone
// would drop the NaN), which marks it invalid.
__device__ __forceinline__ float abs_nf(float v) {
    const float a = fabsf(v);
    return a == a ? a : __builtin_inff();
}

__device__ __forceinline__ float absmax4_nf(float m, float4 v) {
    return fmaxf(fmaxf(fmaxf(m, abs_nf(v.x)), fmaxf(abs_nf(v.y), abs_nf(v.z))), abs_nf(v.w));
}

// A per-token maximum that yields a scale: finite and not negative (NaN fails).
__device__ __forceinline__ bool usable_max(float a) { return a >= 0.0f && a <= 0x1.fffffep127f; }

// Block-wide maximum of one float per thread (NW waves).  `red` must not be
// reused until every thread has read the result: callers alternate buffers.
template <int NW>
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, red[w]);
    return m;
}

// Resolve the source row; an index outside [0, x_rows) marks the row invalid.
__device__ __forceinline__ bool source_row(const int32_t* row_idx, int64_t m, int64_t x_rows,
                                           int64_t* src) {
    if (!row_idx) {
        *src = m;
        return true;
    }
    const int64_t r = row_idx[m];
    const bool ok = (r >= 0) && (r < x_rows);
    *src = ok ? r : 0;
    return ok;
}

__device__ __forceinline__ uint32_t pack4(int8_t a, int8_t b, int8_t c, int8_t d) {
    return static_cast<uint32_t>(static_cast<uint8_t>(a)) |
           (static_cast<uint32_t>(static_cast<uint8_t>(b)) << 8) |
           (static_cast<uint32_t>(static_cast<uint8_t>(c)) << 16) |
           (static_cast<uint32_t>(static_cast<uint8_t>(d)) << 24);
}

// Reciprocals of the smoothing values of the columns a thread holds (float4
// number t + T*i of the row), and whether any of them lies outside
// [2^-120, 2^120] (then that thread takes the exact divisions).  With KEEP
// the smoothing values themselves are kept in keep[] too.
template <int NV, int T, bool KEEP = false>
__device__ __forceinline__ void row_reciprocals(const float4* s4, int K4, float4 (&rv)[NV], bool& odd_t,
                                                float4 (&keep)[NV]) {
    const int t = threadIdx.x;
    odd_t = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * T;
        const float4 sv = j < K4 ? s4[j] : f4(1.0f);
        if constexpr (KEEP) keep[i] = sv;
        rv[i] = make_float4(fast_rcp(sv.x), fast_rcp(sv.y), fast_rcp(sv.z), fast_rcp(sv.w));
        const float lo = fminf(fminf(sv.x, sv.y), fminf(sv.z, sv.w));
        const float hi = fmaxf(fmaxf(sv.x, sv.y), fmaxf(sv.z, sv.w));
        odd_t |= !(lo >= 0x1p-120f && hi <= 0x1p120f);
    }
}

// Thread t's float4 numbers t + T*i of a row (zeros past K).
template <int NV, int T>
__device__ __forceinline__ void load_row(const float4* xr, int K4, float4 (&xv)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = threadIdx.x + i * T;
        xv[i] = j < K4 ? xr[j] : f4(0.0f);
    }
}

// Quantise one row held in registers (xv, as load_row leaves it): the codes
// of float4 number t + T*i (four int8 packed little-endian) are handed to
// emit(i, packed) as soon as they are computed (i < NV with t + T*i < K/4),
// so the caller decides whether they are stored at once or kept.
// Returns the token scale fl(amax/127) (0 for an invalid row) and sets valid
// (false for a bad row index, ok == false, or a row without a finite
// maximum).  GIVEN: the maximum is amax_given instead of the row's own.
// With KEEP the rare exact divisions read the smoothing values from sk
// (kept in registers by row_reciprocals), else from memory (s4): the same
// values either way.  One barrier (the block-wide maximum through red[NW]).
template <int NV, int T, bool GIVEN, bool KEEP, class Emit>
__device__ __forceinline__ float quantize_row_regs(const float4 (&xv)[NV], const float4 (&rv)[NV],
                                                   const float4 (&sk)[NV], bool odd_t, const float4* s4,
                                                   int K4, bool ok, float amax_given, float* red, Emit&& emit,
                                                   bool& valid) {
    auto smooth4 = [&](int i, int j) __attribute__((always_inline)) {
        if constexpr (KEEP) return sk[i];
        else return s4[j];
    };
    constexpr int NW = T / 64;
    const int t = threadIdx.x;
    float amax_loc = 0.0f;   // this thread's approximate maximum
    bool huge_t = false;     // an approximation that is NaN, infinite or >= 2^126
    if constexpr (!GIVEN) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float4 ap = make_float4(xv[i].x * rv[i].x, xv[i].y * rv[i].y,
                                          xv[i].z * rv[i].z, xv[i].w * rv[i].w);
            amax_loc = absmax4(amax_loc, ap);
            huge_t |= !(fabsf(ap.x) < 0x1p126f) || !(fabsf(ap.y) < 0x1p126f) ||
                      !(fabsf(ap.z) < 0x1p126f) || !(fabsf(ap.w) < 0x1p126f);
        }
    }
    float amax = 0.0f;
    if constexpr (GIVEN) {
        // a given maximum: no reduction over the row.  A NaN, negative or
        // infinite one marks the row invalid, like a bad row index.
        amax = amax_given;
        valid = ok && usable_max(amax);
    } else {
        // This wave's exact maximum: the element holding it has an
        // approximation within 2^-21 of the wave's approximate maximum
        // (a shuffle reduction, no barrier), so only elements within
        // 2^-19 of it -- usually one per wave -- are divided exactly; all
        // of the wave's are when the approximations cannot be trusted
        // (an odd smoothing value in the wave, a maximum below 2^-96, or
        // an approximation that is NaN, infinite or near overflow, where
        // fl(x/s) may overflow while x*rcp(s) does not or the reverse).
        // One block-wide maximum of the exact values gives the row's; a
        // non-finite smoothed value makes it +Inf.
        const float amax_w = wave_max(amax_loc);
        const bool all_exact = __any(odd_t) || __any(huge_t) || !(amax_w >= 0x1p-96f);
        const float thresh = amax_w * (1.0f - 0x1p-19f);
        float amax_t = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            if (j >= K4) continue;
            const float xs[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            const float rs[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
            bool any = all_exact;
#pragma unroll
            for (int c = 0; c < 4; ++c) any |= fabsf(xs[c] * rs[c]) >= thresh;
            if (any) {
                const float4 sv = smooth4(i, j);
                const float ss[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (all_exact || fabsf(xs[c] * rs[c]) >= thresh)
                        amax_t = fmaxf(amax_t, abs_nf(xs[c] / ss[c]));
            }
        }
        amax = block_max<NW>(amax_t, red);
        valid = ok && usable_max(amax);
    }
    // tiny rows (or odd smoothing values) take the exact divisions
    const bool exact = odd_t || !(amax >= 0x1p-96f);
    const float scale = valid ? amax / 127.0f : 0.0f;
    const float inv = fast_rcp(scale);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * T;
        if (j >= K4) continue;
        uint32_t packed = 0;
        if (scale != 0.0f) {
            if (exact) {
                const float4 sv = smooth4(i, j);
                packed = pack4(quantize_exact(xv[i].x, sv.x, scale), quantize_exact(xv[i].y, sv.y, scale),
                               quantize_exact(xv[i].z, sv.z, scale), quantize_exact(xv[i].w, sv.w, scale));
            } else if constexpr (KEEP) {
                packed = pack4(quantize_fast_s(xv[i].x, rv[i].x, sk[i].x, scale, inv),
                               quantize_fast_s(xv[i].y, rv[i].y, sk[i].y, scale, inv),
                               quantize_fast_s(xv[i].z, rv[i].z, sk[i].z, scale, inv),
                               quantize_fast_s(xv[i].w, rv[i].w, sk[i].w, scale, inv));
            } else {
                packed = pack4(quantize_fast(xv[i].x, rv[i].x, s4, j, 0, scale, inv),
                               quantize_fast(xv[i].y, rv[i].y, s4, j, 1, scale, inv),
                               quantize_fast(xv[i].z, rv[i].z, s4, j, 2, scale, inv),
                               quantize_fast(xv[i].w, rv[i].w, s4, j, 3, scale, inv));
            }
        }
        emit(i, packed);
    }
    return scale;
}

}  // namespace w8a8
