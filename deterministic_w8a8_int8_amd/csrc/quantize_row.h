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

__device__ __forceinline__ float4 f4(float v) { return make_float4(v, v, v, v); }

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

// The smoothing values of the columns a thread holds (float4 number t + T*i
// of a row; 1 past K), their reciprocals r = rcp(s) (|error| <= 1 ulp), and
// whether any of them lies outside [2^-120, 2^120] (then that thread takes
// the exact divisions).  With KEEP the smoothing values stay in registers
// (sv) for the exact paths; otherwise those paths read them from memory.
template <int NV, int T, bool KEEP>
__device__ __forceinline__ void load_smoothing(const float4* s4, int K4, float4 (&rv)[NV], float4 (&sv)[NV],
                                               bool& odd_t) {
    const int t = threadIdx.x;
    odd_t = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * T;
        const float4 v = j < K4 ? s4[j] : f4(1.0f);
        if constexpr (KEEP) sv[i] = v;
        rv[i] = make_float4(fast_rcp(v.x), fast_rcp(v.y), fast_rcp(v.z), fast_rcp(v.w));
        const float lo = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
        const float hi = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        odd_t |= !(lo >= 0x1p-120f && hi <= 0x1p120f);
    }
}

// Thread t's float4 numbers t + T*i of a row (zeros past K).  The loads are
// non-temporal: each row is read once, and streaming it past the caches
// measured 3% faster on 8192 x 17408 batches.
template <int NV, int T>
__device__ __forceinline__ void load_row(const float4* xr, int K4, float4 (&xv)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = threadIdx.x + i * T;
        if (j < K4) {
            const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(xr + j));
            xv[i] = make_float4(v.x, v.y, v.z, v.w);
        } else {
            xv[i] = f4(0.0f);
        }
    }
}

__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

__device__ __forceinline__ float max4abs(float4 a) {
    return fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
}

// The fast code of one element: t' = (x*r)*inv rounded to nearest even and
// clamped.  near is set when t' lies within 2^-12 of a half-integer (or is
// not finite): |t' - rint(t')| is exact (Sterbenz, or rint(t') = 0), and it
// exceeds 1/2 - 2^-12 exactly when t' is that close to k + 1/2.  Only then
// can rne(t') differ from rne(fl(fl(x/s)/sx)).
__device__ __forceinline__ int fast_code(float x, float r, float inv, bool& near) {
    const float t = (x * r) * inv;
    const float q = rintf(t);
    near |= !(fabsf(t - q) < 0.5f - 0x1p-12f);
    return static_cast<int>(fminf(fmaxf(q, -127.0f), 127.0f));
}

__device__ __forceinline__ uint32_t pack4i(int a, int b, int c, int d) {
    return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
           ((static_cast<uint32_t>(c) & 0xffu) << 16) | (static_cast<uint32_t>(d) << 24);
}

// Quantise R rows held in registers at once (xv[r], as load_row leaves
// them).  rv_at(i) returns the reciprocals of the smoothing values of the
// thread's float4 number t + T*i, sv_at(i, j) the smoothing values themselves
// (j = t + T*i, the float4 index in the row), and odd_t is as load_smoothing
// leaves it: the caller decides where they live (registers, LDS or memory).
// The codes of float4 t + T*i of row r (four int8 packed little-endian) are
// handed to emit(r, i, packed) as soon as they are final (for t + T*i < K/4),
// so the caller decides whether they are stored at once or kept.  scale[r]
// is the token scale fl(amax/127) (0 for an invalid row); valid[r] is false
// for ok[r] == false or a row without a finite maximum.  GIVEN: the maximum
// is amax_given[r] instead of the row's own.  One barrier for all R rows (the
// block-wide maxima through red[R * NW]).
//
// The work per element is kept small, since at HBM speed the scan has few
// vector-ALU cycles to spare per element: the first pass keeps each float4's
// approximate maximum magnitude (m4), so the second pass tests one value per
// float4 for being a maximum candidate; non-finite smoothed values are found
// from a running sum of the approximations (a NaN or infinity propagates; an
// overflow of the sum only sends the wave down the exact path); and the code
// pass takes one branch per float4, to the exact divisions, when any of its
// four values lies near a rounding boundary.
template <int NV, int T, int R, bool GIVEN, class RvAt, class SvAt, class Emit>
__device__ __forceinline__ void quantize_rows_regs(const float4 (&xv)[R][NV], RvAt&& rv_at, SvAt&& smooth4,
                                                   bool odd_t, int K4, const bool (&ok)[R],
                                                   const float (&amax_given)[R], float* red, Emit&& emit,
                                                   float (&scale)[R], bool (&valid)[R]) {
    constexpr int NW = T / 64;
    const int t = threadIdx.x;
    float amax[R];
    if constexpr (GIVEN) {
        // a given maximum: no reduction over the row.  A NaN, negative or
        // infinite one marks the row invalid, like a bad row index.
#pragma unroll
        for (int r = 0; r < R; ++r) amax[r] = amax_given[r];
    } else {
        float m4[R][NV];       // per float4: max |x * r| over its four values
        float amax_loc[R], fin[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            amax_loc[r] = 0.0f;
            fin[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const float4 ap = mul4(xv[r][i], rv_at(i));
                m4[r][i] = max4abs(ap);
                amax_loc[r] = fmaxf(amax_loc[r], m4[r][i]);
                fin[r] += (ap.x + ap.y) + (ap.z + ap.w);
            }
        }
        // This wave's exact maximum: the element holding it has an
        // approximation within 2^-21 of the wave's approximate maximum (a
        // shuffle reduction, no barrier), so only elements within 2^-19 of
        // it -- usually one per wave -- are divided exactly; all of the
        // wave's are when the approximations cannot be trusted (an odd
        // smoothing value in the wave, a maximum below 2^-96 or at least
        // 2^126, or a NaN or infinity among the approximations, where
        // fl(x/s) may overflow while x*rcp(s) does not or the reverse).  One
        // block-wide maximum of the exact values gives the row's; a
        // non-finite smoothed value makes it +Inf.
        float amax_t[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float amax_w = wave_max(amax_loc[r]);
            const bool all_exact = __any(odd_t || !(fin[r] - fin[r] == 0.0f)) ||
                                   !(amax_w >= 0x1p-96f && amax_w < 0x1p126f);
            const float thresh = amax_w * (1.0f - 0x1p-19f);
            amax_t[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int j = t + i * T;
                if (j < K4 && (all_exact || m4[r][i] >= thresh)) {
                    const float4 ap = mul4(xv[r][i], rv_at(i));
                    const float4 sv4 = smooth4(i, j);
                    const float xs[4] = {xv[r][i].x, xv[r][i].y, xv[r][i].z, xv[r][i].w};
                    const float as[4] = {ap.x, ap.y, ap.z, ap.w};
                    const float ss[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (all_exact || fabsf(as[c]) >= thresh) amax_t[r] = fmaxf(amax_t[r], abs_nf(xs[c] / ss[c]));
                }
            }
            amax_t[r] = wave_max(amax_t[r]);
        }
        const int wave = t >> 6;
        if ((t & 63) == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) red[r * NW + wave] = amax_t[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            amax[r] = red[r * NW];
#pragma unroll
            for (int w = 1; w < NW; ++w) amax[r] = fmaxf(amax[r], red[r * NW + w]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        valid[r] = ok[r] && usable_max(amax[r]);
        // tiny rows (or odd smoothing values) take the exact divisions
        const bool exact = odd_t || !(amax[r] >= 0x1p-96f);
        const float sc = valid[r] ? amax[r] / 127.0f : 0.0f;
        scale[r] = sc;
        const float inv = fast_rcp(sc);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            if (j >= K4) continue;
            uint32_t packed = 0;
            if (sc != 0.0f) {
                const float4 x = xv[r][i];
                bool near = exact;
                if (!exact) {
                    const float4 rr = rv_at(i);
                    packed = pack4i(fast_code(x.x, rr.x, inv, near), fast_code(x.y, rr.y, inv, near),
                                    fast_code(x.z, rr.z, inv, near), fast_code(x.w, rr.w, inv, near));
                }
                if (near) {
                    const float4 v = smooth4(i, j);
                    packed = pack4(quantize_exact(x.x, v.x, sc), quantize_exact(x.y, v.y, sc),
                                   quantize_exact(x.z, v.z, sc), quantize_exact(x.w, v.w, sc));
                }
            }
            emit(r, i, packed);
        }
    }
}

}  // namespace w8a8
