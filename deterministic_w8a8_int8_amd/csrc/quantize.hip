// Per-token activation quantisation after the SmoothQuant per-channel divide.
//
// The review page "StartLux-Prism: Fast, exact inference for
// StartLux-Decision models on NVIDIA GPUs", section "Compute shared evidence
// once", says the weights are requantised with SmoothQuant and the
// activations quantised per token for W8A8.  For one row:
//   x' = fl(x / s)   (IEEE division per channel)
//   a  = max |x'|
//   sx = fl(a / 127)
//   q  = clamp(rne(fl(x' / sx)), -127, 127), or 0 when sx == 0
//
// Design (HBM-bound scan, 4 B read + 1 B written per element):
//   - a workgroup of T = 256 or 512 threads handles one row; thread t holds
//     float4 number t + T*i of the row in registers, so each row is read from
//     HBM once and every wave-level load is 1 KiB contiguous;
//   - exact results without a true division per element.  Two correctly
//     rounded divisions per element would cost as much as the memory
//     traffic, so the kernel works with reciprocals and proves, per element,
//     that the cheap value decides the same bits:
//       * r = rcp(s) (|error| <= 1 ulp) is computed once per column of the
//         workgroup's row.  x*r is within 2^-22 (relative) of fl(x/s).
//         Each wave finds its approximate maximum on these values (shuffles
//         only).  Because fl() is monotone, the wave's exact maximum
//         fl(|x_k|/s_k) is reached by an element whose approximation lies
//         within 2^-19 of that approximate maximum; only those few
//         candidates are divided exactly.  One block-wide maximum of the
//         waves' exact maxima is the row's -- a single barrier per row;
//       * with sx = fl(a/127) (a true division, once per row) and inv =
//         rcp(sx), t' = (x*r)*inv is within 2^-14 of t = fl(fl(x/s)/sx)
//         whenever |t| <= 128.  If t' is more than 2^-12 away from every
//         half-integer, rne(t') = rne(t).  Otherwise (about 5 in 10^4
//         elements) both true divisions are done;
//       * where subnormal intermediates void the relative error bounds the
//         exact divisions are used throughout: a thread holding a smoothing
//         value outside [2^-120, 2^120] (for its elements; its wave divides
//         every element for the maximum), a wave whose approximate maximum is
//         below 2^-96 (for its maximum), and a row whose maximum is below
//         2^-96 (for every element);
//   - the row maximum is a wave64 shuffle reduction, then per-wave partial
//     maxima through LDS (max is exact, so order does not matter);
//   - rows longer than the register budget (K > 32768) take an exact
//     two-pass variant that reads x twice;
//   - a row whose smoothed values include a NaN or an infinity (from the
//     input, or from x/s overflowing) has no finite maximum.  Like a row
//     index out of range, it gets sx = NaN and all codes 0.
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int QTHREADS = 256;   // workgroup of the exact two-pass kernel

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

// NV float4 per thread held in registers: K <= NV * 4 * T; ROWS rows per
// workgroup of T threads.  GIVEN: the per-token maximum comes from amax_in
// (a row-parallel layer's global maximum) instead of the row itself.
template <int NV, int T, int ROWS, bool GIVEN>
__global__ __launch_bounds__(T) void quantize_rows_reg(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t M, int64_t K, int8_t* __restrict__ xq,
    float* __restrict__ sx, const float* __restrict__ amax_in) {
    constexpr int NW = T / 64;
    __shared__ float redf[2][NW];
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int K4 = static_cast<int>(K >> 2);
    const int t = threadIdx.x;

    // per-column reciprocals of the smoothing values, shared by the block's
    // rows (the smoothing values themselves are reloaded on the rare exact
    // paths).  A thread holding a smoothing value outside [2^-120, 2^120]
    // takes the exact divisions for all of its elements.
    float4 rv[NV];
    bool odd_t = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * T;
        const float4 sv = j < K4 ? s4[j] : f4(1.0f);
        rv[i] = make_float4(fast_rcp(sv.x), fast_rcp(sv.y), fast_rcp(sv.z), fast_rcp(sv.w));
        const float lo = fminf(fminf(sv.x, sv.y), fminf(sv.z, sv.w));
        const float hi = fmaxf(fmaxf(sv.x, sv.y), fmaxf(sv.z, sv.w));
        odd_t |= !(lo >= 0x1p-120f && hi <= 0x1p120f);
    }

    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * ROWS;
    for (int rr = 0; rr < ROWS; ++rr) {
        const int64_t m = m0 + rr;
        if (m >= M) break;   // uniform across the block
        int64_t src;
        const bool ok = source_row(row_idx, m, x_rows, &src);
        const float4* xr = reinterpret_cast<const float4*>(x + src * ldx);

        float4 xv[NV];
        float amax_loc = 0.0f;   // this thread's approximate maximum
        bool huge_t = false;     // an approximation that is NaN, infinite or >= 2^126
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            xv[i] = j < K4 ? xr[j] : f4(0.0f);
            if constexpr (!GIVEN) {
                const float4 ap = make_float4(xv[i].x * rv[i].x, xv[i].y * rv[i].y,
                                              xv[i].z * rv[i].z, xv[i].w * rv[i].w);
                amax_loc = absmax4(amax_loc, ap);
                huge_t |= !(fabsf(ap.x) < 0x1p126f) || !(fabsf(ap.y) < 0x1p126f) ||
                          !(fabsf(ap.z) < 0x1p126f) || !(fabsf(ap.w) < 0x1p126f);
            }
        }
        float amax = 0.0f;
        bool valid = ok;
        if constexpr (GIVEN) {
            // a given maximum: no reduction over the row.  A NaN or negative
            // one marks the row invalid, like a bad row index.
            amax = amax_in[m];
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
                    const float4 sv = s4[j];
                    const float ss[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (all_exact || fabsf(xs[c] * rs[c]) >= thresh)
                            amax_t = fmaxf(amax_t, abs_nf(xs[c] / ss[c]));
                }
            }
            amax = block_max<NW>(amax_t, redf[rr & 1]);
            valid = ok && usable_max(amax);
        }
        // tiny rows (or odd smoothing values) take the exact divisions
        const bool exact = odd_t || !(amax >= 0x1p-96f);
        const float scale = valid ? amax / 127.0f : 0.0f;
        if (t == 0) sx[m] = valid ? scale : quiet_nan();
        const float inv = fast_rcp(scale);

        uint32_t* qr = reinterpret_cast<uint32_t*>(xq + m * K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = t + i * T;
            if (j >= K4) continue;
            uint32_t packed = 0;
            if (scale != 0.0f) {
                if (exact) {
                    const float4 sv = s4[j];
                    packed = pack4(quantize_exact(xv[i].x, sv.x, scale), quantize_exact(xv[i].y, sv.y, scale),
                                   quantize_exact(xv[i].z, sv.z, scale), quantize_exact(xv[i].w, sv.w, scale));
                } else {
                    packed = pack4(quantize_fast(xv[i].x, rv[i].x, s4, j, 0, scale, inv),
                                   quantize_fast(xv[i].y, rv[i].y, s4, j, 1, scale, inv),
                                   quantize_fast(xv[i].z, rv[i].z, s4, j, 2, scale, inv),
                                   quantize_fast(xv[i].w, rv[i].w, s4, j, 3, scale, inv));
                }
            }
            qr[j] = packed;
        }
    }
}

// Any K: the row is read twice (the second read usually hits L2) and every
// element takes the exact divisions.
// Exact max_k |fl(x[m,k]/s[k])| of one row (every element divided).
// A NaN or infinite smoothed value makes the maximum +Inf.
__device__ __forceinline__ float row_absmax_exact(const float4* xr, const float4* s4, int64_t K4,
                                                  float* red) {
    float amax = 0.0f;
    for (int64_t j = threadIdx.x; j < K4; j += QTHREADS) {
        const float4 a = xr[j], s = s4[j];
        amax = absmax4_nf(amax, make_float4(a.x / s.x, a.y / s.y, a.z / s.z, a.w / s.w));
    }
    return block_max<QTHREADS / 64>(amax, red);
}

// The slice maximum of a row-parallel rank: amax[m] = (max with amax[m] if
// accumulate) of row m's exact smoothed maximum; +Inf for a slice holding a
// NaN or infinite smoothed value; NaN for a bad row index.
__global__ __launch_bounds__(QTHREADS) void row_absmax_kernel(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t K, int accumulate, float* __restrict__ amax_out) {
    __shared__ float red[QTHREADS / 64];
    const int64_t m = blockIdx.x;
    int64_t src;
    const bool ok = source_row(row_idx, m, x_rows, &src);
    const float a = row_absmax_exact(reinterpret_cast<const float4*>(x + src * ldx),
                                     reinterpret_cast<const float4*>(smooth), K >> 2, red);
    if (threadIdx.x == 0) amax_out[m] = !ok ? quiet_nan() : accumulate ? fmaxf(amax_out[m], a) : a;
}

__global__ __launch_bounds__(QTHREADS) void quantize_rows_stream(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t K, int8_t* __restrict__ xq, float* __restrict__ sx,
    const float* __restrict__ amax_in) {
    __shared__ float red[QTHREADS / 64];
    const int64_t m = blockIdx.x;
    int64_t src;
    const bool ok = source_row(row_idx, m, x_rows, &src);
    const float4* xr = reinterpret_cast<const float4*>(x + src * ldx);
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int64_t K4 = K >> 2;

    const float amax = amax_in ? amax_in[m] : row_absmax_exact(xr, s4, K4, red);
    const bool valid = ok && usable_max(amax);
    const float scale = valid ? amax / 127.0f : 0.0f;
    if (threadIdx.x == 0) sx[m] = valid ? scale : quiet_nan();

    uint32_t* qr = reinterpret_cast<uint32_t*>(xq + m * K);
    for (int64_t j = threadIdx.x; j < K4; j += QTHREADS) {
        const float4 a = xr[j], s = s4[j];
        qr[j] = pack4(quantize_exact(a.x, s.x, scale), quantize_exact(a.y, s.y, scale),
                      quantize_exact(a.z, s.z, scale), quantize_exact(a.w, s.w, scale));
    }
}

template <int NV, int T>
hipError_t launch_reg(const QuantArgs& a, hipStream_t stream) {
    // One row per workgroup: measured faster than sharing the reciprocals
    // over several rows, because more workgroups keep more rows in flight.
    if (a.amax)
        hipLaunchKernelGGL((quantize_rows_reg<NV, T, 1, true>), dim3(static_cast<unsigned>(a.M)), dim3(T),
                           0, stream, a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.M, a.K, a.xq, a.sx,
                           a.amax);
    else
        hipLaunchKernelGGL((quantize_rows_reg<NV, T, 1, false>), dim3(static_cast<unsigned>(a.M)), dim3(T),
                           0, stream, a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.M, a.K, a.xq, a.sx,
                           nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    const int64_t n256 = (a.K + 1023) / 1024;   // float4 per thread with 256 threads
    const int64_t n512 = (a.K + 2047) / 2048;   // ... with 512 threads
    if (n256 <= 1) return launch_reg<1, 256>(a, stream);
    if (n256 <= 2) return launch_reg<2, 256>(a, stream);
    if (n256 <= 3) return launch_reg<3, 256>(a, stream);
    if (n256 <= 4) return launch_reg<4, 256>(a, stream);
    if (n256 <= 5) return launch_reg<5, 256>(a, stream);
    if (n256 <= 6) return launch_reg<6, 256>(a, stream);
    if (n512 <= 4) return launch_reg<4, 512>(a, stream);
    if (n512 <= 5) return launch_reg<5, 512>(a, stream);
    if (n512 <= 6) return launch_reg<6, 512>(a, stream);
    if (n512 <= 8) return launch_reg<8, 512>(a, stream);
    if (n512 <= 9) return launch_reg<9, 512>(a, stream);
    if (n512 <= 12) return launch_reg<12, 512>(a, stream);
    if (n512 <= 16) return launch_reg<16, 512>(a, stream);
    hipLaunchKernelGGL(quantize_rows_stream, dim3(static_cast<unsigned>(a.M)), dim3(QTHREADS), 0,
                       stream, a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.K, a.xq, a.sx, a.amax);
    return hipGetLastError();
}

hipError_t launch_row_absmax(const QuantArgs& a, bool accumulate, float* amax_out, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    hipLaunchKernelGGL(row_absmax_kernel, dim3(static_cast<unsigned>(a.M)), dim3(QTHREADS), 0, stream,
                       a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.K, accumulate ? 1 : 0, amax_out);
    return hipGetLastError();
}

}  // namespace w8a8
