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
//   - a workgroup of T = 256, 512 or 1024 threads handles one row; thread t
//     holds float4 number t + T*i of the row in registers, so each row is
//     read from HBM once (non-temporal loads) and every wave-level load is
//     1 KiB contiguous;
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
//         candidates are divided exactly (the test is made once per float4,
//         on the maximum of its four approximations kept from the first
//         pass).  One block-wide maximum of the waves' exact maxima is the
//         row's -- a single barrier per row;
//       * with sx = fl(a/127) (a true division, once per row) and inv =
//         rcp(sx), t' = (x*r)*inv is within 2^-14 of t = fl(fl(x/s)/sx)
//         whenever |t| <= 128.  If t' is more than 2^-12 away from every
//         half-integer, rne(t') = rne(t).  Otherwise (about 5 in 10^4
//         elements) both true divisions are done for its float4 (one
//         branch per float4);
//       * where subnormal intermediates void the relative error bounds the
//         exact divisions are used throughout: a thread holding a smoothing
//         value outside [2^-120, 2^120] (for its elements; its wave divides
//         every element for the maximum), a wave whose approximate maximum is
//         below 2^-96 or at least 2^126 or that holds a non-finite
//         approximation (for its maximum), and a row whose maximum is below
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
#include "quantize_row.h"

namespace w8a8 {

namespace {

constexpr int QTHREADS = 256;   // workgroup of the exact two-pass kernel

// NV float4 per thread held in registers: K <= NV * 4 * T; R rows per
// workgroup of T threads, quantised together (one barrier and one set of
// reciprocals for the R rows; the library launches R = 1).  GIVEN: the per-token maximum comes from
// amax_in (a row-parallel layer's global maximum) instead of the row itself.
// KEEP: the smoothing values stay in registers for the rare exact paths.
template <int NV, int T, int R, bool GIVEN, bool KEEP, int WAVES>
__global__ __launch_bounds__(T, WAVES) void quantize_rows_reg(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t M, int64_t K, int8_t* __restrict__ xq,
    float* __restrict__ sx, const float* __restrict__ amax_in) {
    constexpr int NW = T / 64;
    __shared__ float red[R * NW];
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int K4 = static_cast<int>(K >> 2);
    const int t = threadIdx.x;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * R;

    bool live[R], ok[R];
    float amax_g[R];
    float4 xv[R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t m = m0 + r;
        live[r] = m < M;
        int64_t src = 0;
        ok[r] = live[r] && source_row(row_idx, m, x_rows, &src);
        amax_g[r] = GIVEN && live[r] ? amax_in[m] : 0.0f;
        if (live[r]) {
            load_row<NV, T>(reinterpret_cast<const float4*>(x + src * ldx), K4, xv[r]);
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) xv[r][i] = f4(0.0f);
        }
    }
    float4 rv[NV], sv[NV];
    bool odd_t;
    load_smoothing<NV, T, KEEP>(s4, K4, rv, sv, odd_t);

    float scale[R];
    bool valid[R];
    // The codes are stored after the code pass: its rare exact paths load
    // smoothing values (without KEEP), and loads and stores retire through
    // one in-order counter, so a load issued after a store would wait for
    // that store to complete.
    uint32_t codes[R][NV];
    quantize_rows_regs<NV, T, R, GIVEN>(
        xv, [&](int i) __attribute__((always_inline)) { return rv[i]; },
        [&](int i, int j) __attribute__((always_inline)) {
            if constexpr (KEEP) return sv[i];
            else return s4[j];
        },
        odd_t, K4, ok, amax_g, red,
        [&](int r, int i, uint32_t packed) __attribute__((always_inline)) { codes[r][i] = packed; },
        scale, valid);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (live[r] && t + i * T < K4) reinterpret_cast<uint32_t*>(xq + (m0 + r) * K)[t + i * T] = codes[r][i];
    }
    if (t == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (live[r]) sx[m0 + r] = valid[r] ? scale[r] : quiet_nan();
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

template <int NV, int T, int R, bool KEEP, int WAVES>
hipError_t launch_reg(const QuantArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((a.M + R - 1) / R));
    if (a.amax)
        hipLaunchKernelGGL((quantize_rows_reg<NV, T, R, true, KEEP, WAVES>), grid, dim3(T), 0, stream, a.x, a.ldx,
                           a.x_rows, a.row_idx, a.smooth, a.M, a.K, a.xq, a.sx, a.amax);
    else
        hipLaunchKernelGGL((quantize_rows_reg<NV, T, R, false, KEEP, WAVES>), grid, dim3(T), 0, stream, a.x, a.ldx,
                           a.x_rows, a.row_idx, a.smooth, a.M, a.K, a.xq, a.sx, nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    // Threads per row and float4 per thread by K; the second argument of
    // launch_reg's template is the workgroup size, the last the waves per
    // SIMD its register budget is held to (the most each reaches without
    // spilling).  Measured on 8192-row batches: one row per workgroup beats
    // two (more workgroups, more rows in flight), and 1024 threads beat 512
    // at K = 17408 (155 against 166 us).
    const int64_t n256 = (a.K + 1023) / 1024;    // float4 per thread with 256 threads
    const int64_t n512 = (a.K + 2047) / 2048;    // ... with 512 threads
    const int64_t n1024 = (a.K + 4095) / 4096;   // ... with 1024 threads
    // A few rows (decode steps, answer rows): latency, not rows in flight,
    // sets the time, and a row split over more threads is quantised sooner
    // (1 to 64 rows, K = 3072: 4.0 -> 3.6 us with 1024 threads; K = 5120:
    // 4.4 -> 3.9 us with 512; no change at 256 rows)
    if (a.M <= 64 && n256 > 2) {
        if (n1024 <= 1) return launch_reg<1, 1024, 1, false, 8>(a, stream);
        if (n512 <= 3) return launch_reg<3, 512, 1, false, 8>(a, stream);
    }
    if (n256 <= 1) return launch_reg<1, 256, 1, false, 8>(a, stream);
    if (n256 <= 2) return launch_reg<2, 256, 1, false, 8>(a, stream);
    if (n256 <= 3) return launch_reg<3, 256, 1, false, 8>(a, stream);
    if (n256 <= 4) return launch_reg<4, 256, 1, false, 8>(a, stream);
    if (n256 <= 5) return launch_reg<5, 256, 1, false, 8>(a, stream);
    if (n256 <= 6) return launch_reg<6, 256, 1, false, 6>(a, stream);
    if (n512 <= 4) return launch_reg<4, 512, 1, false, 8>(a, stream);
    if (n512 <= 5) return launch_reg<5, 512, 1, false, 6>(a, stream);
    if (n512 <= 6) return launch_reg<6, 512, 1, false, 6>(a, stream);
    if (n512 <= 8) return launch_reg<8, 512, 1, false, 4>(a, stream);
    if (n1024 <= 5) return launch_reg<5, 1024, 1, false, 8>(a, stream);
    if (n512 <= 12) return launch_reg<12, 512, 1, false, 2>(a, stream);
    if (n512 <= 16) return launch_reg<16, 512, 1, false, 2>(a, stream);
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
