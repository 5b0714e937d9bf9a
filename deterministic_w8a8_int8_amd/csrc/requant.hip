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
// the same symmetric round-half-even rule as the activations.
//
// Design: a one-off pass (1 byte read and 1 written per weight, plus the
// block scales and the smoothing vector).  One 256-thread workgroup per
// weight row; each thread takes 16 consecutive columns at a time (one
// 16-byte load of codes, four float4 of smoothing values, one block scale:
// 16 columns never straddle a 32-column block).  Pass 1 finds the exact row
// maximum (max is exact, order free); pass 2 recomputes w' -- the codes are
// re-read from L2 -- and stores the new codes.  True IEEE divisions
// throughout (they, not HBM, set the speed): this runs once per model load.
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int RQ_THREADS = 256;

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

__device__ __forceinline__ uint32_t code(float w, float sc, int shift) {
    float r = rintf(w / sc);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (static_cast<uint32_t>(static_cast<int>(r)) & 255u) << shift;
}

__global__ __launch_bounds__(RQ_THREADS) void requantize_q8_0_kernel(
    const int8_t* __restrict__ q, const uint16_t* __restrict__ d, const float* __restrict__ smooth,
    int64_t K, int8_t* __restrict__ wq, float* __restrict__ sw) {
    __shared__ float red[RQ_THREADS / 64];
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
            amax = fmaxf(fmaxf(fmaxf(amax, fabsf(w.x)), fmaxf(fabsf(w.y), fabsf(w.z))), fabsf(w.w));
        }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < RQ_THREADS / 64; ++i) m = fmaxf(m, red[i]);
    const float sc = m / 127.0f;
    if (threadIdx.x == 0) sw[n] = sc;

    i32x4* out = reinterpret_cast<i32x4*>(wq + n * K);
    for (int64_t j = threadIdx.x; j < K16; j += RQ_THREADS) {
        i32x4 packed = {0, 0, 0, 0};
        if (sc != 0.0f) {
            const i32x4 q16 = qr[j];
            const float dv = f16_bits_to_f32(dr[j >> 1]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 w = smoothed4(static_cast<uint32_t>(q16[c]), dv, s4[4 * j + c]);
                packed[c] = static_cast<int32_t>(code(w.x, sc, 0) | code(w.y, sc, 8) | code(w.z, sc, 16) |
                                                 code(w.w, sc, 24));
            }
        }
        out[j] = packed;
    }
}

}  // namespace

hipError_t launch_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N,
                                  int64_t K, int8_t* wq, float* sw, hipStream_t stream) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(requantize_q8_0_kernel, dim3(static_cast<unsigned>(N)), dim3(RQ_THREADS), 0,
                       stream, q, d, smooth, K, wq, sw);
    return hipGetLastError();
}

}  // namespace w8a8
