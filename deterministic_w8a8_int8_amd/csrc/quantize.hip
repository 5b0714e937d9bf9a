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
//   - one 256-thread workgroup per output row; thread t holds float4 number
//     t + 256*i of the row in registers, so the row is read from HBM once
//     and every wave-level load is 1 KiB contiguous;
//   - x' is kept in registers between the max and the quantisation;
//   - the row maximum is a wave64 shuffle reduction, then four partial
//     maxima through LDS (max is exact, so order does not matter);
//   - rows longer than the register budget (K > 32768) take a two-pass
//     variant that reads x twice, recomputing the identical quotients;
//   - both divisions are true IEEE divisions (hipcc's default expansion is
//     correctly rounded), and rne is v_rndne_f32.
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int QTHREADS = 256;

__device__ __forceinline__ int8_t quantize_one(float v, float scale) {
    if (scale == 0.0f) return 0;
    const float t = v / scale;
    float r = rintf(t);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(r));
}

__device__ __forceinline__ uint32_t pack4(float4 v, float scale) {
    const uint32_t b0 = static_cast<uint8_t>(quantize_one(v.x, scale));
    const uint32_t b1 = static_cast<uint8_t>(quantize_one(v.y, scale));
    const uint32_t b2 = static_cast<uint8_t>(quantize_one(v.z, scale));
    const uint32_t b3 = static_cast<uint8_t>(quantize_one(v.w, scale));
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ float4 smooth4(float4 a, float4 s) {
    return make_float4(a.x / s.x, a.y / s.y, a.z / s.z, a.w / s.w);
}

__device__ __forceinline__ float absmax4(float m, float4 v) {
    return fmaxf(fmaxf(fmaxf(m, fabsf(v.x)), fmaxf(fabsf(v.y), fabsf(v.z))), fabsf(v.w));
}

// Block-wide maximum of one float per thread (4 waves).
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return v;
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

// NV float4 per thread held in registers: K <= NV * 4 * 256.
template <int NV>
__global__ __launch_bounds__(QTHREADS) void quantize_rows_reg(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t K, int8_t* __restrict__ xq, float* __restrict__ sx) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    int64_t src;
    const bool ok = source_row(row_idx, m, x_rows, &src);
    const float4* xr = reinterpret_cast<const float4*>(x + src * ldx);
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int K4 = static_cast<int>(K >> 2);
    const int t = threadIdx.x;

    float4 v[NV];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * QTHREADS;
        if (j < K4) {
            v[i] = smooth4(xr[j], s4[j]);
            amax = absmax4(amax, v[i]);
        } else {
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    amax = block_max(amax, red);
    const float scale = ok ? amax / 127.0f : 0.0f;
    if (t == 0) sx[m] = ok ? scale : quiet_nan();

    uint32_t* qr = reinterpret_cast<uint32_t*>(xq + m * K);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = t + i * QTHREADS;
        if (j < K4) qr[j] = pack4(v[i], scale);
    }
}

// Any K: the row is read twice (the second read usually hits L2); the
// quotients are recomputed bit-identically.
__global__ __launch_bounds__(QTHREADS) void quantize_rows_stream(
    const float* __restrict__ x, int64_t ldx, int64_t x_rows, const int32_t* __restrict__ row_idx,
    const float* __restrict__ smooth, int64_t K, int8_t* __restrict__ xq, float* __restrict__ sx) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    int64_t src;
    const bool ok = source_row(row_idx, m, x_rows, &src);
    const float4* xr = reinterpret_cast<const float4*>(x + src * ldx);
    const float4* s4 = reinterpret_cast<const float4*>(smooth);
    const int64_t K4 = K >> 2;

    float amax = 0.0f;
    for (int64_t j = threadIdx.x; j < K4; j += QTHREADS) amax = absmax4(amax, smooth4(xr[j], s4[j]));
    amax = block_max(amax, red);
    const float scale = ok ? amax / 127.0f : 0.0f;
    if (threadIdx.x == 0) sx[m] = ok ? scale : quiet_nan();

    uint32_t* qr = reinterpret_cast<uint32_t*>(xq + m * K);
    for (int64_t j = threadIdx.x; j < K4; j += QTHREADS) qr[j] = pack4(smooth4(xr[j], s4[j]), scale);
}

template <int NV>
hipError_t launch_reg(const QuantArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(quantize_rows_reg<NV>, dim3(static_cast<unsigned>(a.M)), dim3(QTHREADS), 0,
                       stream, a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.K, a.xq, a.sx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    const int64_t need = (a.K + 4 * QTHREADS - 1) / (4 * QTHREADS);  // float4 per thread
    if (need <= 1) return launch_reg<1>(a, stream);
    if (need <= 2) return launch_reg<2>(a, stream);
    if (need <= 3) return launch_reg<3>(a, stream);
    if (need <= 4) return launch_reg<4>(a, stream);
    if (need <= 5) return launch_reg<5>(a, stream);
    if (need <= 6) return launch_reg<6>(a, stream);
    if (need <= 8) return launch_reg<8>(a, stream);
    if (need <= 10) return launch_reg<10>(a, stream);
    if (need <= 12) return launch_reg<12>(a, stream);
    if (need <= 14) return launch_reg<14>(a, stream);
    if (need <= 17) return launch_reg<17>(a, stream);
    if (need <= 20) return launch_reg<20>(a, stream);
    if (need <= 24) return launch_reg<24>(a, stream);
    if (need <= 32) return launch_reg<32>(a, stream);
    hipLaunchKernelGGL(quantize_rows_stream, dim3(static_cast<unsigned>(a.M)), dim3(QTHREADS), 0,
                       stream, a.x, a.ldx, a.x_rows, a.row_idx, a.smooth, a.K, a.xq, a.sx);
    return hipGetLastError();
}

}  // namespace w8a8
