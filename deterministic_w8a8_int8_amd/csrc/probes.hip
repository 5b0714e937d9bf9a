// Diagnostics: sustained int8 MFMA throughput with no memory traffic, a
// plain streaming read of device memory, and a narrowing stream (4 bytes
// read, 1 written per element).
//
// The int8 matrix cores of MI355X do not sustain their nominal rate on
// every operand stream.  With zero or constant operands they run near the
// nominal 5 POP/s.  With operands that change every instruction and whose
// bits toggle, the sustained rate is markedly lower.  This kernel measures
// that ceiling, so a GEMM's throughput can be judged against what the
// matrix cores deliver on comparable data as well as against the nominal
// peak.
//
// Each wave keeps eight 32x32 int32 accumulators and cycles through four
// register-resident operand sets (A in 4 fragments, B in 2), so every
// v_mfma_i32_32x32x32_i8 sees new operands and no memory is touched inside
// the loop.  Operand kinds:
//   0  A and B uniform on [-128, 127]
//   1  A shaped like per-token-quantised activations (mostly 0 and +-1, a few
//      large outlier values), B uniform
//   2, 3  as 0 and 1, with each 32x32x32 product replaced by two
//      v_mfma_i32_16x16x64_i8 on the same operand registers (the same number
//      of operations, 16x16 accumulators)
// The operands come from an integer hash of the thread and slot numbers.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int CEIL_THREADS = 512;

__device__ __forceinline__ void mfma_acc(i32x16& c, const i32x4& a, const i32x4& b) {
    asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Two 16x16x64 products on two 16x16 accumulators: the operations of one
// 32x32x32 product.
__device__ __forceinline__ void mfma_acc16(i32x4& c0, i32x4& c1, const i32x4& a, const i32x4& b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c0) : "v"(a), "v"(b));
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c1) : "v"(a), "v"(b));
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ int activation_like_byte(uint32_t h) {
    const uint32_t r = h & 255u;
    const int v = r < 180 ? 0 : r < 230 ? 1 : r < 250 ? 2 : 20 + static_cast<int>((h >> 8) % 100u);
    return ((h >> 20) & 1u) ? -v : v;
}

template <int KIND, bool MF16>
__global__ __launch_bounds__(CEIL_THREADS) void mfma_ceiling_kernel(int32_t* sink, int64_t iters) {
    const uint32_t t = threadIdx.x + blockIdx.x * CEIL_THREADS;
    i32x4 a[4][4], b[4][2];
    // the operand loops unrolled, so that the operands live in registers
    // (indexed dynamically they were placed in scratch memory); the byte
    // loop stays rolled (unrolled, its hash arithmetic spilled)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t w = 0;
#pragma nounroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t h = mix32(t * 4096u + s * 256u + i * 16u + e * 4u + q);
                    const int v = KIND == 0 ? static_cast<int>(h & 255u) - 128 : activation_like_byte(h);
                    w |= (static_cast<uint32_t>(v) & 255u) << (8 * q);
                }
                a[s][i][e] = static_cast<int32_t>(w);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) b[s][j][e] = static_cast<int32_t>(mix32(t * 4096u + 2048u + s * 64u + j * 8u + e));
    }
    int32_t x = 0;
    if constexpr (MF16) {
        i32x4 c[4][2][2];
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 2; ++j)
                for (int h = 0; h < 2; ++h)
                    for (int e = 0; e < 4; ++e) c[i][j][h][e] = 0;
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) mfma_acc16(c[i][j][0], c[i][j][1], a[s][i], b[s][j]);
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 2; ++j)
                for (int h = 0; h < 2; ++h)
                    for (int e = 0; e < 4; ++e) x ^= c[i][j][h][e];
    } else {
        i32x16 c[4][2];
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 2; ++j)
                for (int e = 0; e < 16; ++e) c[i][j][e] = 0;
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) mfma_acc(c[i][j], a[s][i], b[s][j]);
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        for (int i = 0; i < 4; ++i)
            for (int j = 0; j < 2; ++j)
                for (int e = 0; e < 16; ++e) x ^= c[i][j][e];
    }
    // keeps the products alive; the sink is written only for this one value
    if (x == 0x7a5c3e1f) sink[0] = x;
}

// Streaming read: workgroup b reads its own contiguous chunk of the buffer,
// every wave instruction 1 KiB (64 lanes x 16 bytes, nontemporal), eight
// independent loads in flight per thread, and xors them.  A grid-stride
// pattern (consecutive instructions of a wave 8 MB apart) sustained 6.1-6.5
// TB/s over 4 GiB; contiguous chunks 7.0-7.1 TB/s.  The sink is written only
// if the xor equals a fixed constant.
constexpr int READ_THREADS = 256;
constexpr int READ_UNROLL = 8;

__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const i32x4* __restrict__ p,
                                                                   int64_t n16, int64_t chunk16,
                                                                   int32_t* sink) {
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * chunk16;
    const int64_t b1 = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
    i32x4 acc = {0, 0, 0, 0};
    int64_t i = b0 + threadIdx.x;
    for (; i + (READ_UNROLL - 1) * READ_THREADS < b1; i += READ_UNROLL * READ_THREADS) {
        i32x4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * READ_THREADS);
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u];
    }
    for (; i < b1; i += READ_THREADS) acc ^= __builtin_nontemporal_load(p + i);
    const int32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x7a5c3e1f) sink[0] = x;
}

// Narrowing stream, the traffic mix of the activation quantizer with none of
// its arithmetic: 4 bytes read and 1 byte written per element.  Workgroup b
// takes its own contiguous chunk of float4s; per iteration each thread
// issues eight nontemporal 16-byte loads, then eight 4-byte stores (the top
// byte of each float; a wave instruction stores 256 contiguous bytes, as the
// quantizer's code stores do).  Nothing else runs, so its rate bounds what
// any quantizer moving these bytes can sustain on the GPU.
__global__ __launch_bounds__(READ_THREADS) void stream_narrow_kernel(const i32x4* __restrict__ p,
                                                                     uint32_t* __restrict__ q, int64_t n16,
                                                                     int64_t chunk16) {
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * chunk16;
    const int64_t b1 = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
    auto narrow = [](const i32x4& v) __attribute__((always_inline)) {
        return (static_cast<uint32_t>(v[0]) >> 24) | ((static_cast<uint32_t>(v[1]) >> 24) << 8) |
               ((static_cast<uint32_t>(v[2]) >> 24) << 16) | ((static_cast<uint32_t>(v[3]) >> 24) << 24);
    };
    int64_t i = b0 + threadIdx.x;
    for (; i + (READ_UNROLL - 1) * READ_THREADS < b1; i += READ_UNROLL * READ_THREADS) {
        i32x4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * READ_THREADS);
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) q[i + u * READ_THREADS] = narrow(v[u]);
    }
    for (; i < b1; i += READ_THREADS) q[i] = narrow(__builtin_nontemporal_load(p + i));
}

}  // namespace

hipError_t launch_stream_narrow(const void* src, int64_t n_floats, void* dst, hipStream_t stream) {
    const int64_t n16 = n_floats / 4;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n16 + READ_THREADS - 1) / READ_THREADS, 256 * 16));
    const int64_t chunk16 = (n16 + blocks - 1) / blocks;
    hipLaunchKernelGGL(stream_narrow_kernel, dim3(static_cast<unsigned>(blocks)), dim3(READ_THREADS), 0,
                       stream, static_cast<const i32x4*>(src), static_cast<uint32_t*>(dst), n16, chunk16);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, int32_t* sink, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n16 + READ_THREADS - 1) / READ_THREADS, 256 * 16));
    const int64_t chunk16 = (n16 + blocks - 1) / blocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(READ_THREADS), 0,
                       stream, static_cast<const i32x4*>(buf), n16, chunk16, sink);
    return hipGetLastError();
}

int64_t mfma_ceiling_ops(int64_t blocks, int64_t iters) {
    // per iteration and wave: 32 MFMAs of 32*32*32 multiply-adds (2 ops each)
    return blocks * (CEIL_THREADS / 64) * iters * 32 * (2LL * 32 * 32 * 32);
}

hipError_t launch_mfma_ceiling(int kind, int64_t blocks, int64_t iters, int32_t* sink,
                               hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(blocks)), block(CEIL_THREADS);
    switch (kind) {
        case 0: hipLaunchKernelGGL((mfma_ceiling_kernel<0, false>), grid, block, 0, stream, sink, iters); break;
        case 1: hipLaunchKernelGGL((mfma_ceiling_kernel<1, false>), grid, block, 0, stream, sink, iters); break;
        case 2: hipLaunchKernelGGL((mfma_ceiling_kernel<0, true>), grid, block, 0, stream, sink, iters); break;
        default: hipLaunchKernelGGL((mfma_ceiling_kernel<1, true>), grid, block, 0, stream, sink, iters); break;
    }
    return hipGetLastError();
}

}  // namespace w8a8
