// Device-side helpers shared by the gfx950 kernels of the W8A8 layer.
//
// The fixed binary32 epilogue lives here, once, so the tiled GEMM, the
// skinny GEMM and the candidate read-out all round the same way.  The
// review page "StartLux-Prism: Fast, exact inference for StartLux-Decision
// models on NVIDIA GPUs", section "Bitwise consistency is not lossless
// quantization", asks for scaling, the residual addition and the read-out
// to follow one fixed rounding sequence.
//
// Every translation unit is compiled with -ffp-contract=off.  The pragma
// below repeats that, so no multiply-add in these helpers can be fused,
// whatever flags a user builds with.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace w8a8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// y = fl(fl(fl(float(acc)) * sx) * sw): int32 -> binary32 (ties to even,
// v_cvt_f32_i32), token scale, then channel scale, one rounding each.
__device__ __forceinline__ float scale_acc(int32_t acc, float sxm, float swn) {
    const float t0 = static_cast<float>(acc);
    const float t1 = t0 * sxm;
    const float t2 = t1 * swn;
    return t2;
}

// The same followed by one rounded addition of the residual.
__device__ __forceinline__ float scale_acc_residual(int32_t acc, float sxm, float swn, float r) {
    const float t2 = scale_acc(acc, sxm, swn);
    const float y = t2 + r;
    return y;
}

// A 16-byte output store, marked non-temporal when `stream_out` (the nt bit:
// the line is streamed to memory rather than kept).  Outputs much larger
// than the 256 MB last-level cache are written that way, so that they do not
// leave it full of dirty lines for the next kernel's reads to wait behind.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_out4(float* p, float4 v, bool stream_out) {
    if (stream_out)
        __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
    else
        *reinterpret_cast<float4*>(p) = v;
}

// Outputs of at least this many bytes are stored non-temporally.
constexpr int64_t STREAM_OUT_BYTES = 64ll << 20;

// Quiet NaN for outputs whose inputs were rejected on the device.
__device__ __forceinline__ float quiet_nan() { return __builtin_nanf(""); }

typedef __attribute__((address_space(3))) int8_t lds_i8;

// One wave instruction: every lane copies 16 bytes from gbase + voff into LDS
// at lds + 16*lane (global_load_lds_dwordx4; the LDS base goes through M0).
// Issued as inline asm so that the compiler does not make later LDS reads of
// other buffers wait for this copy; callers wait with an explicit vmcnt.
// M0 is an input operand ("{m0}"), so the compiler writes it and knows it is
// used.  An SALU write of M0 needs one wait state before an LDS DMA reads it;
// the compiler's hazard check does not look inside inline asm, hence the
// s_nop 0 ahead of the copy.
__device__ __forceinline__ void lds_fill16(const int8_t* gbase, uint32_t voff, lds_i8* lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "{m0}"(lds)
                 : "memory");
}

// The same copy with the non-temporal cache policy (nt): for data read once
// per launch, streamed past the caches.
__device__ __forceinline__ void lds_fill16_nt(const int8_t* gbase, uint32_t voff, lds_i8* lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(gbase), "{m0}"(lds)
                 : "memory");
}

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wave64 maximum of a float through cross-lane shuffles (max is exact, so
// the shuffle order cannot change the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace w8a8
