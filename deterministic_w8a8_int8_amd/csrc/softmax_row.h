// The candidate softmax of one row in one wave, shared by the softmax
// kernel and the fused answer head so that both give the same bits.  The
// operation sequence and the exp it uses (Cody and Waite's reduction with a
// degree-13 Taylor polynomial) are described at the top of softmax.hip.
#pragma once

#include "device_common.h"

namespace w8a8 {

constexpr double LN2_HI = 0x1.62e42fefa0000p-1;
constexpr double LN2_LO = 0x1.cf79abc9e3b3ap-40;
constexpr double INV_LN2 = 0x1.71547652b82fep+0;

__device__ __forceinline__ double exp64_nonpositive(double z) {
    if (z < -746.0) return 0.0;  // below half the smallest subnormal
    const double k = rint(z * INV_LN2);
    const double r = (z - k * LN2_HI) - k * LN2_LO;
    // 1/n!, n = 13 .. 0
    constexpr double c[14] = {
        0x1.6124613a86d09p-33, 0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26,
        0x1.27e4fb7789f5cp-22, 0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16,
        0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10, 0x1.1111111111111p-7,
        0x1.5555555555555p-5,  0x1.5555555555555p-3,  0x1.0000000000000p-1,
        0x1.0000000000000p+0,  0x1.0000000000000p+0};
    double p = c[0];
#pragma unroll
    for (int n = 1; n < 14; ++n) p = fma(p, r, c[n]);
    return ldexp(p, static_cast<int>(k));
}

// Called by all 64 lanes of one wave; lane c holds the binary32 logit of
// candidate c when live (c < C <= 64).  Returns lane c's probability: the
// exact maximum, exp64 of each difference, their sum in candidate order
// (lane 0 adds them one by one), one division.  NaN for every candidate of
// a row holding a non-finite logit.  No LDS and no barrier: it may run in
// one wave of a larger workgroup.
__device__ __forceinline__ double candidate_softmax_wave(float lf, bool live, int C) {
    const bool bad = live && !isfinite(lf);
    const double l = static_cast<double>(lf);
    double mx = live ? l : -INFINITY;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off, 64));
    const bool row_bad = __any(bad);
    const double e = live ? exp64_nonpositive(l - mx) : 0.0;
    double s = __shfl(e, 0, 64);
    for (int j = 1; j < C; ++j) s += __shfl(e, j, 64);
    return row_bad ? static_cast<double>(quiet_nan()) : e / s;
}

}  // namespace w8a8
