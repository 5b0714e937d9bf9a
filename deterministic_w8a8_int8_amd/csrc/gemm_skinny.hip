// Skinny-M W8A8 GEMM (M <= 64): the weight-streaming kernel used for the
// full-vocabulary lm_head and for the candidate-only read-out.
//
// The read-out follows the review page "StartLux-Prism: Fast, exact inference
// for StartLux-Decision models on NVIDIA GPUs".  Section "Compute shared
// evidence once" confines the read-out to the answer positions.  Section
// "Bitwise consistency is not lossless quantization" fixes the read-out
// path.  The candidate form follows the dsiab.com post on moving decision
// models from vLLM to Prism, section "方案": score only the candidate rows
// of the lm_head.  The arithmetic is the same as the tiled GEMM: exact int32
// dot products and the shared fixed epilogue.  So a candidate logit is
// bit-identical to the matching column of the full product.
//
// Design (HBM-bound: each weight byte is used by only M <= 64 rows):
//   - a wave owns 16 weight rows (output columns) and all M activation rows,
//     as R = ceil(M/16) v_mfma_i32_16x16x64_i8 accumulators;
//   - weight fragments stream straight from HBM into VGPRs, 16 bytes per lane,
//     U = 8 K-steps (512 bytes of every row, 4 full cache lines) per batch,
//     with the next batch in flight while the current one multiplies.  No LDS
//     and no barrier is involved;
//   - activation fragments are small and shared by every wave.  They come
//     through L1/L2; lanes whose row is >= M feed zeros and issue no load;
//   - as in the tiled kernel, any lane -> k assignment that A and B share
//     gives the same exact sum.  The 16x16 result tile puts row
//     4*(lane/16) + e and column lane % 16 in lane `lane`, element e;
//   - gathered mode reads weight row gather[j] for output column j, bounds-
//     checked against V: an id outside [0, V) reads row 0 and writes a quiet
//     NaN, then ORs bit 0 into err_flag.  Owner mode writes only column j of
//     row j / C (the candidate read-out).
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int STHREADS = 256;   // 4 waves, 16 columns each
constexpr int U = 8;            // K-steps of 64 bytes per streamed batch

template <int R>
__global__ __launch_bounds__(STHREADS) void gemm_skinny(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* residual, float* y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, const int32_t* __restrict__ gather, int64_t V, int64_t owner_c,
    int32_t* __restrict__ err_flag) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 16;
    if (n0 >= N) return;

    // this lane's weight row
    const int64_t n = min(n0 + (lane & 15), N - 1);
    int64_t wrow = n;
    bool bad_id = false;
    if (gather) {
        const int64_t id = gather[n];
        bad_id = (id < 0) || (id >= V);
        wrow = bad_id ? 0 : id;
    }
    const int kq = (lane >> 4) * 16;  // this lane's 16-byte slot inside a 64-byte K-step
    const int8_t* wp = W + wrow * K + kq;
    const int8_t* ap[R];
    bool arow_ok[R];
#pragma unroll
    for (int g = 0; g < R; ++g) {
        const int64_t m = 16 * g + (lane & 15);
        arow_ok[g] = m < M;
        ap[g] = A + (arow_ok[g] ? m : 0) * K + kq;
    }

    i32x4 acc[R];
#pragma unroll
    for (int g = 0; g < R; ++g) acc[g] = i32x4{0, 0, 0, 0};

    const int64_t steps = K >> 6;
    const int64_t batches = steps / U;
    i32x4 wcur[U];
    if (batches > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) wcur[u] = *reinterpret_cast<const i32x4*>(wp + u * 64);
    }
    for (int64_t b = 0; b < batches; ++b) {
        i32x4 wnext[U];
        const bool more = (b + 1) < batches;
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                wnext[u] = *reinterpret_cast<const i32x4*>(wp + ((b + 1) * U + u) * 64);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t koff = (b * U + u) * 64;
#pragma unroll
            for (int g = 0; g < R; ++g) {
                const i32x4 a = arow_ok[g] ? *reinterpret_cast<const i32x4*>(ap[g] + koff)
                                           : i32x4{0, 0, 0, 0};
                acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wcur[u], acc[g], 0, 0, 0);
            }
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < U; ++u) wcur[u] = wnext[u];
        }
    }
    // remaining K-steps (K/64 not a multiple of U)
    for (int64_t s = batches * U; s < steps; ++s) {
        const i32x4 wv = *reinterpret_cast<const i32x4*>(wp + s * 64);
#pragma unroll
        for (int g = 0; g < R; ++g) {
            const i32x4 a = arow_ok[g] ? *reinterpret_cast<const i32x4*>(ap[g] + s * 64)
                                       : i32x4{0, 0, 0, 0};
            acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wv, acc[g], 0, 0, 0);
        }
    }

    // epilogue: lane holds rows 16g + 4*(lane/16) + e of column n0 + lane%16
    const int64_t col = n0 + (lane & 15);
    if (col >= N) return;
    const float swn = sw[wrow];
    bool flagged = false;
#pragma unroll
    for (int g = 0; g < R; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = 16 * g + 4 * (lane >> 4) + e;
            if (m >= M) continue;
            if (owner_c > 0) {
                if (col / owner_c != m) continue;
                y[col] = bad_id ? quiet_nan() : scale_acc(acc[g][e], sx[m], swn);
                flagged |= bad_id;
            } else {
                const int64_t o = m * ldy + col;
                if (bad_id) {
                    y[o] = quiet_nan();
                    flagged = true;
                } else {
                    y[o] = residual ? scale_acc_residual(acc[g][e], sx[m], swn, residual[o])
                                    : scale_acc(acc[g][e], sx[m], swn);
                }
            }
        }
    }
    if (flagged && err_flag) atomicOr(err_flag, 1);
}

template <int R>
hipError_t launch_r(const SkinnyArgs& a, hipStream_t stream) {
    const int64_t blocks = (a.N + 63) / 64;
    hipLaunchKernelGGL(gemm_skinny<R>, dim3(static_cast<unsigned>(blocks)), dim3(STHREADS), 0,
                       stream, a.xq, a.sx, a.w, a.sw, a.residual, a.y, a.M, a.N, a.K, a.ldy,
                       a.gather, a.V, a.owner_c, a.err_flag);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.M <= 16) return launch_r<1>(a, stream);
    if (a.M <= 32) return launch_r<2>(a, stream);
    if (a.M <= 48) return launch_r<3>(a, stream);
    return launch_r<4>(a, stream);
}

}  // namespace w8a8
