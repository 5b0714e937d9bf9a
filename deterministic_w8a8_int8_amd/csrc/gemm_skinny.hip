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
//   - weight fragments stream straight from HBM into VGPRs, 16 bytes per
//     lane (plain loads: the non-temporal policy measured 8-27% slower here,
//     unlike the LDS-staged stream below).  U K-steps of 64 bytes are one batch: every row of the wave gets
//     U*64 contiguous bytes.  The activation fragments of the same K-steps are
//     loaded in the same batch, and the next batch is in flight while the
//     current one multiplies.  No LDS, no barrier;
//   - lanes whose activation row is >= M feed zeros and issue no load; for
//     M <= 16 with M*(K+16) <= 40 KiB the activation rows are first staged in
//     LDS, so the weight stream is the only vector-memory traffic;
//   - as in the tiled kernel, any lane -> k assignment that A and B share
//     gives the same exact sum.  The 16x16 result tile puts row
//     4*(lane/16) + e and column lane % 16 in lane `lane`, element e;
//   - K-parallel mode (KSPLIT > 1, for outputs too narrow to fill the GPU,
//     such as the candidate read-out): KSPLIT waves of one workgroup share a
//     16-column tile, each takes a contiguous slice of the K-steps, and the
//     int32 partials are added through LDS.  Integer addition is exact, so
//     the slice count never changes a bit;
//   - gathered mode reads weight row gather[j] for output column j, bounds-
//     checked against V: an id outside [0, V) reads row 0 and writes a quiet
//     NaN, then ORs bit 0 into err_flag.  Owner mode writes only column j of
//     row j / C (the candidate read-out).
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

// R: 16-row activation groups; U: K-steps per streamed batch;
// KSPLIT: waves sharing one column tile (1 = four independent column tiles per workgroup).
// ALDS: activation rows staged in LDS (R == 1, M * K small enough).
template <int R, int U, int KSPLIT, bool ALDS>
__global__ __launch_bounds__(KSPLIT > 1 ? 64 * KSPLIT : 256) void gemm_skinny(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* residual, float* y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, const int32_t* __restrict__ gather, int64_t V, int64_t owner_c,
    int32_t* __restrict__ err_flag) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n0 = KSPLIT > 1 ? static_cast<int64_t>(blockIdx.x) * 16
                                  : (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 16;
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

    // this wave's K-steps
    const int64_t steps = K >> 6;
    int64_t s0 = 0, s1 = steps;
    if (KSPLIT > 1) {
        const int64_t per = (steps + KSPLIT - 1) / KSPLIT;
        s0 = min(static_cast<int64_t>(wave) * per, steps);
        s1 = min(s0 + per, steps);
    }

    // Activation rows in LDS: loaded once per workgroup (16-byte pieces,
    // coalesced), row pitch K + 16 bytes so the active lanes of a fragment
    // read hit different banks.
    extern __shared__ __attribute__((aligned(16))) int8_t a_lds[];
    const int64_t apitch = K + 16;
    if constexpr (ALDS) {
        const int64_t pieces = M * (K >> 4);
        for (int64_t p = threadIdx.x; p < pieces; p += blockDim.x) {
            const int64_t m = p / (K >> 4), c = p % (K >> 4);
            *reinterpret_cast<i32x4*>(a_lds + m * apitch + c * 16) =
                *reinterpret_cast<const i32x4*>(A + m * K + c * 16);
        }
        __syncthreads();
    }
    // Only after every wave has done its share of the staging may a wave
    // without columns leave (uniform across the workgroup in K-parallel mode).
    if (n0 >= N) return;
    const int8_t* al = a_lds + (arow_ok[0] ? static_cast<int64_t>(lane & 15) : 0) * apitch + kq;

    i32x4 acc[R];
#pragma unroll
    for (int g = 0; g < R; ++g) acc[g] = i32x4{0, 0, 0, 0};

    auto a_frag = [&](int g, int64_t s) -> i32x4 {
        if constexpr (ALDS) {
            return arow_ok[0] ? *reinterpret_cast<const i32x4*>(al + s * 64) : i32x4{0, 0, 0, 0};
        } else {
            return arow_ok[g] ? *reinterpret_cast<const i32x4*>(ap[g] + s * 64) : i32x4{0, 0, 0, 0};
        }
    };
    struct Batch {
        i32x4 w[U];
        i32x4 a[ALDS ? 1 : R][ALDS ? 1 : U];
    };
    auto load = [&](Batch& bt, int64_t s) {
#pragma unroll
        for (int u = 0; u < U; ++u) bt.w[u] = *reinterpret_cast<const i32x4*>(wp + (s + u) * 64);
        if constexpr (!ALDS) {
#pragma unroll
            for (int g = 0; g < R; ++g)
#pragma unroll
                for (int u = 0; u < U; ++u) bt.a[g][u] = a_frag(g, s + u);
        }
    };
    auto multiply = [&](const Batch& bt, int64_t s) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < R; ++g) {
                const i32x4 a = ALDS ? a_frag(g, s + u) : bt.a[ALDS ? 0 : g][ALDS ? 0 : u];
                acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bt.w[u], acc[g], 0, 0, 0);
            }
    };

    const int64_t batches = (s1 - s0) / U;
    Batch cur, nxt;
    if (batches > 0) load(cur, s0);
    for (int64_t b = 0; b < batches; ++b) {
        const bool more = (b + 1) < batches;
        if (more) load(nxt, s0 + (b + 1) * U);
        multiply(cur, s0 + b * U);
        if (more) cur = nxt;
    }
    // remaining K-steps of the slice
    for (int64_t s = s0 + batches * U; s < s1; ++s) {
        const i32x4 wv = *reinterpret_cast<const i32x4*>(wp + s * 64);
#pragma unroll
        for (int g = 0; g < R; ++g)
            acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_frag(g, s), wv, acc[g], 0, 0, 0);
    }

    if constexpr (KSPLIT > 1) {
        // add the slices' exact int32 partials through LDS; wave 0 finishes
        __shared__ int32_t red[KSPLIT][R * 4][64];
#pragma unroll
        for (int g = 0; g < R; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][g * 4 + e][lane] = acc[g][e];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int g = 0; g < R; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int32_t t = 0;
                for (int w = 0; w < KSPLIT; ++w) t += red[w][g * 4 + e][lane];
                acc[g][e] = t;
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


// ---- Weight stream through LDS (full products with at most 16 activation
// rows staged in LDS, and enough column tiles to fill the GPU: the
// full-vocabulary read-out).  Loads in the MFMA fragment layout touch 16 rows
// x 64 bytes per wave instruction; a streaming probe over the lm_head's 1.27
// GB read that pattern at 5.1 TB/s and whole 1 KiB-contiguous instructions at
// 6.8 TB/s (with no LDS, many waves per CU).  Here the copy instructions
// (global_load_lds_dwordx4) read RB = 64*KS contiguous bytes of 16/KS rows
// each into LDS, and the fragments are read from LDS.  Each wave streams its
// own 16 weight rows through its own NST-stage ring, so no barrier is
// needed: a wave waits only for its own copies.  The ring bounds the bytes in
// flight: 4 waves x 4 stages of 256-byte rows (two workgroups per CU) took
// the 3 x 248000 x 5120 read-out from 216.7 to 211.9 us; 512- and 1024-byte
// rows per stage, with fewer waves or stages, were slower (223-349 us).
// The copies carry the non-temporal cache policy: streaming the lm_head past
// the caches took the read-out from 211 to 189 us (0.84 of HBM peak).
//   Stage t holds K-bytes [RB t, RB (t+1)) of the wave's 16 rows.  Copy
// instruction j (0..KS-1) covers rows RPI*j .. RPI*j + RPI-1 (RPI = 16/KS):
// lane l reads row r = RPI*j + l/CPR (CPR = 4*KS chunks of 16 bytes per row
// and stage), chunk c = (l % CPR) ^ r, and lands at j*1024 + 16*l.  So chunk c
// of row r sits at (r/RPI)*1024 + (r%RPI)*RB + 16*(c ^ r): a fragment read (16
// rows at one chunk) hits 16 different 16-byte bank groups.
constexpr int WL_KSTEPS = 4;                      // 64-byte K-steps per stage
constexpr int WL_RB = 64 * WL_KSTEPS;             // bytes per row and stage
constexpr int WL_CPR = WL_RB / 16;                // 16-byte chunks per row and stage
constexpr int WL_RPI = 64 / WL_CPR;               // rows per copy instruction
constexpr int WL_STAGE = 16 * WL_RB;              // bytes per wave-stage
constexpr int WL_NST = 4;                         // stages per wave ring
constexpr int WL_RING = WL_NST * WL_STAGE;        // bytes per wave
constexpr int WL_WAVES = 4;
static_assert(WL_CPR >= 16 && WL_RPI * WL_CPR == 64 && WL_NST >= 2, "weight stream layout");
static_assert((WL_NST - 2) * WL_KSTEPS <= 63, "copies in flight must fit the 6-bit vmcnt");

// wait until the copies of stage t have landed, with `after` later stages
// (KS instructions each) still allowed in flight
template <int A>
__device__ __forceinline__ void wl_wait(int after) {
    if constexpr (A == 0) {
        wait_vm<0>();
    } else {
        if (after >= A) wait_vm<A * WL_KSTEPS>();
        else wl_wait<A - 1>(after);
    }
}

__global__ __launch_bounds__(64 * WL_WAVES) void gemm_skinny_wlds(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* residual, float* y, int64_t M, int64_t N, int64_t K,
    int64_t ldy) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: copy bases in SGPRs
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * WL_WAVES + wave) * 16;
    extern __shared__ __attribute__((aligned(1024))) int8_t wl_lds[];
    int8_t* const a_lds = wl_lds + WL_WAVES * WL_RING;
    const int64_t apitch = K + 16;
    const int kq = (lane >> 4) * 16;
    {   // the activation rows, once per workgroup (as in the ALDS path)
        const int64_t pieces = M * (K >> 4);
        for (int64_t p = threadIdx.x; p < pieces; p += blockDim.x) {
            const int64_t m = p / (K >> 4), c = p % (K >> 4);
            *reinterpret_cast<i32x4*>(a_lds + m * apitch + c * 16) =
                *reinterpret_cast<const i32x4*>(A + m * K + c * 16);
        }
        __syncthreads();
    }
    if (n0 >= N) return;
    const bool arow_ok = (lane & 15) < M;
    const int8_t* al = a_lds + (arow_ok ? (lane & 15) : 0) * apitch + kq;
    auto a_frag = [&](int64_t s) -> i32x4 {
        return arow_ok ? *reinterpret_cast<const i32x4*>(al + s * 64) : i32x4{0, 0, 0, 0};
    };

    // copy offsets of this lane (rows past N read row N-1; those columns are
    // never stored)
    uint32_t woff[WL_KSTEPS];
#pragma unroll
    for (int j = 0; j < WL_KSTEPS; ++j) {
        const int r = WL_RPI * j + lane / WL_CPR;
        const int64_t row = min(n0 + r, N - 1);
        woff[j] = static_cast<uint32_t>((row - n0) * K) + static_cast<uint32_t>(16 * ((lane % WL_CPR) ^ r));
    }
    lds_i8* const ring = (lds_i8*)wl_lds + wave * WL_RING;
    const int8_t* const wbase = W + n0 * K;
    const int64_t nstages = K / WL_RB;
    auto issue = [&](int64_t t) __attribute__((always_inline)) {
        lds_i8* const dst = ring + (t % WL_NST) * WL_STAGE;
        const int8_t* const src = wbase + t * WL_RB;
#pragma unroll
        for (int j = 0; j < WL_KSTEPS; ++j) lds_fill16_nt(src, woff[j], dst + j * 1024);   // read once: streamed
    };
    // fragment of K-step s of a stage: row r = lane & 15, chunk 4s + lane/16
    const int fr = lane & 15;
    const int frow_off = (fr / WL_RPI) * 1024 + (fr % WL_RPI) * WL_RB;
    const int8_t* const ring_g = wl_lds + wave * WL_RING;

    i32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < WL_NST - 1; ++t)
        if (t < nstages) issue(t);
    for (int64_t t = 0; t < nstages; ++t) {
        wl_wait<WL_NST - 2>(static_cast<int>(min(static_cast<int64_t>(WL_NST - 2), nstages - 1 - t)));
        // the buffer of stage t-1, multiplied in the last iteration: every
        // LDS read of it has returned before the copy may overwrite it
        if (t + WL_NST - 1 < nstages) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(t + WL_NST - 1);
        }
        const int8_t* const st = ring_g + (t % WL_NST) * WL_STAGE + frow_off;
#pragma unroll
        for (int s = 0; s < WL_KSTEPS; ++s) {
            const int c = 4 * s + (lane >> 4);
            const i32x4 wv = *reinterpret_cast<const i32x4*>(st + 16 * (c ^ fr));
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_frag(t * WL_KSTEPS + s), wv, acc, 0, 0, 0);
        }
    }
    // K-steps past the last whole stage, straight from memory
    const int8_t* const wp = W + min(n0 + (lane & 15), N - 1) * K + kq;
    for (int64_t s = nstages * WL_KSTEPS; s < (K >> 6); ++s) {
        const i32x4 wv = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wp + s * 64));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_frag(s), wv, acc, 0, 0, 0);
    }

    // epilogue: lane holds rows 4*(lane/16) + e of column n0 + lane%16
    const int64_t col = n0 + (lane & 15);
    if (col >= N) return;
    const float swn = sw[col];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t m = 4 * (lane >> 4) + e;
        if (m >= M) continue;
        const int64_t o = m * ldy + col;
        y[o] = residual ? scale_acc_residual(acc[e], sx[m], swn, residual[o]) : scale_acc(acc[e], sx[m], swn);
    }
}

template <int R, int U, int KSPLIT, bool ALDS>
hipError_t launch_r(const SkinnyArgs& a, hipStream_t stream) {
    const int64_t tiles = (a.N + 15) / 16;
    const int64_t blocks = KSPLIT > 1 ? tiles : (tiles + 3) / 4;
    const int threads = KSPLIT > 1 ? 64 * KSPLIT : 256;
    const size_t lds = ALDS ? static_cast<size_t>(a.M * (a.K + 16)) : 0;
    hipLaunchKernelGGL((gemm_skinny<R, U, KSPLIT, ALDS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), lds, stream, a.xq, a.sx, a.w, a.sw, a.residual, a.y, a.M, a.N,
                       a.K, a.ldy, a.gather, a.V, a.owner_c, a.err_flag);
    return hipGetLastError();
}

// Activation rows go to LDS when they fit comfortably (R == 1 only).
constexpr int64_t kSkinnyLdsBytes = 40 * 1024;

template <int R, int U, bool ALDS>
hipError_t launch_rk(const SkinnyArgs& a, hipStream_t stream) {
    // Narrow outputs cannot fill 256 CUs with one wave per 16 columns: split K
    // over up to 16 waves per column tile instead.
    const int64_t tiles = (a.N + 15) / 16;
    const int64_t steps = a.K >> 6;
    if constexpr (R == 1) {
        // 16 waves per workgroup leave 128 VGPRs per lane: use 4-step batches
        if (tiles < 256 && steps >= 64) return launch_r<1, 4, 16, ALDS>(a, stream);
    }
    if (tiles < 1024 && steps >= 32) return launch_r<R, U, 4, ALDS>(a, stream);
    return launch_r<R, U, 1, ALDS>(a, stream);
}

}  // namespace

bool skinny_streams_lds(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = (N + 15) / 16;
    return M >= 1 && M <= 16 && M * (K + 16) <= kSkinnyLdsBytes && tiles >= 1024 && K >= WL_RB &&
           K * 16 < (int64_t(1) << 32);
}

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    const int64_t tiles = (a.N + 15) / 16;
    const int64_t a_bytes = a.M * (a.K + 16);
    if (!a.gather && a.owner_c == 0 && skinny_streams_lds(a.M, a.N, a.K)) {
        const size_t lds = static_cast<size_t>(WL_WAVES * WL_RING + a_bytes);
        hipLaunchKernelGGL(gemm_skinny_wlds, dim3(static_cast<unsigned>((tiles + WL_WAVES - 1) / WL_WAVES)),
                           dim3(64 * WL_WAVES), lds, stream, a.xq, a.sx, a.w, a.sw, a.residual, a.y, a.M, a.N,
                           a.K, a.ldy);
        return hipGetLastError();
    }
    if (a.M <= 16) {
        if (a.M * (a.K + 16) <= kSkinnyLdsBytes) return launch_rk<1, 8, true>(a, stream);
        return launch_rk<1, 8, false>(a, stream);
    }
    if (a.M <= 32) return launch_rk<2, 4, false>(a, stream);
    if (a.M <= 48) return launch_rk<3, 4, false>(a, stream);
    return launch_rk<4, 4, false>(a, stream);
}

}  // namespace w8a8
