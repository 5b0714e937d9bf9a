// Tiled int8 x int8 -> int32 GEMM on gfx950 matrix cores, with integer
// split-K and the fixed binary32 scale-and-residual epilogue fused in.
//
// What it computes is defined on the review page "StartLux-Prism: Fast,
// exact inference for StartLux-Decision models on NVIDIA GPUs", section
// "Bitwise consistency is not lossless quantization": the int8 products
// accumulate exactly in int32, split-K partial sums stay integers, and
// scaling and the residual addition follow a fixed rounding sequence.  No
// floating-point atomic appears anywhere: the float atomic accumulation that
// page describes flipped a near-tie decision between runs.
//
// Design (CDNA4, wave64):
//   - 256 threads = 4 waves in a 2 x 2 arrangement.  Each wave owns a
//     (32*WTM) x (32*WTN) block of the output as WTM*WTN accumulators of
//     v_mfma_i32_32x32x32_i8 (16 int32 per lane each).
//   - Both operands are K-contiguous (activation [M,K], weight [N,K]).  One
//     K stage is 128 bytes per row: one cache line of every row of the tile.
//     It is copied HBM -> LDS with global_load_lds_dwordx4, which needs no
//     VGPR staging.  Each wave instruction fills 1 KiB of LDS = 8 rows.
//   - LDS holds two stages (double buffer).  Stage s+1 is in flight while
//     the MFMAs consume stage s.  There is one barrier per stage.
//   - 16-byte chunks of a row are XOR-swizzled with (row & 7) ^ ((row >> 3) & 1).
//     Then the 8- or 16-lane groups that a ds_read_b128 serves together hit
//     distinct banks, for either 32 or 64 LDS banks.
//   - Integer accumulation is exact, so any lane -> k assignment gives the
//     same sum, provided A and B use the same one.  Only the placement of the
//     32 x 32 result tile matters.
//   - Block ids are renumbered for the 8 XCDs: the hardware deals workgroups
//     round-robin over XCDs, and the renumbering gives each XCD a contiguous
//     range of tiles, rastered in groups of `group_m` tile rows.  The tiles
//     running together on one XCD then share A and B panels in that XCD's L2.
//   - Split-K: blockIdx picks (tile, chunk).  Every chunk writes its int32
//     partial tile to the workspace in register order: coalesced 256-byte
//     wave stores.  It bumps the tile's arrival counter (an integer atomic
//     on a counter, never on data).  The last arriver adds the other
//     chunks' partials onto its own, resets the counter and runs the
//     epilogue.  The int32 sum is exact, so the arrival order cannot change
//     a bit.
//   - The epilogue stages sx and sw of the tile in LDS.  It computes
//     fl(fl(fl(float(acc))*sx)*sw) (+ r), rounding once per step, with no
//     fused multiply-add (the whole file is built with -ffp-contract=off).
#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int BK = 128;        // K bytes per stage
constexpr int THREADS = 256;   // 4 waves
constexpr int NXCD = 8;        // XCDs on MI355X

template <int WTM, int WTN>
struct Tile {
    static constexpr int BM = 64 * WTM;
    static constexpr int BN = 64 * WTN;
    static constexpr int A_BYTES = BM * BK;
    static constexpr int B_BYTES = BN * BK;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = BM / 32;   // 8 rows per wave instruction, 4 waves
    static constexpr int B_LOADS = BN / 32;
    static constexpr int ACC_PER_WAVE = WTM * WTN * 16 * 64;  // int32 per wave
};

typedef __attribute__((address_space(3))) int8_t lds_i8;

// One wave instruction: every lane copies 16 bytes from gbase + voff into LDS
// at lds + 16*lane (global_load_lds_dwordx4; the LDS base goes through M0).
// Issued as inline asm so that the compiler does not make later LDS reads of
// the other buffer wait for this copy; the caller waits with vmcnt(0)
// before the barrier that publishes the stage.
__device__ __forceinline__ void lds_fill16(const int8_t* gbase, uint32_t voff, lds_i8* lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "s"(lds)
                 : "memory");
}

__device__ __forceinline__ void wait_fills() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keeps the scheduler from mixing the work of neighbouring output tiles,
// which bounds register pressure in the epilogue.
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// Swizzle of the 16-byte chunk index inside a 128-byte LDS row.
__device__ __forceinline__ int row_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int WTM, int WTN>
__global__ __launch_bounds__(THREADS, 1) void gemm_tiled(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ B,
    const float* __restrict__ sw, const float* residual, float* y, int M, int N, int K,
    int tiles_m, int tiles_n, int group_m, int splitk, int kb_per_split,
    int32_t* __restrict__ counters, int32_t* __restrict__ partials) {
    using T = Tile<WTM, WTN>;
    __shared__ __attribute__((aligned(1024))) int8_t smem[2 * T::STAGE];
    __shared__ int last_flag;

    // ---- block -> (tile, split), XCD-contiguous and grouped along M
    const int nblocks = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid % NXCD, slot = bid / NXCD;
    const int per = nblocks / NXCD, extra = nblocks % NXCD;
    const int lid = (xcd < extra) ? xcd * (per + 1) + slot
                                  : extra * (per + 1) + (xcd - extra) * per + slot;
    const int split = lid % splitk;
    const int tile = lid / splitk;
    const int group_size = group_m * tiles_n;
    const int g = tile / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = tile - g * group_size;
    const int tm = first_m + in_g % gm;
    const int tn = in_g / gm;

    const int row0 = tm * T::BM;
    const int col0 = tn * T::BN;
    const int KB = K >> 6;                               // 64-byte k-blocks
    const int kb0 = min(split * kb_per_split, KB);
    const int kb1 = min(kb0 + kb_per_split, KB);
    const int nkb = kb1 - kb0;
    const int nst = (nkb + 1) >> 1;                      // stages (last may be half)
    const bool half_last = (nkb & 1) != 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- per-lane global offsets for the LDS fills
    // Instruction j of wave w fills LDS rows 8*(w + 4j) .. +7; lane l lands in
    // row 8*(w+4j) + l/8 at physical chunk l%8, which holds logical chunk
    // (l%8) ^ swz(row).
    // With r = 8*(w+4j) + l/8: r & 7 = l/8 and (r >> 3) & 1 = w & 1, so the
    // logical chunk a lane fetches is the same for every j.
    const int lrow = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow ^ (wave & 1);
    uint32_t a_off[T::A_LOADS], b_off[T::B_LOADS];
#pragma unroll
    for (int j = 0; j < T::A_LOADS; ++j) {
        const int r = 8 * (wave + 4 * j) + lrow;
        const int gr = min(row0 + r, M - 1);
        a_off[j] = static_cast<uint32_t>(gr - row0) * static_cast<uint32_t>(K) +
                   static_cast<uint32_t>(lchunk * 16);
    }
#pragma unroll
    for (int j = 0; j < T::B_LOADS; ++j) {
        const int r = 8 * (wave + 4 * j) + lrow;
        const int gc = min(col0 + r, N - 1);
        b_off[j] = static_cast<uint32_t>(gc - col0) * static_cast<uint32_t>(K) +
                   static_cast<uint32_t>(lchunk * 16);
    }
    const int8_t* a_base = A + static_cast<int64_t>(row0) * K + kb0 * 64;
    const int8_t* b_base = B + static_cast<int64_t>(col0) * K + kb0 * 64;

    auto issue = [&](int st, int buf) {
        // In a half stage the upper 64 bytes may lie past the chunk (or the
        // matrix): fold those lanes onto the lower half, whose bytes are valid.
        const bool half = half_last && (st == nst - 1);
        const uint32_t fold = (half && lchunk >= 4) ? 64u : 0u;
        const int8_t* ga = a_base + st * BK;
        const int8_t* gb = b_base + st * BK;
        lds_i8* la = (lds_i8*)smem + buf * T::STAGE + 8 * wave * BK;
        lds_i8* lb = la + T::A_BYTES;
#pragma unroll
        for (int j = 0; j < T::A_LOADS; ++j) lds_fill16(ga, a_off[j] - fold, la + 32 * j * BK);
#pragma unroll
        for (int j = 0; j < T::B_LOADS; ++j) lds_fill16(gb, b_off[j] - fold, lb + 32 * j * BK);
    };

    // ---- per-lane LDS read offsets for the MFMA operands
    // Fragment i of this wave: rows wm*32*WTM + 32*i + (lane & 31); K sub-step
    // s (32 bytes) uses logical chunk 2s + (lane >> 5).
    const int rsw = row_swz(lane & 31);
    const int a_row_off = (wm * 32 * WTM + (lane & 31)) * BK;
    const int b_row_off = (wn * 32 * WTN + (lane & 31)) * BK;
    int chunk_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) chunk_off[s] = ((2 * s + (lane >> 5)) ^ rsw) * 16;

    i32x16 acc[WTM][WTN];
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    auto substep = [&](const int8_t* la, const int8_t* lb, int s) {
        i32x4 a[WTM], b[WTN];
#pragma unroll
        for (int i = 0; i < WTM; ++i)
            a[i] = *reinterpret_cast<const i32x4*>(la + a_row_off + i * 32 * BK + chunk_off[s]);
#pragma unroll
        for (int j = 0; j < WTN; ++j)
            b[j] = *reinterpret_cast<const i32x4*>(lb + b_row_off + j * 32 * BK + chunk_off[s]);
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
            for (int j = 0; j < WTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    };

    if (nst > 0) issue(0, 0);
    for (int st = 0; st < nst; ++st) {
        wait_fills();     // this wave's copies of stage st have landed
        __syncthreads();  // ... and every wave's; buffer (st+1)&1 is free again
        if (st + 1 < nst) issue(st + 1, (st + 1) & 1);
        const int8_t* la = smem + (st & 1) * T::STAGE;
        const int8_t* lb = la + T::A_BYTES;
        substep(la, lb, 0);
        substep(la, lb, 1);
        if (!(half_last && st == nst - 1)) {
            substep(la, lb, 2);
            substep(la, lb, 3);
        }
    }

    // ---- integer split-K: last arriver sums the partials in chunk order
    if (splitk > 1) {
        const int ntiles = tiles_m * tiles_n;
        const size_t tile_elems = static_cast<size_t>(T::BM) * T::BN;
        int32_t* mine = partials + (static_cast<size_t>(split) * ntiles + tile) * tile_elems +
                        static_cast<size_t>(wave) * T::ACC_PER_WAVE;
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
            for (int j = 0; j < WTN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[((i * WTN + j) * 16 + e) * 64 + lane] = acc[i][j][e];
        wait_fills();
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) last_flag = (atomicAdd(&counters[tile], 1) == splitk - 1);
        __syncthreads();
        if (!last_flag) return;
        __threadfence();
        if (threadIdx.x == 0) counters[tile] = 0;
        // Integer addition is exact and associative, so adding the other
        // chunks onto this block's own partial (in increasing c) gives the
        // same int32 as P_0 + P_1 + ... + P_{S-1}.  One 32x32 accumulator at
        // a time keeps the register footprint small.
        const int32_t* p0 = partials + static_cast<size_t>(tile) * tile_elems +
                            static_cast<size_t>(wave) * T::ACC_PER_WAVE;
        const size_t cstride = static_cast<size_t>(ntiles) * tile_elems;
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
#pragma unroll
            for (int j = 0; j < WTN; ++j) {
                i32x16 v = acc[i][j];
                const int32_t* pj = p0 + ((i * WTN + j) * 16) * 64 + lane;
                for (int c = 0; c < splitk; ++c) {
                    if (c == split) continue;
                    const int32_t* pc = pj + c * cstride;
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] += pc[e * 64];
                }
                acc[i][j] = v;
                sched_fence();
            }
        }
    }

    // ---- epilogue, in WTM passes of 64 rows.  Every wave parks one 32-row
    // slice of its accumulators in LDS (row-major int32, rows padded by 8
    // words so the two half-waves of a ds_write land in different banks).
    // Then all 256 threads sweep the 64 x BN slice in float4 chunks along
    // rows.  Each wave handles one 1 KiB row segment: 16-byte residual loads
    // and 16-byte output stores, fully coalesced.
    constexpr int LDR = T::BN + 8;                     // staged row pitch (int32)
    int32_t* stage = reinterpret_cast<int32_t*>(smem);
    float* s_sx = reinterpret_cast<float*>(smem + 64 * LDR * 4);
    float* s_sw = s_sx + T::BM;
    __syncthreads();  // all waves are done reading the operand buffers
    for (int t = threadIdx.x; t < T::BM; t += THREADS) s_sx[t] = sx[min(row0 + t, M - 1)];
    for (int t = threadIdx.x; t < T::BN; t += THREADS) s_sw[t] = sw[min(col0 + t, N - 1)];

    const bool vec_ok = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(residual) & 15) == 0;
    constexpr int C4 = T::BN / 4;                      // float4 chunks per staged row
    constexpr int ROWS_PER_SWEEP = THREADS / C4;
    const int c4 = threadIdx.x % C4;
    const int rsub = threadIdx.x / C4;
    const int col = col0 + 4 * c4;
#pragma unroll
    for (int pass = 0; pass < WTM; ++pass) {
        // accumulator slice i = pass of every wave -> staged rows wm*32 + r
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
            const int lc = wn * 32 * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int lr = wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                stage[lr * LDR + lc] = acc[pass][j][e];
            }
            sched_fence();
        }
        __syncthreads();
        const float4 sw4 = *reinterpret_cast<const float4*>(s_sw + 4 * c4);
        for (int r = rsub; r < 64; r += ROWS_PER_SWEEP) {
            // staged row r is tile row (r / 32) * 32 * WTM + pass * 32 + r % 32
            const int lr = (r >> 5) * 32 * WTM + pass * 32 + (r & 31);
            const int row = row0 + lr;
            if (row >= M) continue;
            const int4 a4 = *reinterpret_cast<const int4*>(stage + r * LDR + 4 * c4);
            const float sxm = s_sx[lr];
            const size_t o = static_cast<size_t>(row) * N + col;
            if (vec_ok && col + 3 < N) {
                float4 v;
                if (residual) {
                    const float4 r4 = *reinterpret_cast<const float4*>(residual + o);
                    v.x = scale_acc_residual(a4.x, sxm, sw4.x, r4.x);
                    v.y = scale_acc_residual(a4.y, sxm, sw4.y, r4.y);
                    v.z = scale_acc_residual(a4.z, sxm, sw4.z, r4.z);
                    v.w = scale_acc_residual(a4.w, sxm, sw4.w, r4.w);
                } else {
                    v.x = scale_acc(a4.x, sxm, sw4.x);
                    v.y = scale_acc(a4.y, sxm, sw4.y);
                    v.z = scale_acc(a4.z, sxm, sw4.z);
                    v.w = scale_acc(a4.w, sxm, sw4.w);
                }
                *reinterpret_cast<float4*>(y + o) = v;
            } else {
                const int32_t av[4] = {a4.x, a4.y, a4.z, a4.w};
                const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (col + q < N) {
                        y[o + q] = residual ? scale_acc_residual(av[q], sxm, swv[q], residual[o + q])
                                            : scale_acc(av[q], sxm, swv[q]);
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <int WTM, int WTN>
hipError_t launch_kind(const GemmArgs& a, const GemmPlan& p, void* workspace, hipStream_t stream) {
    using T = Tile<WTM, WTN>;
    const int64_t ntiles = p.tiles_m * p.tiles_n;
    const int KB = static_cast<int>(a.K >> 6);
    const int kb_per_split = (KB + p.splitk - 1) / p.splitk;
    int32_t* counters = nullptr;
    int32_t* partials = nullptr;
    if (p.splitk > 1) {
        counters = static_cast<int32_t*>(workspace);
        const size_t cbytes = ((static_cast<size_t>(ntiles) * 4 + 255) / 256) * 256;
        partials = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + cbytes);
    }
    const unsigned nblocks = static_cast<unsigned>(ntiles * p.splitk);
    hipLaunchKernelGGL((gemm_tiled<WTM, WTN>), dim3(nblocks), dim3(THREADS), 0, stream, a.xq, a.sx,
                       a.w, a.sw, a.residual, a.y, static_cast<int>(a.M), static_cast<int>(a.N),
                       static_cast<int>(a.K), static_cast<int>(p.tiles_m),
                       static_cast<int>(p.tiles_n), p.group_m, p.splitk, kb_per_split, counters,
                       partials);
    (void)sizeof(T);
    return hipGetLastError();
}

int tile_override = -1;

}  // namespace

void set_tile_override(int kind) { tile_override = kind; }

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int splitk) {
    (void)K;
    struct Cand {
        TileKind kind;
        int bm, bn;
        double weight;  // relative per-CU throughput of the tile shape
    };
    static const Cand cands[] = {
        {TILE_256x256, 256, 256, 1.00},
        {TILE_256x128, 256, 128, 0.90},
        {TILE_128x128, 128, 128, 0.75},
    };
    const int ncu = 256;
    int best = 0;
    double best_score = -1.0;
    for (int c = 0; c < 3; ++c) {
        const int64_t tm = (M + cands[c].bm - 1) / cands[c].bm;
        const int64_t tn = (N + cands[c].bn - 1) / cands[c].bn;
        const int64_t blocks = tm * tn * splitk;
        const int64_t rounds = (blocks + ncu - 1) / ncu;
        // useful work over the slots the rounds occupy, times the shape's speed
        const double useful = static_cast<double>(M) * static_cast<double>(N) /
                              (static_cast<double>(tm * cands[c].bm) * static_cast<double>(tn * cands[c].bn));
        const double fill = static_cast<double>(blocks) / static_cast<double>(rounds * ncu);
        const double score = useful * fill * cands[c].weight;
        if (score > best_score + 1e-9) {
            best_score = score;
            best = c;
        }
    }
    if (tile_override >= 0 && tile_override < 3) best = tile_override;
    GemmPlan p;
    p.kind = cands[best].kind;
    p.bm = cands[best].bm;
    p.bn = cands[best].bn;
    p.tiles_m = (M + p.bm - 1) / p.bm;
    p.tiles_n = (N + p.bn - 1) / p.bn;
    p.splitk = splitk;
    p.group_m = 8;
    return p;
}

size_t gemm_workspace_bytes(const GemmPlan& p) {
    if (p.splitk <= 1) return 0;
    const size_t ntiles = static_cast<size_t>(p.tiles_m * p.tiles_n);
    const size_t cbytes = ((ntiles * 4 + 255) / 256) * 256;
    return cbytes + static_cast<size_t>(p.splitk) * ntiles * p.bm * p.bn * 4;
}

hipError_t launch_gemm_tiled(const GemmArgs& a, const GemmPlan& p, void* workspace,
                             hipStream_t stream) {
    switch (p.kind) {
        case TILE_256x256: return launch_kind<4, 4>(a, p, workspace, stream);
        case TILE_256x128: return launch_kind<4, 2>(a, p, workspace, stream);
        case TILE_128x128: return launch_kind<2, 2>(a, p, workspace, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace w8a8
