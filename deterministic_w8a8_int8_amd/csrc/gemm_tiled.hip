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
// Design (CDNA4, wave64).  One kernel template, several tile configurations
// (Cfg below); results never depend on the configuration:
//   - WGM x WGN waves per workgroup.  Each wave owns a (32*WTM) x (32*WTN)
//     block of the output as WTM*WTN accumulators of v_mfma_i32_32x32x32_i8
//     (16 int32 per lane each, held in AGPRs).
//   - Both operands are K-contiguous (activation [M,K], weight [N,K]).  One
//     K stage is BK bytes (64 or 128) of every row of the tile.  It is
//     copied HBM -> LDS with global_load_lds_dwordx4, which needs no VGPR
//     staging.  Each wave instruction fills 1 KiB of LDS.
//   - NST LDS stages.  NST - 1 stages are being copied in while one is
//     multiplied.  There is one barrier per stage.  Configurations with two
//     waves per SIMD (8 waves, or 2 workgroups per CU) let one wave issue
//     MFMAs while the other waits on LDS, a barrier or its epilogue.
//   - 16-byte chunks of a row are XOR-swizzled (row_swz).  Then the 8- or
//     16-lane groups that a ds_read_b128 serves together hit distinct banks,
//     for either 32 or 64 LDS banks.
//   - Integer accumulation is exact, so any lane -> k assignment gives the
//     same sum, provided A and B use the same one.  Only the placement of the
//     32 x 32 result tile matters.  The weight fragment is the MFMA's first
//     operand, so each tile holds the transposed block: lane l, element e is
//     output row (l % 32) and column 8*(e/4) + 4*(l/32) + e%4.  Four
//     consecutive elements are four adjacent columns of one row, written
//     with one 16-byte store.
//   - Block ids are renumbered for the 8 XCDs: the hardware deals workgroups
//     round-robin over XCDs, and the renumbering gives each XCD a contiguous
//     range of tiles, rastered in groups of `group_m` tile rows.  The tiles
//     running together on one XCD then share A and B panels in that XCD's L2.
//   - Split-K: blockIdx picks (tile, chunk).  Every chunk writes its int32
//     partial tile, row-major, to its own slice of the workspace through the
//     same LDS-staged, coalesced path as the epilogue.  A second kernel on
//     the same stream (splitk_reduce) adds the S slices of each output, in
//     chunk order, and runs the epilogue.  No workgroup waits for another
//     and no cache is flushed inside the GEMM: a device-scope fence per tile
//     would write back and invalidate the XCD's L2 under the other
//     workgroups' operand panels.  The int32 sum is exact, so neither the
//     order nor S can change a bit.
//   - The epilogue stages sx and sw of the tile in LDS.  It computes
//     fl(fl(fl(float(acc))*sx)*sw) (+ r), rounding once per step, with no
//     fused multiply-add (the whole file is built with -ffp-contract=off).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int NXCD = 8;        // XCDs on MI355X

// A tile configuration.
//   WGM x WGN   waves per workgroup        WTM x WTN  32x32 MFMA tiles per wave
//   BK_         K bytes per LDS stage      NST_       LDS stages
//   OCC_        workgroups per CU the register budget is sized for
//   PREFETCH_   touch the L2 lines of a later stage (256-row tiles, NST = 2)
//   EPI_H_      the LDS-staged epilogue parks the wave rows in EPI_H_ groups
//               (one group per pass), so that a pass fits in the LDS
//   MF16_       v_mfma_i32_16x16x64_i8 instead of v_mfma_i32_32x32x32_i8
//               (NST = 2, BK = 128, LDS-staged epilogue)
template <int WGM_, int WGN_, int WTM_, int WTN_, int BK_, int NST_, int OCC_, bool DIRECT_EPI_ = false,
          bool PREFETCH_ = false, int EPI_H_ = 1, bool MF16_ = false>
struct Cfg {
    static constexpr bool DIRECT_EPI = DIRECT_EPI_;
    static constexpr bool PREFETCH = PREFETCH_;
    static constexpr int EPI_H = EPI_H_;
    static constexpr bool MF16 = MF16_;
    static_assert(!MF16_ || (NST_ == 2 && BK_ == 128 && !DIRECT_EPI_), "16x16x64 path");
    static constexpr int WGM = WGM_, WGN = WGN_, WTM = WTM_, WTN = WTN_;
    static constexpr int NW = WGM * WGN;
    static constexpr int THREADS = 64 * NW;
    static constexpr int BM = 32 * WTM * WGM;
    static constexpr int BN = 32 * WTN * WGN;
    static constexpr int BK = BK_;
    static constexpr int NST = NST_;
    static constexpr int OCC = OCC_;
    static constexpr int CHUNKS = BK / 16;            // 16-byte chunks per LDS row
    static constexpr int ROWS_PER_FILL = 64 / CHUNKS; // rows one wave instruction fills
    static constexpr int A_BYTES = BM * BK;
    static constexpr int B_BYTES = BN * BK;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = BM / (ROWS_PER_FILL * NW);
    static constexpr int B_LOADS = BN / (ROWS_PER_FILL * NW);
    static constexpr int LPS = A_LOADS + B_LOADS;     // fill instructions per wave per stage
    static constexpr int SUBSTEPS = BK / 32;          // MFMA K-steps per stage
    static constexpr int ACC_PER_WAVE = WTM * WTN * 16 * 64;  // int32 per wave
    static_assert(WGM % EPI_H_ == 0, "wave-row groups");
    static constexpr int STAGED_ROWS = 32 * WGM / EPI_H_;   // epilogue rows per pass
    static constexpr int LDR = BN + 4;                // staged row pitch (int32), 4 mod 64 banks
    static constexpr int EPI_BYTES = DIRECT_EPI ? 0 : STAGED_ROWS * LDR * 4 + (BM + BN) * 4;
    static constexpr int LDS_BYTES = NST * STAGE > EPI_BYTES ? NST * STAGE : EPI_BYTES;
    static_assert(A_LOADS * ROWS_PER_FILL * NW == BM && B_LOADS * ROWS_PER_FILL * NW == BN,
                  "fills must cover the tile");
    static_assert(NST >= 2 && NST <= 4, "pipeline depth");
    static_assert(DIRECT_EPI || (STAGED_ROWS * (BN / 4)) % THREADS == 0, "epilogue sweep");
    static constexpr int PF_BYTES = PREFETCH ? 512 : 0;  // landing area of the L2 touches
    static_assert(LDS_BYTES + PF_BYTES <= 160 * 1024, "LDS per workgroup");
    static_assert(!PREFETCH || (NST == 2 && BM == 256 && BN % 8 == 0 && BN / 8 <= 64),
                  "prefetch layout");
};

// One wave instruction that touches one L2 line per lane: each lane copies 4
// bytes from gbase + voff into LDS at lds + 4*lane, a landing area nobody
// reads.  Its only purpose is to bring the line into the XCD's L2.  M0 is
// passed as in lds_fill16, with the same wait state.
__device__ __forceinline__ void l2_touch4(const int8_t* gbase, uint32_t voff, lds_i8* lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(gbase), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ void wait_fills() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One v_mfma_i32_32x32x32_i8 on a 32x32 int32 tile: c += w_frag * x_frag^T,
// i.e. the weight rows index the tile's first dimension (see the layout note
// at the top).  The builtin lets the compiler place the accumulator and
// insert the wait states its result needs; the scheduling barrier after it
// keeps the instruction order of the main loop as written in the source
// (MFMAs interleaved with LDS reads and fills).
__device__ __forceinline__ void mfma_32x32x32_i8(i32x16& c, const i32x4& x_frag, const i32x4& w_frag) {
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(w_frag, x_frag, c, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Generous wait states after the last MFMA before its results are read by
// other instructions (an MFMA written in inline asm is not tracked by the
// compiler's hazard recognizer in every case).
__device__ __forceinline__ void mfma_drain() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Chunks per thread whose LDS reads are issued before the first store of a
// sweep batch in the 16x16x64 configurations (at most; the largest divisor of
// the chunks per pass).
constexpr int MF16_SWEEP_BATCH = 8;

constexpr int largest_divisor_upto(int n, int cap) {
    int d = cap < n ? cap : n;
    while (d > 1 && n % d != 0) --d;
    return d;
}

// Keeps the scheduler from mixing the work of neighbouring output tiles,
// which bounds register pressure in the epilogue.
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// Swizzle of the 16-byte chunk index inside an LDS row of CHUNKS chunks.
// For 128-byte rows a 128-bit LDS read is served 32 lanes at a time over a
// 512-byte window (four rows): the swizzle is constant on row pairs and
// steps through 0..7 over rows 0..15, so the 16 rows of a fragment read at
// two neighbouring logical chunks hit 32 distinct 16-byte bank groups, and
// any 16 of those lanes hit 16 distinct groups of a 256-byte window.
template <int CHUNKS>
__device__ __forceinline__ int row_swz(int r) {
    if constexpr (CHUNKS == 8) return ((r >> 2) & 3) * 2 + ((r >> 1) & 1);
    else return ((r >> 1) & 3) ^ (((r >> 3) & 1) * 3);
}

template <class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void gemm_tiled(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ B,
    const float* __restrict__ sw, const float* residual, float* y, int M, int N, int K,
    int tiles_m, int tiles_n, int group_m, int splitk, int kb_per_split,
    int32_t* __restrict__ partials, int stream_out) {
    constexpr int WTM = C::WTM, WTN = C::WTN, BK = C::BK, NST = C::NST;
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS_BYTES + C::PF_BYTES];

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

    const int row0 = tm * C::BM;
    const int col0 = tn * C::BN;
    const int KB = K >> 6;                       // 64-byte k-blocks
    const int kb0 = min(split * kb_per_split, KB);
    const int kb1 = min(kb0 + kb_per_split, KB);
    const int nkb = kb1 - kb0;
    constexpr int KB_PER_STAGE = BK / 64;
    const int nst = (nkb + KB_PER_STAGE - 1) / KB_PER_STAGE;
    const bool half_last = (nkb % KB_PER_STAGE) != 0;   // only with BK = 128

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = wave / C::WGN, wn = wave % C::WGN;

    // ---- LDS fills.  Instruction j of wave w fills LDS rows RPF*(w + NW*j) ..
    // +RPF-1 (RPF = rows per fill, 1 KiB); lane l lands in row
    // RPF*(w + NW*j) + l / CHUNKS at physical chunk l % CHUNKS, which holds
    // logical chunk (l % CHUNKS) ^ swz(row).  With NW even, the swizzle of
    // that row depends on the lane alone (RPF*NW is a multiple of 16).
    // Per-lane byte offsets (rows past the end of the matrix clamped to its
    // last row) are computed once; a stage then costs two scalar adds per
    // operand, and one fill instruction about four instructions, so that a
    // fill fits in the issue slots of one MFMA.
    static_assert(C::NW % 2 == 0, "fill swizzle must not depend on the fill index");
    constexpr int RPF = C::ROWS_PER_FILL;
    const int lrow = lane / C::CHUNKS;
    const int lchunk = (lane % C::CHUNKS) ^ row_swz<C::CHUNKS>(RPF * wave + lrow);
    const uint32_t koff = static_cast<uint32_t>(lchunk * 16);
    // A half stage (BK = 128, odd number of k-blocks) must not read past the
    // chunk or the matrix: lanes of the upper half re-read the lower half,
    // whose bytes are valid and are never multiplied.
    const uint32_t half_adj = lchunk >= 4 ? 64u : 0u;
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j) {
        const int gr = min(row0 + RPF * (wave + C::NW * j) + lrow, M - 1);
        a_off[j] = static_cast<uint32_t>(gr - row0) * static_cast<uint32_t>(K) + koff;
    }
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
        const int gc = min(col0 + RPF * (wave + C::NW * j) + lrow, N - 1);
        b_off[j] = static_cast<uint32_t>(gc - col0) * static_cast<uint32_t>(K) + koff;
    }
    const int8_t* a_tile = A + static_cast<int64_t>(row0) * K + kb0 * 64;
    const int8_t* b_tile = B + static_cast<int64_t>(col0) * K + kb0 * 64;
    lds_i8* const l_wave = (lds_i8*)smem + RPF * wave * BK;

    // Where stage st goes: scalar sources, this wave's LDS slice of buffer
    // buf, and the half-stage lane adjustment.
    struct FillStage {
        const int8_t* ga;
        const int8_t* gb;
        lds_i8* l;
        uint32_t adj;
    };
    auto fill_stage = [&](int st, int buf) -> FillStage {
        const bool half = half_last && (st == nst - 1);
        return FillStage{a_tile + st * BK, b_tile + st * BK, l_wave + buf * C::STAGE,
                         half ? half_adj : 0u};
    };
    // Fill instruction d of a stage: the A fills, then the B fills.
    auto issue_one = [&](const FillStage& f, int d) {
        if (d < C::A_LOADS) {
            lds_fill16(f.ga, a_off[d] - f.adj, f.l + RPF * C::NW * d * BK);
        } else {
            const int e = d - C::A_LOADS;
            lds_fill16(f.gb, b_off[e] - f.adj, f.l + C::A_BYTES + RPF * C::NW * e * BK);
        }
    };
    auto issue = [&](int st, int buf) {
        const FillStage f = fill_stage(st, buf);
#pragma unroll
        for (int d = 0; d < C::LPS; ++d) issue_one(f, d);
    };

    // ---- per-lane LDS read offsets for the MFMA operands.  Fragment i of this
    // wave covers rows wm*32*WTM + 32*i + (lane & 31); K sub-step s (32 bytes)
    // uses logical chunk 2s + (lane >> 5).  Those rows are congruent to
    // lane & 15 modulo 16, which fixes the swizzle.
    const int rsw = row_swz<C::CHUNKS>(lane & 15);
    const int a_row_off = (wm * 32 * WTM + (lane & 31)) * BK;
    const int b_row_off = (wn * 32 * WTN + (lane & 31)) * BK;
    int chunk_off[C::SUBSTEPS];
#pragma unroll
    for (int s = 0; s < C::SUBSTEPS; ++s) chunk_off[s] = ((2 * s + (lane >> 5)) ^ rsw) * 16;

    // Accumulators: WTM x WTN tiles of 32x32 (16 int32 per lane each), or
    // with 16x16x64 MFMAs 2*WTM x 2*WTN tiles of 16x16 (4 int32 per lane).
    constexpr int AM = C::MF16 ? 2 * WTM : WTM, AN = C::MF16 ? 2 * WTN : WTN;
    using AccV = typename std::conditional<C::MF16, i32x4, i32x16>::type;
    constexpr int AE = C::MF16 ? 4 : 16;
    AccV acc[AM][AN];
#pragma unroll
    for (int i = 0; i < AM; ++i)
#pragma unroll
        for (int j = 0; j < AN; ++j)
#pragma unroll
            for (int e = 0; e < AE; ++e) acc[i][j][e] = 0;

    // Fragments of one 32-byte K sub-step: WTM activation and WTN weight
    // fragments, 16 bytes per lane each.
    struct Frags {
        i32x4 a[WTM], b[WTN];
    };
    // ---- 16x16x64 fragments (MF16).  Fragment q of 16 rows starting at row
    // wm*32*WTM + 16*q (activations) or wn*32*WTN + 16*q (weights); in
    // K-block u of the 128-byte stage, lane l reads row (l & 15), logical
    // chunk 4u + (l >> 4).  The held set is the smaller of the two.
    constexpr int MF_FA = 2 * WTM, MF_FB = 2 * WTN;
    constexpr bool MF_HOLD_B = MF_FB <= MF_FA;
    constexpr int MF_NH = MF_HOLD_B ? MF_FB : MF_FA;
    constexpr int MF_NS = MF_HOLD_B ? MF_FA : MF_FB;
    constexpr int MF_FILL_EVERY = MF_NS * MF_NH / C::LPS > 1 ? MF_NS * MF_NH / C::LPS : 1;
    // product group of K-block 0 that reads the first held fragment of K-block 1
    constexpr int MF_H1_FIRST = MF_NS - MF_NH - 1 > 0 ? MF_NS - MF_NH - 1 : 0;
    static_assert(MF_NS >= MF_NH && MF_H1_FIRST + MF_NH <= MF_NS, "held reads of K-block 1 inside K-block 0");
    const int mf_sw = row_swz<C::CHUNKS>(lane & 15);
    const int mf_c0 = (((lane >> 4)) ^ mf_sw) * 16, mf_c1 = ((4 + (lane >> 4)) ^ mf_sw) * 16;
    const int mf_a = (wm * 32 * WTM + (lane & 15)) * BK, mf_b = (wn * 32 * WTN + (lane & 15)) * BK;
    auto mf_frag = [&](const int8_t* la, const int8_t* lb, bool is_b, int q, int u) __attribute__((always_inline)) {
        const int8_t* base = is_b ? lb + mf_b : la + mf_a;
        return *reinterpret_cast<const i32x4*>(base + q * 16 * BK + (u ? mf_c1 : mf_c0));
    };
    auto mf_held = [&](const int8_t* la, const int8_t* lb, int q, int u) __attribute__((always_inline)) {
        return mf_frag(la, lb, MF_HOLD_B, q, u);
    };
    auto mf_strm = [&](const int8_t* la, const int8_t* lb, int q, int u) __attribute__((always_inline)) {
        return mf_frag(la, lb, !MF_HOLD_B, q, u);
    };
    // product (streamed o, held k); the weight fragment is the first operand,
    // so lane l's four results are four adjacent columns of row l & 15
    auto mf_mma = [&](int o, int k, const i32x4& sv, const i32x4& hv) __attribute__((always_inline)) {
        if constexpr (C::MF16) {
            if constexpr (MF_HOLD_B) acc[o][k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(hv, sv, acc[o][k], 0, 0, 0);
            else acc[k][o] = __builtin_amdgcn_mfma_i32_16x16x64_i8(sv, hv, acc[k][o], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto load_frag = [&](Frags& f, const int8_t* la, const int8_t* lb, int s, int q) {
        if (q < WTM)
            f.a[q] = *reinterpret_cast<const i32x4*>(la + a_row_off + q * 32 * BK + chunk_off[s]);
        else
            f.b[q - WTM] =
                *reinterpret_cast<const i32x4*>(lb + b_row_off + (q - WTM) * 32 * BK + chunk_off[s]);
    };
    // ---- main loop: NST - 1 stages in flight.  At iteration st the wave waits
    // until its copies of stage st have landed (later stages may still be
    // pending); the barrier publishes stage st to every wave and frees the
    // buffer of stage st - 1, into which stage st + NST - 1 is copied while
    // stage st is multiplied.
    //
    // Instruction schedule of one stage (the MFMA is inline asm with a memory
    // clobber, so MFMAs, LDS reads and fills stay in this order): after each
    // MFMA of sub-step s the wave issues one LDS read of a sub-step s+1
    // fragment and, during the first sub-steps, one fill instruction of the
    // next stage.  Those issue in the shadow of the running MFMA instead of
    // stalling the matrix core in a block of their own.
    if constexpr (NST >= 3 && !C::MF16) {
        // Publish-ahead pipeline (64-byte stages).  The barrier of iteration
        // st publishes stage st+1 and frees the buffer of stage st-1, into
        // which stage st + NST - 1 is copied.  The first fragments of each
        // stage are read during the previous stage's last MFMAs, so no stage
        // starts with the matrix core waiting on LDS.
        static_assert(C::SUBSTEPS == 2, "publish-ahead pipeline uses 64-byte stages");
#pragma unroll
        for (int p = 0; p < NST - 1; ++p)
            if (p < nst) issue(p, p);
        Frags f0, f1;
        if (nst > 0) {
            const int pend0 = min(NST - 2, nst - 1);              // stages issued after stage 0
            if (pend0 >= 2) wait_vm<2 * C::LPS>();
            else if (pend0 == 1) wait_vm<C::LPS>();
            else wait_vm<0>();
            __syncthreads();
            const int8_t* la = smem;
#pragma unroll
            for (int q = 0; q < WTM + WTN; ++q) load_frag(f0, la, la + C::A_BYTES, 0, q);
        }
        for (int st = 0; st < nst; ++st) {
            const bool more = st + 1 < nst;
            const bool fill = st + NST - 1 < nst;
            if (more) {
                const int pend = min(st + NST - 2, nst - 1) - (st + 1);   // issued after st+1
                if constexpr (NST >= 4) {
                    if (pend >= 1) wait_vm<C::LPS>();
                    else wait_vm<0>();
                } else {
                    wait_vm<0>();
                }
                __syncthreads();
            }
            const int8_t* la = smem + (st % NST) * C::STAGE;
            const int8_t* lb = la + C::A_BYTES;
            const int8_t* la_n = smem + ((st + 1) % NST) * C::STAGE;
            const int8_t* lb_n = la_n + C::A_BYTES;
            const FillStage fs = fill_stage(st + NST - 1, (st + NST - 1) % NST);
            int q = 0, d = 0;
            // sub-step 0: MFMAs on f0; read sub-step 1 into f1; copy stage st+NST-1
#pragma unroll
            for (int i = 0; i < WTM; ++i) {
#pragma unroll
                for (int j = 0; j < WTN; ++j) {
                    mfma_32x32x32_i8(acc[i][j], f0.a[i], f0.b[j]);
                    if (q < WTM + WTN) load_frag(f1, la, lb, 1, q++);
                    if (d < C::LPS) {
                        if (fill) issue_one(fs, d);
                        ++d;
                    }
                }
            }
#pragma unroll
            for (; q < WTM + WTN; ++q) load_frag(f1, la, lb, 1, q);
#pragma unroll
            for (; d < C::LPS; ++d)
                if (fill) issue_one(fs, d);
            // sub-step 1: MFMAs on f1; read the next stage's sub-step 0 into f0
            q = 0;
#pragma unroll
            for (int i = 0; i < WTM; ++i) {
#pragma unroll
                for (int j = 0; j < WTN; ++j) {
                    mfma_32x32x32_i8(acc[i][j], f1.a[i], f1.b[j]);
                    // (q advances unconditionally so every register index
                    // stays a compile-time constant)
                    if (q < WTM + WTN) {
                        if (more) load_frag(f0, la_n, lb_n, 0, q);
                        ++q;
                    }
                }
            }
#pragma unroll
            for (; q < WTM + WTN; ++q)
                if (more) load_frag(f0, la_n, lb_n, 0, q);
        }
    } else {
        // ---- L2 prefetch (PREFETCH configurations).  The copies of a stage
        // mostly miss in L2: the workgroups of an XCD run in step, so the
        // ones sharing an operand panel request its lines together and all
        // wait for the memory-side cache.  Here, PF_DIST stages ahead, wave 0
        // touches one line per row of a quarter of the tile's activation rows
        // (quarter tn % 4) and wave 1 of an eighth of its weight rows (eighth
        // tm % 8).  Tiles are rastered 8 tile rows by consecutive tile
        // columns per XCD, so the workgroups that share a panel split its
        // rows between them instead of each touching all of them.  A touch
        // is issued after the stage's copies, and waves 0 and 1 wait for all
        // but their last vector-memory operation, so nothing waits on a
        // touch until it is a stage old.  One line per row: with
        // K % 128 == 64 half the rows' stage slices straddle two lines and
        // only the first is touched.
        constexpr int PF_DIST = 2;
        const bool pf_wave = C::PREFETCH && wave < 2;
        const int8_t* pf_base = a_tile;
        uint32_t pf_off = 0;
        lds_i8* const pf_lds = (lds_i8*)smem + C::LDS_BYTES + 256 * (wave & 1);
        if (pf_wave) {
            if (wave == 0) {
                const int gr = min(row0 + (tn & 3) * (C::BM / 4) + lane % (C::BM / 4), M - 1);
                pf_off = static_cast<uint32_t>(gr - row0) * static_cast<uint32_t>(K);
            } else {
                const int gc = min(col0 + (tm & 7) * (C::BN / 8) + lane % (C::BN / 8), N - 1);
                pf_base = b_tile;
                pf_off = static_cast<uint32_t>(gc - col0) * static_cast<uint32_t>(K);
            }
        }
        auto prefetch = [&](int st) __attribute__((always_inline)) {
            l2_touch4(pf_base + min(st, nst - 1) * BK, pf_off, pf_lds);
        };
        if (pf_wave && nst > 0) {
#pragma unroll
            for (int p = 1; p < PF_DIST; ++p) prefetch(p);
        }
    #pragma unroll
        for (int p = 0; p < NST - 1; ++p)
            if (p < nst) issue(p, p);
        if constexpr (C::MF16) {
        // ---- 16x16x64 MFMAs.  A 64-byte K-block of the stage takes 2*WTM x
        // 2*WTN products.  The smaller fragment set (held) is read at the start
        // of the K-block (the second K-block's one fragment per product group
        // during the first); the larger (streamed) passes through a ring of
        // three, read two product groups ahead in the shadow of a product.
        // Product group o multiplies streamed fragment o by every held one.
        // The copies of the next stage are spread evenly over the first
        // K-block's products (in a burst, or over the whole stage, they
        // measured 6-10% slower).  The barrier that publishes the next stage
        // comes two product groups before the end of the stage: by then every
        // LDS read of the stage has been issued (the barrier waits for them),
        // so the next stage's first fragments are read while the last two
        // groups multiply, and the matrix pipe does not idle at the stage
        // boundary.
        i32x4 h[2][MF_NH];
        i32x4 sr[3];
        i32x4 nx[2];   // the next stage's first two streamed fragments
        if (nst > 0) {
            wait_vm<0>();
            __syncthreads();
    #pragma unroll
            for (int q = 0; q < MF_NH; ++q) h[0][q] = mf_held(smem, smem + C::A_BYTES, q, 0);
            sr[0] = mf_strm(smem, smem + C::A_BYTES, 0, 0);
            sr[1] = mf_strm(smem, smem + C::A_BYTES, 1 % MF_NS, 1 / MF_NS);
        }
        for (int st = 0; st < nst; ++st) {
            const bool more = st + 1 < nst;
            const FillStage fs = fill_stage(min(st + 1, nst - 1), (st + 1) % 2);
            const int8_t* la = smem + (st % 2) * C::STAGE;
            const int8_t* lb = la + C::A_BYTES;
            const int8_t* la_n = smem + ((st + 1) % 2) * C::STAGE;
            const int8_t* lb_n = la_n + C::A_BYTES;
            const int nkb_st = (half_last && st == nst - 1) ? 1 : 2;
            if (st > 0) {
                sr[0] = nx[0];
                sr[1] = nx[1];
            }
            int d = 0;   // copies of the next stage issued so far
    #pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (u >= nkb_st) break;
                if ((u == 0) == (wave >= C::NW / 2)) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int o = 0; o < MF_NS; ++o) {
                    const int g = u * MF_NS + o;   // running index over the stage
                    if (u == nkb_st - 1 && o == MF_NS - 2) {
                        // publish the next stage: its copies have landed (the
                        // touch of the L2 prefetch may still be in flight)
                        while (d < C::LPS) issue_one(fs, d++);
                        if (pf_wave) prefetch(st + PF_DIST);
                        if (pf_wave) wait_vm<1>();
                        else wait_vm<0>();
                        __syncthreads();
                        if (more) {   // (never in a short last stage, whose products use h[0])
    #pragma unroll
                            for (int q = 0; q < MF_NH; ++q) h[0][q] = mf_held(la_n, lb_n, q, 0);
                            nx[0] = mf_strm(la_n, lb_n, 0, 0);
                            nx[1] = mf_strm(la_n, lb_n, 1 % MF_NS, 1 / MF_NS);
                        }
                    }
                    const i32x4 cur = sr[g % 3];
                    if (u == 0 && nkb_st > 1) {
    #pragma unroll
                        for (int q = 0; q < MF_NH; ++q)
                            if (o == MF_H1_FIRST + q) h[1][q] = mf_held(la, lb, q, 1);
                    }
    #pragma unroll
                    for (int k = 0; k < MF_NH; ++k) {
                        mf_mma(o, k, cur, h[u][k]);
                        if (k == 0 && g + 2 < 2 * MF_NS && (g + 2) / MF_NS < nkb_st)
                            sr[(g + 2) % 3] = mf_strm(la, lb, (g + 2) % MF_NS, (g + 2) / MF_NS);
                        if ((g * MF_NH + k) % MF_FILL_EVERY == 0 && d < C::LPS) issue_one(fs, d++);
                    }
                }
            }
        }
        } else {
        for (int st = 0; st < nst; ++st) {
            const int pending = min(st + NST - 2, nst - 1) - st;   // stages issued after st
            if constexpr (NST >= 4) {
                if (pending >= 2) wait_vm<2 * C::LPS>();
                else if (pending == 1) wait_vm<C::LPS>();
                else wait_vm<0>();
            } else if constexpr (NST == 3) {
                if (pending >= 1) wait_vm<C::LPS>();
                else wait_vm<0>();
            } else {
                // the touch of the previous stage may still be in flight
                if (pf_wave && st > 0) wait_vm<1>();
                else wait_vm<0>();
            }
            __syncthreads();
            // The copy of stage st + NST - 1 is issued unconditionally, with
            // the stage clamped to the last one: past the end it re-reads
            // bytes in bounds into a buffer nobody reads again, which keeps
            // a branch out of every fill.  All copies land before the
            // epilogue reuses the LDS (wait_fills after the loop).
            const FillStage fs = fill_stage(min(st + NST - 1, nst - 1), (st + NST - 1) % NST);
            const int8_t* la = smem + (st % NST) * C::STAGE;
            const int8_t* lb = la + C::A_BYTES;
            int d = 0;   // fill instructions issued so far in this stage
            {
            const int nsub = (half_last && st == nst - 1) ? 2 : C::SUBSTEPS;
            Frags f[2];
    #pragma unroll
            for (int q = 0; q < WTM + WTN; ++q) load_frag(f[0], la, lb, 0, q);
    #pragma unroll
            for (int s = 0; s < C::SUBSTEPS; ++s) {
                if (s >= nsub) break;
                const Frags& cur = f[s & 1];
                Frags& nxt = f[(s + 1) & 1];
                int q = 0;   // next-sub-step fragments issued so far
                // Waves w and w + NW/2 share a SIMD and its matrix pipe.  The
                // arbiter favours the older wave, which would run its whole
                // stage first and leave the younger one to finish alone (a
                // lone wave cannot keep the pipe full) while it waits at the
                // barrier.  Taking turns at priority, the younger wave in the
                // first half of the stage and the older in the second, keeps
                // the two in step.
                if ((s < C::SUBSTEPS / 2) == (wave >= C::NW / 2)) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int i = 0; i < WTM; ++i) {
    #pragma unroll
                    for (int j = 0; j < WTN; ++j) {
                        mfma_32x32x32_i8(acc[i][j], cur.a[i], cur.b[j]);
                        if (s + 1 < C::SUBSTEPS && q < WTM + WTN) load_frag(nxt, la, lb, s + 1, q++);
                        if (d < C::LPS) issue_one(fs, d++);
                    }
                }
                if (s + 1 < C::SUBSTEPS) {
                    while (q < WTM + WTN) load_frag(nxt, la, lb, s + 1, q++);
                }
            }
            }   // 32x32x32 stage body
            while (d < C::LPS) issue_one(fs, d++);
            if (pf_wave) prefetch(st + PF_DIST);
        }
        }   // 32x32x32 loop
    }
    __builtin_amdgcn_s_setprio(0);
    mfma_drain();
    wait_fills();

    // ---- integer split-K: this chunk's raw int32 partial goes, row-major,
    // to slice `split` of the workspace instead of the epilogue
    int32_t* part = partials ? partials + static_cast<size_t>(split) * static_cast<size_t>(M) *
                                              static_cast<size_t>(N)
                             : nullptr;

    if constexpr (C::DIRECT_EPI) {
        // ---- epilogue straight from the accumulators: every lane writes four
        // adjacent outputs of its row per 16-byte store.  No LDS, no barrier.
        const bool vec_ok = (N & 3) == 0 &&
                            (part || ((reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                                      (reinterpret_cast<uintptr_t>(residual) & 15) == 0));
        // Weight scales are loaded per column fragment (16 per lane) so that
        // wide tiles do not hold WTN x 16 of them beside the accumulators.
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
            float swv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int col = col0 + wn * 32 * WTN + j * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                swv[e] = part ? 0.0f : sw[min(col, N - 1)];
            }
#pragma unroll
            for (int i = 0; i < WTM; ++i) {
                const int row = row0 + wm * 32 * WTM + i * 32 + (lane & 31);
                if (row >= M) continue;
                const float sxm = part ? 0.0f : sx[row];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = col0 + wn * 32 * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                    const size_t o = static_cast<size_t>(row) * N + col;
                    const i32x4 a = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                     acc[i][j][4 * g + 3]};
                    if (vec_ok && col + 3 < N) {
                        if (part) {
                            *reinterpret_cast<i32x4*>(part + o) = a;
                            continue;
                        }
                        float4 v;
                        if (residual) {
                            const float4 r4 = *reinterpret_cast<const float4*>(residual + o);
                            v.x = scale_acc_residual(a[0], sxm, swv[4 * g], r4.x);
                            v.y = scale_acc_residual(a[1], sxm, swv[4 * g + 1], r4.y);
                            v.z = scale_acc_residual(a[2], sxm, swv[4 * g + 2], r4.z);
                            v.w = scale_acc_residual(a[3], sxm, swv[4 * g + 3], r4.w);
                        } else {
                            v.x = scale_acc(a[0], sxm, swv[4 * g]);
                            v.y = scale_acc(a[1], sxm, swv[4 * g + 1]);
                            v.z = scale_acc(a[2], sxm, swv[4 * g + 2]);
                            v.w = scale_acc(a[3], sxm, swv[4 * g + 3]);
                        }
                        store_out4(y + o, v, stream_out);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (col + q >= N) continue;
                            if (part) part[o + q] = a[q];
                            else y[o + q] = residual ? scale_acc_residual(a[q], sxm, swv[4 * g + q], residual[o + q])
                                                     : scale_acc(a[q], sxm, swv[4 * g + q]);
                        }
                    }
                }
                sched_fence();
            }
        }
    } else {
        // ---- epilogue, in WTM * EPI_H passes of STAGED_ROWS rows.  In pass
        // (i, h) every wave of wave-row group h parks slice i (32 rows) of its
        // accumulators in LDS (row-major int32, four adjacent columns per
        // 16-byte write; rows padded by 4 words so that the 16 lanes of one
        // write phase, 16 different rows, hit 16 different bank groups).  Then
        // all threads sweep the parked rows in float4 chunks along rows (chunk
        // c of the pass is parked row c / (BN/4), column chunk c % (BN/4)),
        // one 16-byte residual load and one 16-byte output store per chunk,
        // whole rows per wave instruction.
        constexpr int LDR = C::LDR;
        constexpr int H = C::EPI_H;
        constexpr int WRP = C::WGM / H;                    // wave rows parked per pass
        int32_t* stage = reinterpret_cast<int32_t*>(smem);
        float* s_sx = reinterpret_cast<float*>(smem + C::STAGED_ROWS * LDR * 4);
        float* s_sw = s_sx + C::BM;
        __syncthreads();  // all waves are done reading the operand buffers
        if (!part) {   // raw int32 output reads no scales
            for (int t = threadIdx.x; t < C::BM; t += C::THREADS) s_sx[t] = sx[min(row0 + t, M - 1)];
            for (int t = threadIdx.x; t < C::BN; t += C::THREADS) s_sw[t] = sw[min(col0 + t, N - 1)];
        }

        // (a partial slice starts 16-byte aligned whenever N % 4 == 0: the
        // workspace is 256-byte aligned)
        const bool vec_ok = (N & 3) == 0 &&
                            (part || ((reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                                      (reinterpret_cast<uintptr_t>(residual) & 15) == 0));
        constexpr int C4 = C::BN / 4;                      // float4 chunks per staged row
        constexpr int CPT = C::STAGED_ROWS * C4 / C::THREADS;   // chunks per thread per pass
        // chunks read from LDS before the first store of a batch (bounded so
        // that the batch fits beside the accumulators still held)
        constexpr int KB = C::MF16 ? largest_divisor_upto(CPT, MF16_SWEEP_BATCH) : CPT <= 8 ? CPT : (CPT % 2 == 0 ? 2 : 1);
        static_assert(CPT % KB == 0, "sweep batches");
        // 16x16x64 accumulators: in every pass each wave parks PT of its
        // 16-row tiles (staged rows (wm * PT + q) * 16 + (lane & 15)), so every
        // wave frees accumulator registers from the first pass on and the
        // sweeps have room for larger batches.
        constexpr int PT = C::MF16 ? C::STAGED_ROWS / (16 * C::WGM) : 1;
        constexpr int NPASS = C::MF16 ? 2 * WTM / PT : WTM * H;
        static_assert(!C::MF16 || (PT >= 1 && C::STAGED_ROWS == 16 * C::WGM * PT && (2 * WTM) % PT == 0),
                      "16-row parking");
        // staged row r of pass (i, h) is tile row (h * WRP + r / 32) * 32 * WTM + i * 32 + r % 32
        auto tile_row = [](int r, int i, int h) { return (h * WRP + (r >> 5)) * 32 * WTM + i * 32 + (r & 31); };
        // Interior tile with aligned rows: a straight-line sweep, the LDS reads
        // of a batch issued before its first store.  Otherwise the checked
        // loop below.
        const bool fast = vec_ok && row0 + C::BM <= M && col0 + C::BN <= N;
        // Pass (i, h) with wrp wave rows per pass: the waves of wave-row
        // group h park accumulator slice i (32 rows of each wave).
        auto park = [&](int i, int h, int wrp) __attribute__((always_inline)) {
            if (wm / wrp != h) return;
            if constexpr (C::MF16) {
                // 16-row tiles 2i and 2i+1 of this wave -> staged rows
                // (wm % wrp) * 32 + 16 * hh + (lane & 15)
    #pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int lr = (wm % wrp) * 32 + 16 * hh + (lane & 15);
    #pragma unroll
                    for (int j = 0; j < 2 * WTN; ++j) {
                        const int lc = wn * 32 * WTN + j * 16 + 4 * (lane >> 4);
                        *reinterpret_cast<i32x4*>(stage + lr * LDR + lc) = acc[2 * i + hh][j];
                    }
                    sched_fence();
                }
            } else {
                // accumulator slice i of this wave -> staged rows (wm % wrp) * 32 + r
                const int lr = (wm % wrp) * 32 + (lane & 31);
    #pragma unroll
                for (int j = 0; j < WTN; ++j) {
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int lc = wn * 32 * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                        *reinterpret_cast<i32x4*>(stage + lr * LDR + lc) =
                            i32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                  acc[i][j][4 * g + 3]};
                    }
                    sched_fence();
                }
            }
        };

        // ---- residual epilogue of an interior tile.  Here the sweep needs
        // the residual, and a wave's vector-memory counter retires in order:
        // a residual load issued after the wave's stores can only be waited
        // for together with those stores, which made every batch of the
        // sweep wait for the previous batch's writes to complete.  Instead
        // the residual of the next pass is copied into LDS
        // (global_load_lds_dwordx4, each lane the chunks it will use itself)
        // before this pass's stores, so a pass waits only for the previous
        // pass's stores, issued a whole pass earlier.  Passes are half as
        // tall (RH = 2H groups of one wave row) so that the parking area, the
        // scales and two residual buffers fit in the LDS.
        constexpr int RH = 2 * H;
        constexpr int RROWS = 32 * C::WGM / RH;                // staged rows per pass
        constexpr int RCPT = RROWS * C4 / C::THREADS;          // chunks per thread per pass
        constexpr int RES_BYTES = RROWS * C::BN * 4;           // one pass of residual
        constexpr int RB0 = (RROWS * LDR * 4 + 511) / 512 * 512;
        constexpr int RB1 = ((C::STAGED_ROWS * LDR + C::BM + C::BN) * 4 + 511) / 512 * 512;
        constexpr bool RES_LDS = C::MF16 && C::WGM % RH == 0 && RROWS == 32 &&
                                 RROWS * C4 % C::THREADS == 0 && RB0 + RES_BYTES <= C::STAGED_ROWS * LDR * 4 &&
                                 RB1 + RES_BYTES <= C::LDS_BYTES;
        if constexpr (RES_LDS) {
            // (every lane offset below stays under 2^32 bytes from the tile's first row)
            if (fast && residual && !part && static_cast<int64_t>(C::BM) * N * 4 < (int64_t(1) << 32)) {
                const int8_t* res_tile = reinterpret_cast<const int8_t*>(residual + static_cast<size_t>(row0) * N);
                auto res_fill = [&](int pass) __attribute__((always_inline)) {
                    const int i = pass / RH, h = pass % RH;
                    lds_i8* const buf = (lds_i8*)smem + ((pass & 1) ? RB1 : RB0);
    #pragma unroll
                    for (int k = 0; k < RCPT; ++k) {
                        const int c = threadIdx.x + k * C::THREADS;
                        const int r = c / C4, c4 = c % C4;
                        const int lr = (h + (r >> 5)) * 32 * WTM + i * 32 + (r & 31);
                        const uint32_t off = (static_cast<uint32_t>(lr) * static_cast<uint32_t>(N) +
                                              static_cast<uint32_t>(col0 + 4 * c4)) * 4u;
                        lds_fill16(res_tile, off, buf + (k * C::THREADS + 64 * wave) * 16);
                    }
                };
                res_fill(0);
    #pragma unroll
                for (int pass = 0; pass < WTM * RH; ++pass) {
                    const int i = pass / RH, h = pass % RH;
                    park(i, h, 1);
                    __syncthreads();
                    // this pass's residual has landed (the previous pass's
                    // RCPT stores may still be in flight)
                    if (pass == 0) wait_vm<0>();
                    else wait_vm<RCPT>();
                    if (pass + 1 < WTM * RH) res_fill(pass + 1);
                    const float* rbuf = reinterpret_cast<const float*>(smem + ((pass & 1) ? RB1 : RB0));
    #pragma unroll
                    for (int k = 0; k < RCPT; ++k) {
                        const int c = threadIdx.x + k * C::THREADS;
                        const int r = c / C4, c4 = c % C4;
                        const int lr = (h + (r >> 5)) * 32 * WTM + i * 32 + (r & 31);
                        const i32x4 a = *reinterpret_cast<const i32x4*>(stage + r * LDR + 4 * c4);
                        const float4 r4 = *reinterpret_cast<const float4*>(rbuf + 4 * c);
                        const float sxm = s_sx[lr];
                        const float4 sw4 = *reinterpret_cast<const float4*>(s_sw + 4 * c4);
                        float4 v;
                        v.x = scale_acc_residual(a[0], sxm, sw4.x, r4.x);
                        v.y = scale_acc_residual(a[1], sxm, sw4.y, r4.y);
                        v.z = scale_acc_residual(a[2], sxm, sw4.z, r4.z);
                        v.w = scale_acc_residual(a[3], sxm, sw4.w, r4.w);
                        store_out4(y + static_cast<size_t>(row0 + lr) * N + col0 + 4 * c4, v, stream_out);
                        sched_fence();
                    }
                    __syncthreads();
                }
                return;
            }
        }

        auto park16 = [&](int pass) __attribute__((always_inline)) {
            if constexpr (C::MF16) {
    #pragma unroll
                for (int q = 0; q < PT; ++q) {
                    const int lr = (wm * PT + q) * 16 + (lane & 15);
    #pragma unroll
                    for (int j = 0; j < 2 * WTN; ++j) {
                        const int lc = wn * 32 * WTN + j * 16 + 4 * (lane >> 4);
                        *reinterpret_cast<i32x4*>(stage + lr * LDR + lc) = acc[pass * PT + q][j];
                    }
                    sched_fence();
                }
            }
        };
        // tile row of staged row r in pass `pass`
        auto trow = [&](int r, int pass) __attribute__((always_inline)) {
            if constexpr (C::MF16)
                return (r / (16 * PT)) * 32 * WTM + 16 * (pass * PT + (r / 16) % PT) + (r & 15);
            else
                return tile_row(r, pass / H, pass % H);
        };
    #pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            if constexpr (C::MF16) park16(pass);
            else park(pass / H, pass % H, WRP);
            __syncthreads();
            if (fast) {
    #pragma unroll
                for (int k0 = 0; k0 < CPT; k0 += KB) {
                    i32x4 av[KB];
                    float sxv[KB];
                    float4 swv[KB];
                    size_t ov[KB];
    #pragma unroll
                    for (int k = 0; k < KB; ++k) {
                        const int c = threadIdx.x + (k0 + k) * C::THREADS;
                        const int r = c / C4, c4 = c % C4;
                        const int lr = trow(r, pass);
                        av[k] = *reinterpret_cast<const i32x4*>(stage + r * LDR + 4 * c4);
                        sxv[k] = s_sx[lr];
                        swv[k] = *reinterpret_cast<const float4*>(s_sw + 4 * c4);
                        ov[k] = static_cast<size_t>(row0 + lr) * N + col0 + 4 * c4;
                    }
                    if (part) {
    #pragma unroll
                        for (int k = 0; k < KB; ++k) *reinterpret_cast<i32x4*>(part + ov[k]) = av[k];
                    } else if (residual) {
                        float4 rv[KB];
    #pragma unroll
                        for (int k = 0; k < KB; ++k) rv[k] = *reinterpret_cast<const float4*>(residual + ov[k]);
    #pragma unroll
                        for (int k = 0; k < KB; ++k) {
                            float4 v;
                            v.x = scale_acc_residual(av[k][0], sxv[k], swv[k].x, rv[k].x);
                            v.y = scale_acc_residual(av[k][1], sxv[k], swv[k].y, rv[k].y);
                            v.z = scale_acc_residual(av[k][2], sxv[k], swv[k].z, rv[k].z);
                            v.w = scale_acc_residual(av[k][3], sxv[k], swv[k].w, rv[k].w);
                            store_out4(y + ov[k], v, stream_out);
                        }
                    } else {
    #pragma unroll
                        for (int k = 0; k < KB; ++k) {
                            float4 v;
                            v.x = scale_acc(av[k][0], sxv[k], swv[k].x);
                            v.y = scale_acc(av[k][1], sxv[k], swv[k].y);
                            v.z = scale_acc(av[k][2], sxv[k], swv[k].z);
                            v.w = scale_acc(av[k][3], sxv[k], swv[k].w);
                            store_out4(y + ov[k], v, stream_out);
                        }
                    }
                    sched_fence();
                }
                __syncthreads();
                continue;
            }
            for (int c = threadIdx.x; c < C::STAGED_ROWS * C4; c += C::THREADS) {
                const int r = c / C4, c4 = c % C4;
                const int lr = trow(r, pass);
                const int row = row0 + lr;
                const int col = col0 + 4 * c4;
                if (row >= M) continue;
                const int4 a4 = *reinterpret_cast<const int4*>(stage + r * LDR + 4 * c4);
                const float sxm = s_sx[lr];
                const float4 sw4 = *reinterpret_cast<const float4*>(s_sw + 4 * c4);
                const size_t o = static_cast<size_t>(row) * N + col;
                if (vec_ok && col + 3 < N) {
                    if (part) {
                        *reinterpret_cast<int4*>(part + o) = a4;
                        continue;
                    }
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
                    store_out4(y + o, v, stream_out);
                } else {
                    const int32_t av[4] = {a4.x, a4.y, a4.z, a4.w};
                    const float swv[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (col + q >= N) continue;
                        if (part) part[o + q] = av[q];
                        else y[o + q] = residual ? scale_acc_residual(av[q], sxm, swv[q], residual[o + q])
                                                 : scale_acc(av[q], sxm, swv[q]);
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ---- split-K reduction and epilogue: y = epi(P_0 + P_1 + ... + P_{S-1}).
// An HBM-bound stream (4S bytes of partials (+4 of residual) read and 4
// written per output).  VEC: one thread per 4 consecutive outputs of a row,
// for N % 4 == 0 and 16-byte aligned float buffers; else one per output.
// The residual may be y itself: each output is read and written by the
// same thread.
constexpr int REDUCE_THREADS = 256;

template <bool VEC>
__global__ __launch_bounds__(REDUCE_THREADS) void splitk_reduce(
    const int32_t* __restrict__ P, int S, const float* __restrict__ sx,
    const float* __restrict__ sw, const float* residual, float* y, int64_t M, int64_t N, int stream_out) {
    const int64_t MN = M * N;
    const int64_t units = VEC ? MN / 4 : MN;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * REDUCE_THREADS;
    for (int64_t u = static_cast<int64_t>(blockIdx.x) * REDUCE_THREADS + threadIdx.x; u < units;
         u += stride) {
        if constexpr (VEC) {
            const int64_t o = 4 * u;
            const int64_t m = o / N;
            const int64_t n = o - m * N;
            i32x4 a = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(P + o));
#pragma unroll 4
            for (int c = 1; c < S; ++c)
                a += __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(P + c * MN + o));
            const float sxm = sx[m];
            const float4 sw4 = *reinterpret_cast<const float4*>(sw + n);
            float4 v;
            if (residual) {
                const float4 r4 = *reinterpret_cast<const float4*>(residual + o);
                v.x = scale_acc_residual(a[0], sxm, sw4.x, r4.x);
                v.y = scale_acc_residual(a[1], sxm, sw4.y, r4.y);
                v.z = scale_acc_residual(a[2], sxm, sw4.z, r4.z);
                v.w = scale_acc_residual(a[3], sxm, sw4.w, r4.w);
            } else {
                v.x = scale_acc(a[0], sxm, sw4.x);
                v.y = scale_acc(a[1], sxm, sw4.y);
                v.z = scale_acc(a[2], sxm, sw4.z);
                v.w = scale_acc(a[3], sxm, sw4.w);
            }
            store_out4(y + o, v, stream_out);
        } else {
            const int64_t m = u / N;
            const int64_t n = u - m * N;
            int32_t a = P[u];
            for (int c = 1; c < S; ++c) a += P[c * MN + u];
            y[u] = residual ? scale_acc_residual(a, sx[m], sw[n], residual[u])
                            : scale_acc(a, sx[m], sw[n]);
        }
    }
}

}  // namespace

static bool stream_output(const GemmArgs& a) { return a.M * a.N * 4 >= STREAM_OUT_BYTES; }

hipError_t launch_reduce(const GemmArgs& a, int S, const int32_t* partials, hipStream_t stream) {
    const int64_t MN = a.M * a.N;
    const bool vec = (a.N & 3) == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.sw) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.residual) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(partials) & 15) == 0;
    const int64_t units = vec ? MN / 4 : MN;
    // one unit per thread, up to 32 workgroups per CU (then a grid-stride
    // loop): small reductions are latency-bound, and one round of loads per
    // thread beat four (256 x 5120 at S = 4: 45.3 -> 43.4 us for the whole
    // split-K product; 32 x 5120 at S = 8: 26.7 -> 23.4 us)
    const int64_t blocks = std::max<int64_t>(
        1, std::min<int64_t>((units + REDUCE_THREADS - 1) / REDUCE_THREADS, 256 * 32));
    if (vec)
        hipLaunchKernelGGL((splitk_reduce<true>), dim3(static_cast<unsigned>(blocks)),
                           dim3(REDUCE_THREADS), 0, stream, partials, S, a.sx, a.sw, a.residual,
                           a.y, a.M, a.N, static_cast<int>(stream_output(a)));
    else
        hipLaunchKernelGGL((splitk_reduce<false>), dim3(static_cast<unsigned>(blocks)),
                           dim3(REDUCE_THREADS), 0, stream, partials, S, a.sx, a.sw, a.residual,
                           a.y, a.M, a.N, static_cast<int>(stream_output(a)));
    return hipGetLastError();
}

namespace {

// The configurations, indexed by TileKind.
// 256x256, 4 waves of 128x128 on 16x16x64 MFMAs (256 accumulator registers
// a wave), 128-byte stages x2.  With 32x32x32 MFMAs this configuration spilled
// 308 bytes per lane and ran 4x slower; never chosen automatically (the 8-wave
// 256x256 configuration is faster), kept as a forced alternative.
using Cfg0 = Cfg<2, 2, 4, 4, 128, 2, 1, false, true, 2, true>;
using Cfg1 = Cfg<2, 4, 4, 2, 64, 4, 1>;   // 256x256, 8 waves, 64-byte stages x4
using Cfg2 = Cfg<2, 2, 4, 2, 64, 3, 2>;   // 256x128, 4 waves, 2 workgroups per CU
using Cfg3 = Cfg<2, 2, 2, 2, 64, 4, 2>;   // 128x128, 4 waves, 2 workgroups per CU
using Cfg4 = Cfg<2, 4, 4, 2, 128, 2, 1, false, true, 1, true>;  // 256x256, 8 waves, 128-byte stages x2
using Cfg5 = Cfg<2, 4, 4, 2, 128, 2, 1, true, true>;   // as 4, epilogue stored from the accumulators
// 256x320, 8 waves of 64x160, 128-byte stages x2, LDS-staged epilogue in
// two groups of wave rows (64 rows x 320 columns per pass): N = 5120 is 16
// such tiles, so M = 8192 makes 512 tiles, two full rounds on 256 CUs where
// 256x256 tiles make 2.5
using Cfg6 = Cfg<4, 2, 2, 5, 128, 2, 1, false, true, 2, true>;

template <class C>
hipError_t launch_cfg(const GemmArgs& a, const GemmPlan& p, void* workspace, hipStream_t stream) {
    const int64_t ntiles = p.tiles_m * p.tiles_n;
    const int KB = static_cast<int>(a.K >> 6);
    const int kb_per_split = (KB + p.splitk - 1) / p.splitk;
    int32_t* partials = a.acc_out ? a.acc_out : p.splitk > 1 ? static_cast<int32_t*>(workspace) : nullptr;
    const unsigned nblocks = static_cast<unsigned>(ntiles * p.splitk);
    hipLaunchKernelGGL((gemm_tiled<C>), dim3(nblocks), dim3(C::THREADS), 0, stream, a.xq, a.sx, a.w,
                       a.sw, a.residual, a.y, static_cast<int>(a.M), static_cast<int>(a.N),
                       static_cast<int>(a.K), static_cast<int>(p.tiles_m),
                       static_cast<int>(p.tiles_n), p.group_m, p.splitk, kb_per_split, partials,
                       static_cast<int>(stream_output(a)));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splitk <= 1 || a.acc_out) return e;
    return launch_reduce(a, p.splitk, partials, stream);
}

struct KindInfo {
    int bm, bn;
    int per_cu;     // workgroups resident per CU
    double weight;  // relative per-CU throughput of the shape (measured: with
                    // 16x16x64 MFMAs the 256x320 tile runs gate+up 8192x34816x5120
                    // 4% faster than 256x256 despite 14 rounds of 1.25x work)
};
// Same order as TileKind and the Cfg list.
const KindInfo kKinds[TILE_KINDS] = {
    {Cfg0::BM, Cfg0::BN, Cfg0::OCC, 0.95},
    {Cfg1::BM, Cfg1::BN, Cfg1::OCC, 0.93},
    {Cfg2::BM, Cfg2::BN, Cfg2::OCC, 0.85},
    {Cfg3::BM, Cfg3::BN, Cfg3::OCC, 0.70},
    {Cfg4::BM, Cfg4::BN, Cfg4::OCC, 1.00},
    {Cfg5::BM, Cfg5::BN, Cfg5::OCC, 0.97},
    {Cfg6::BM, Cfg6::BN, Cfg6::OCC, 1.07},
};

// Process-wide tuning hook; an atomic so that host threads may set and read
// it concurrently (a plan reads it once).
std::atomic<int> tile_override{-1};

}  // namespace

void set_tile_override(int kind) { tile_override.store(kind, std::memory_order_relaxed); }
int tile_override_value() { return tile_override.load(std::memory_order_relaxed); }

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int splitk) {
    (void)K;
    const int ncu = 256;
    int best = 0;
    double best_score = -1.0;
    for (int c = 0; c < TILE_KINDS; ++c) {
        const KindInfo& k = kKinds[c];
        const int64_t tm = (M + k.bm - 1) / k.bm;
        const int64_t tn = (N + k.bn - 1) / k.bn;
        const int64_t blocks = tm * tn * splitk;
        const int64_t slots = static_cast<int64_t>(ncu) * k.per_cu;
        const int64_t rounds = (blocks + slots - 1) / slots;
        // useful work over the slots the rounds occupy, times the shape's speed
        const double useful = static_cast<double>(M) * static_cast<double>(N) /
                              (static_cast<double>(tm * k.bm) * static_cast<double>(tn * k.bn));
        const double fill = static_cast<double>(blocks) / static_cast<double>(rounds * slots);
        const double score = useful * fill * k.weight;
        if (score > best_score + 1e-9) {
            best_score = score;
            best = c;
        }
    }
    const int ov = tile_override_value();
    if (ov >= 0 && ov < TILE_KINDS) best = ov;
    GemmPlan p;
    p.kind = static_cast<TileKind>(best);
    p.bm = kKinds[best].bm;
    p.bn = kKinds[best].bn;
    p.tiles_m = (M + p.bm - 1) / p.bm;
    p.tiles_n = (N + p.bn - 1) / p.bn;
    p.splitk = splitk;
    p.group_m = 8;
    return p;
}

double tiled_time_estimate_us(int64_t M, int64_t N, int64_t K, int splitk) {
    const GemmPlan p = plan_gemm(M, N, K, splitk);
    const KindInfo& k = kKinds[p.kind];
    const int64_t blocks = p.tiles_m * p.tiles_n * splitk;
    const int64_t slots = static_cast<int64_t>(256) * k.per_cu;
    const int64_t rounds = (blocks + slots - 1) / slots;
    const int64_t kps = (K / 64 + splitk - 1) / splitk * 64;
    // int8 operations per second per CU: 256x320 tiles sustain 10.1e12
    // (one round of 218 tiles at K = 5120 takes 91 us, 8 of them launch,
    // prologue and epilogue); the other configurations in proportion to
    // their weights above
    const double rate = 10.1e12 * k.weight / kKinds[TILE_KIND_6].weight;
    double t = static_cast<double>(rounds) * 2.0 * k.bm * k.bn * static_cast<double>(kps) * k.per_cu / rate + 8e-6;
    if (splitk > 1) t += 5e-6 + (4.0 * splitk + 8.0) * static_cast<double>(M) * static_cast<double>(N) / 4.0e12;
    return t * 1e6;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int splitk) {
    if (splitk <= 1) return 0;
    // S row-major int32 slices of the output, rounded up to 256 bytes
    const size_t bytes = static_cast<size_t>(splitk) * static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
    return (bytes + 255) / 256 * 256;
}

hipError_t launch_gemm_tiled(const GemmArgs& a, const GemmPlan& p, void* workspace,
                             hipStream_t stream) {
    switch (p.kind) {
        case 0: return launch_cfg<Cfg0>(a, p, workspace, stream);
        case 1: return launch_cfg<Cfg1>(a, p, workspace, stream);
        case 2: return launch_cfg<Cfg2>(a, p, workspace, stream);
        case 3: return launch_cfg<Cfg3>(a, p, workspace, stream);
        case 4: return launch_cfg<Cfg4>(a, p, workspace, stream);
        case 5: return launch_cfg<Cfg5>(a, p, workspace, stream);
        case 6: return launch_cfg<Cfg6>(a, p, workspace, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace w8a8
