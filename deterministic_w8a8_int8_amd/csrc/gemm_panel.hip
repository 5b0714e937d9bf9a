// Column-panel int8 x int8 -> int32 GEMM for mid-sized M (a few hundred
// tokens: one request, or a shared-evidence batch), with the same fixed
// binary32 epilogue as the other kernels.
//
// What it computes is defined on the review page "StartLux-Prism: Fast,
// exact inference for StartLux-Decision models on NVIDIA GPUs", section
// "Bitwise consistency is not lossless quantization": exact int32
// accumulation, integer split-K partials, and one fixed rounding sequence
// for the scales and the residual.
//
// Why a separate kernel.  With M of a few hundred rows, a 256x256 output
// tile per CU leaves most of the 256 CUs idle (N = 34816 is only 136 such
// tiles) and the weight stream, not the matrix cores, sets the time.  Here
// the output is cut into column panels sized so that the panels (times the
// row and K splits) match the CU count:
//   - one workgroup = 4 waves, one per SIMD, one workgroup per CU.  It owns
//     a panel of ncb <= NB blocks of 16 output columns, a range of rows
//     and a range of K;
//   - the 4 waves split the rows (mw <= MW blocks of 16 rows each) and all
//     of them sweep the whole panel, so every weight byte is fetched from
//     HBM once per workgroup and each activation row once per panel;
//   - the weight panel goes HBM -> VGPR -> LDS through a ring of 3 stages of
//     4 K-blocks (256 bytes of K per row).  A stage is loaded one stage
//     ahead and written to LDS at the end of the next stage, into the ring
//     slot freed by the barrier at its start.  16-byte chunks of a row are
//     XOR-swizzled with the row index, so the 16 rows one fragment read
//     touches hit distinct banks;
//   - activation fragments go HBM/L2 -> VGPR directly (each wave reads only
//     its own rows), two K-blocks ahead of their use;
//   - v_mfma_i32_16x16x64_i8 with the weight fragment as first operand: lane
//     l, element e of a 16x16 tile is output row (l % 16) and column
//     4*(l/16) + e, so each lane stores four adjacent outputs of one row with
//     one 16-byte store;
//   - integer accumulation is exact, so the lane -> k assignment (shared by
//     both operands), the panel widths, the row and K splits never change a
//     bit.  With K splits every workgroup writes its raw int32 partial to
//     its own slice of the workspace, and the split-K reduction kernel adds
//     the slices in order and runs the epilogue.
// All memory operations are ordinary loads and stores, so the compiler's
// own wait counts order them; nothing waits on a copy it does not need.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int NXCD = 8;             // XCDs on MI355X
constexpr int PANEL_THREADS = 256;  // 4 waves, one per SIMD
constexpr int KBS = 4;              // 64-byte K-blocks per LDS stage
constexpr int NSTB = 3;             // LDS ring stages
constexpr int ROW_BYTES = 64 * KBS; // bytes of one weight row in a stage
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: raw 32-bit data

struct PanelParams {
    int M, N, K;
    int P, cb_base, cb_extra;   // panels; panel p has cb_base + (p < cb_extra) column blocks
    int R, rb_total;            // row splits over ceil(M/16) row blocks
    int S, kb_per_split;        // K splits (64-byte K-blocks per split)
};

template <int MW, int NB, bool DEEP>
__global__ __launch_bounds__(PANEL_THREADS, 1) void gemm_panel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ B,
    const float* __restrict__ sw, const float* residual, float* y, int32_t* __restrict__ partials,
    PanelParams pp) {
    constexpr int STAGE_BYTES = NB * 16 * ROW_BYTES;
    __shared__ __attribute__((aligned(1024))) int8_t smem[NSTB * STAGE_BYTES];

    const int M = pp.M, N = pp.N, K = pp.K;
    // ---- block -> (panel, K split, row split); consecutive ids share an XCD,
    // so the row splits of one panel read its weights through the same L2
    const int nblocks = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid % NXCD, slot = bid / NXCD;
    const int per = nblocks / NXCD, extra = nblocks % NXCD;
    const int lid = (xcd < extra) ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    const int r = lid % pp.R;
    const int split = (lid / pp.R) % pp.S;
    const int p = lid / (pp.R * pp.S);

    const int cb0 = p * pp.cb_base + min(p, pp.cb_extra);
    const int ncb = pp.cb_base + (p < pp.cb_extra ? 1 : 0);
    const int c0 = 16 * cb0;
    const int KB = K >> 6;
    const int kb0 = min(split * pp.kb_per_split, KB);
    const int nkb = min(kb0 + pp.kb_per_split, KB) - kb0;
    const int nst = (nkb + KBS - 1) / KBS;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // rows: split r gets row blocks [rs0, rs1); wave w a balanced share of them
    const int rs0 = r * pp.rb_total / pp.R, rs1 = (r + 1) * pp.rb_total / pp.R;
    const int nrb = rs1 - rs0;
    const int rbw = rs0 + wave * nrb / 4;
    const int mw = rs0 + (wave + 1) * nrb / 4 - rbw;   // <= MW (host-checked)

    // ---- weight staging: thread t copies chunk (t % 16) of row t/16 + 16q of
    // the stage, for q < NB.  Stored at physical chunk t % 16 of that row,
    // which holds logical chunk (t % 16) ^ (t / 16).  Column blocks past the
    // panel (q >= ncb) re-read block ncb-1 (a cache hit, no extra HBM
    // traffic) into LDS rows nobody stores results from, so every thread
    // issues the same loads in every stage: the compiler's wait counts then
    // need no merge over paths.  DEEP: two staging sets keep two stages (2 x
    // NB x 4 KiB per CU) of weights in flight (the stream is latency-bound:
    // bandwidth = bytes in flight / latency); otherwise one.
    const int t = threadIdx.x;
    const int st_lc = (t & 15) ^ (t >> 4);
    // All global reads are raw buffer loads: a 32-bit per-lane offset fixed
    // for the whole loop, plus a scalar offset for the stage or K-block, so
    // no address arithmetic sits in the loop.  The buffer ranges cover
    // exactly this panel's weight rows and this row split's activation rows;
    // the hardware returns zeros past them (every read here is inside by
    // construction).
    const int b_rows = min(c0 + NB * 16, N) - c0;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B + static_cast<int64_t>(c0) * K), 0, b_rows * K, kBufferFlags);
    uint32_t b_off[NB];   // byte offset of the row (clamped to N-1) and chunk inside the panel
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int col = min(c0 + 16 * min(q, ncb - 1) + (t >> 4), N - 1);
        b_off[q] = static_cast<uint32_t>(col - c0) * static_cast<uint32_t>(K) + st_lc * 16;
    }
    constexpr int NSET = DEEP ? 2 : 1;   // weight staging register sets
    constexpr int NPAIR = DEEP ? 4 : 2;  // activation pair buffers
    i32x4 bs[NSET][NB];
    // Load stage st (clamped to the last stage) into `dst`.  In a short last
    // stage the chunks past its K-blocks re-read chunk lc % 4 (inside the
    // stage's first K-block, so inside the matrix); those bytes are never
    // multiplied.
    auto stage_load = [&](i32x4* dst, int st) __attribute__((always_inline)) {
        st = min(st, nst - 1);
        const int kin = nkb - st * KBS;
        const int lcd = ((st_lc >> 2) < kin ? 0 : (st_lc & 3) - st_lc) * 16;
        const int soff = (kb0 * 64) + st * ROW_BYTES;
#pragma unroll
        for (int q = 0; q < NB; ++q)
            dst[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, static_cast<int>(b_off[q]) + lcd, soff, 0);
    };
    auto stage_store = [&](const i32x4* src, int slot_) __attribute__((always_inline)) {
        int8_t* dst = smem + slot_ * STAGE_BYTES + 16 * t;
#pragma unroll
        for (int q = 0; q < NB; ++q) *reinterpret_cast<i32x4*>(dst + q * 16 * ROW_BYTES) = src[q];
    };

    // ---- fragment addresses.  Weight fragment (column block j, K-block u of
    // a stage): row 16j + l%16, logical chunk 4u + l/16, physical chunk
    // (4u + l/16) ^ (l%16).
    const int f_row = lane & 15;
    const int f_grp = lane >> 4;
    int f_off[KBS];
#pragma unroll
    for (int u = 0; u < KBS; ++u) f_off[u] = f_row * ROW_BYTES + (((4 * u + f_grp) ^ f_row) * 16);
    // Activation fragment (row block i of the wave, K-block kb): row
    // 16*(rbw+i) + l%16 (clamped to M-1), bytes 64*kb + 16*(l/16).
    const int a_row0 = 16 * rs0;
    const int a_rows = max(min(16 * rs1, M) - a_row0, 1);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A + static_cast<int64_t>(min(a_row0, M - 1)) * K), 0, a_rows * K, kBufferFlags);
    int a_off[MW];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
        const int row = min(16 * (rbw + i) + f_row, min(16 * rs1, M) - 1);
        a_off[i] = (row - min(a_row0, M - 1)) * K + 16 * f_grp;
    }
    auto a_frag = [&](int i, int kbc) __attribute__((always_inline)) -> i32x4 {   // kbc: clamped K-block
        return __builtin_amdgcn_raw_buffer_load_b128(ra, a_off[i], (kb0 + kbc) * 64, 0);
    };

    i32x4 acc[MW][NB];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    // Activation fragments of two consecutive K-blocks (a "pair").  Every wave
    // runs all MW x NB products: rows past its own (i >= mw) multiply clamped
    // rows and columns past the panel (j >= ncb) multiply stale LDS rows;
    // neither is ever stored, and in lockstep waves and panels the busiest one
    // sets the time anyway.  K-block indices past the split are clamped to its
    // last K-block (in-bounds reads whose products are never added).
    struct APair {
        i32x4 v[MW][2];
    };
    auto load_a = [&](APair& ap, int kb) __attribute__((always_inline)) {   // K-blocks kb, kb+1 of this split
        const int k0 = min(kb, nkb - 1), k1 = min(kb + 1, nkb - 1);
#pragma unroll
        for (int i = 0; i < MW; ++i) {
            ap.v[i][0] = a_frag(i, k0);
            ap.v[i][1] = a_frag(i, k1);
        }
    };

    // Weight fragments go through a ring of RING registers.  A stage is
    // G = 4*NB groups (group g: K-block g / NB, column block g % NB); group g
    // runs MW MFMAs on ring register g % RING, and right after its first MFMA
    // the wave reads the fragment of group g + RING - 1 (past the stage's end:
    // the next stage's first groups, whose slot is already published).
    constexpr int RING = MW >= 3 ? 4 : 8;
    constexpr int G = KBS * NB;
    static_assert(G % RING == 0, "the ring phase must repeat every stage");
    i32x4 fr[RING];
    auto read_frag = [&](int slot_, int g) __attribute__((always_inline)) {
        fr[g % RING] = *reinterpret_cast<const i32x4*>(smem + slot_ * STAGE_BYTES + f_off[g / NB] +
                                                       (g % NB) * 16 * ROW_BYTES);
    };

    // ---- one stage; the instruction order is written out and pinned with
    // scheduling barriers (the compiler would otherwise sink every prefetch to
    // its first use), and the compiler places the waits.
    //   - Stage st uses ring slot st % 3.  Activation pair p (K-blocks 2p,
    //     2p+1 of the split) lives in buffer p % NPAIR: stage st multiplies
    //     pairs 2st and 2st+1.  During K-block 0 the wave loads pair
    //     2st + NPAIR - 1 and during K-block 2 pair 2st + NPAIR, each into the
    //     buffer the previous pair just released: activations run 2*NPAIR - 2
    //     K-blocks ahead.
    //   - During K-block 2, after that prefetch, staging set st % NSET (stage
    //     st+2, loaded NSET stages ago) goes to the slot stage st-1 used (free
    //     since the barrier at the top of this stage; the next barrier
    //     publishes it before anyone reads it), and stage st + 2 + NSET starts
    //     loading into it.
    //   - The vector-memory counter retires loads in issue order, so a wait
    //     for an activation pair also waits for every weight load issued
    //     before it.  The first pair loaded after a weight load is used
    //     2*NPAIR - 2 K-blocks later, at K-block 2 NSET stages on (NPAIR =
    //     2*NSET), exactly when that weight load is stored: the weights keep
    //     their NSET stages of lead.
    // FULL: all 4 K-blocks present (every stage but a short last one); ODD:
    // the parity of st, which fixes the buffers at compile time.
    APair abuf[NPAIR];
    auto run_stage = [&](int st, auto full_tag, auto odd_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr int ODD = decltype(odd_tag)::value;
        constexpr int SET = NSET == 2 ? ODD : 0;
        if (st > 0) __syncthreads();
        const int slot_ = st % NSTB;
        const int nslot = (st + 1) % NSTB;
        const int kin = FULL ? KBS : nkb - st * KBS;   // K-blocks in this stage (uniform)
        const int kb = st * KBS;
#pragma unroll
        for (int u = 0; u < KBS; ++u) {
            if (!FULL && u >= kin) break;                // (uniform)
            const APair& cur = abuf[(2 * ODD + (u >> 1)) % NPAIR];
            const int h = u & 1;
            // prefetch during K-blocks 0 and 2: pair 2st + u/2 + NPAIR - 1
            APair* al = (u & 1) ? nullptr : &abuf[(2 * ODD + (u >> 1) + NPAIR - 1) % NPAIR];
            const int ak0 = min(kb + u + 2 * NPAIR - 2, nkb - 1), ak1 = min(kb + u + 2 * NPAIR - 1, nkb - 1);
            int issued = 0;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int g = u * NB + j;
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fr[g % RING], cur.v[i][h], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (i == 0) {
                        const int gn = g + RING - 1;
                        read_frag(gn < G ? slot_ : nslot, gn < G ? gn : gn - G);
                        __builtin_amdgcn_sched_barrier(0);
                    } else if (al && issued < 2 * MW) {
                        const int li = issued >> 1, lh = issued & 1;
                        al->v[li][lh] = a_frag(li, lh ? ak1 : ak0);
                        ++issued;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if (al) {
#pragma unroll
                for (int q = 0; q < 2 * MW; ++q)
                    if (q >= issued) al->v[q >> 1][q & 1] = a_frag(q >> 1, (q & 1) ? ak1 : ak0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (FULL && u == 2) {
                stage_store(bs[SET], (st + 2) % NSTB);
                stage_load(bs[SET], st + 2 + NSET);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (!FULL) {   // a short last stage: nothing later reads these
            stage_store(bs[SET], (st + 2) % NSTB);
            stage_load(bs[SET], st + 2 + NSET);
        }
    };

    // ---- prologue: stages 0 and 1 into the ring with one memory latency
    // (without DEEP, stage 1 borrows the fragment ring and a pair buffer as
    // staging space), the next NSET stages in flight, activation pairs
    // 0 .. NPAIR-2 and the first fragments in registers
    if (nst > 0) {   // (uniform) an empty K split multiplies nothing
        if constexpr (DEEP) {
            stage_load(bs[0], 0);
            stage_load(bs[1], 1);
#pragma unroll
            for (int pr = 0; pr + 1 < NPAIR; ++pr) load_a(abuf[pr], 2 * pr);
            stage_store(bs[0], 0);
            stage_store(bs[1], 1);
            stage_load(bs[0], 2);
            stage_load(bs[1], 3);
        } else {
            static_assert(RING + 2 * MW >= NB, "prologue staging space");
            i32x4 tmp[RING + 2 * MW];
            stage_load(bs[0], 0);
            stage_load(tmp, 1);
            load_a(abuf[0], 0);
            stage_store(bs[0], 0);
            stage_store(tmp, 1);
            stage_load(bs[0], 2);
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < RING - 1; ++g) read_frag(0, g);
    }
    using F = std::true_type;
    using T = std::false_type;
    using E = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    const int nfull = nkb / KBS;
    int st = 0;
    if constexpr (DEEP) {   // buffers alternate with the stage parity
        for (; st + 1 < nfull; st += 2) {
            run_stage(st, F{}, E{});
            run_stage(st + 1, F{}, O{});
        }
        if (st < nfull) run_stage(st++, F{}, E{});
        if (st < nst) {
            if (st & 1) run_stage(st, T{}, O{});
            else run_stage(st, T{}, E{});
        }
    } else {
        for (; st < nfull; ++st) run_stage(st, F{}, E{});
        if (st < nst) run_stage(st, T{}, E{});
    }

    // ---- epilogue straight from the accumulators (an empty K split still
    // writes its zero partial)
    const int nlane0 = 4 * f_grp;
    const bool vec_ok = (N & 3) == 0 &&
                        (partials || ((reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                                      (reinterpret_cast<uintptr_t>(residual) & 15) == 0));
    int32_t* part = partials ? partials + static_cast<size_t>(split) * static_cast<size_t>(M) *
                                              static_cast<size_t>(N)
                             : nullptr;
    const bool sw_vec = (reinterpret_cast<uintptr_t>(sw) & 15) == 0;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
        if (i >= mw) continue;
        const int m = 16 * (rbw + i) + f_row;
        if (m >= M) continue;
        const float sxm = part ? 0.0f : sx[m];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j >= ncb) continue;
            const int n = c0 + 16 * j + nlane0;
            if (n >= N) continue;
            const size_t o = static_cast<size_t>(m) * static_cast<size_t>(N) + static_cast<size_t>(n);
            const i32x4 a = acc[i][j];
            if (vec_ok && n + 3 < N) {
                if (part) {
                    *reinterpret_cast<i32x4*>(part + o) = a;
                    continue;
                }
                float s0, s1, s2, s3;
                if (sw_vec) {
                    const float4 s4 = *reinterpret_cast<const float4*>(sw + n);
                    s0 = s4.x, s1 = s4.y, s2 = s4.z, s3 = s4.w;
                } else {
                    s0 = sw[n], s1 = sw[n + 1], s2 = sw[n + 2], s3 = sw[n + 3];
                }
                float4 v;
                if (residual) {
                    const float4 r4 = *reinterpret_cast<const float4*>(residual + o);
                    v.x = scale_acc_residual(a[0], sxm, s0, r4.x);
                    v.y = scale_acc_residual(a[1], sxm, s1, r4.y);
                    v.z = scale_acc_residual(a[2], sxm, s2, r4.z);
                    v.w = scale_acc_residual(a[3], sxm, s3, r4.w);
                } else {
                    v.x = scale_acc(a[0], sxm, s0);
                    v.y = scale_acc(a[1], sxm, s1);
                    v.z = scale_acc(a[2], sxm, s2);
                    v.w = scale_acc(a[3], sxm, s3);
                }
                *reinterpret_cast<float4*>(y + o) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e >= N) continue;
                    if (part) part[o + e] = a[e];
                    else y[o + e] = residual ? scale_acc_residual(a[e], sxm, sw[n + e], residual[o + e])
                                             : scale_acc(a[e], sxm, sw[n + e]);
                }
            }
        }
    }
}

// Template configurations (MW row blocks per wave, NB column blocks per
// panel, DEEP pipeline).  Registers per lane: 4*MW*NB accumulators,
// 16*MW (32*MW with DEEP) activation, 4*NB (8*NB with DEEP) weight staging
// and a ring of 4 or 8 weight fragments, within 512.
struct PanelKind {
    int mw, nb;
    bool deep;
};
constexpr PanelKind kPanelKinds[] = {{1, 8, true}, {2, 8, true}, {2, 12, true}, {3, 8, true}, {4, 9, false}, {6, 9, false}};
constexpr int kNumPanelKinds = sizeof(kPanelKinds) / sizeof(kPanelKinds[0]);

constexpr int NCU = 256;

}  // namespace

// Choose row splits R, column panels P and K splits S <= max_splitk for the
// panel kernel by a simple time model: the busiest wave's MFMA count, its
// LDS traffic, HBM bytes (weights once, partials when S > 1) and L2 traffic
// (every panel reads all activation rows of its K range).  Returns false
// when no configuration fits (M beyond 4 * 16 * 6 rows per split, etc.).
bool plan_panel(int64_t M, int64_t N, int64_t K, int max_splitk, bool residual, PanelPlan* out) {
    if (M <= 0 || N <= 0 || K <= 0) return false;
    const int64_t rb = (M + 15) / 16, cb = (N + 15) / 16, KB = K / 64;
    const double f = 2.0e9;         // sustained clock under MFMA load (Hz)
    const double hbm = 6.0e12;      // sustained HBM bytes/s
    const double l2 = 20.0e12;      // L2 -> CU bytes/s, whole chip
    const double lds = 128.0;       // LDS bytes per clock per CU
    double best = 1e30;
    PanelPlan bp{};
    for (int kind = 0; kind < kNumPanelKinds; ++kind) {
        const int MW = kPanelKinds[kind].mw, NB = kPanelKinds[kind].nb;
        for (int R = 1; R <= 8; ++R) {
            if (R > rb) break;
            const int64_t rbs = (rb + R - 1) / R;
            const int64_t mw = (rbs + 3) / 4;
            if (mw > MW) continue;
            for (int S = 1; S <= max_splitk; ++S) {
                int64_t kps = (KB + S - 1) / S;
                kps = (kps + KBS - 1) / KBS * KBS;
                if (S > 1 && (static_cast<int64_t>(S) - 1) * kps >= KB) continue;   // no empty splits
                const int64_t pmin = (cb + NB - 1) / NB;
                int64_t P = std::max<int64_t>(pmin, NCU / (static_cast<int64_t>(R) * S));
                P = std::min<int64_t>(P, cb);
                const int64_t ncb = (cb + P - 1) / P;
                if (ncb > NB) continue;
                const int64_t wgs = P * R * S;
                if (wgs > static_cast<int64_t>(1) << 30) continue;
                const int64_t rounds = (wgs + NCU - 1) / NCU;
                const int64_t nkb = std::min<int64_t>(kps, KB);
                // every wave runs its configuration's full MW x NB products
                const double mfma_s = static_cast<double>(rounds * MW * NB * nkb) * 16.0 / f;
                const double lds_s = static_cast<double>(rounds * nkb) * (4.0 * NB + ncb) * 1024.0 / lds / f;
                double hbm_bytes = static_cast<double>(N) * K + static_cast<double>(M) * K +
                                   4.0 * M * N * (residual ? 2.0 : 1.0);
                if (S > 1) hbm_bytes += 8.0 * S * M * N;
                const double l2_bytes = static_cast<double>(P) * M * K + static_cast<double>(R) * N * K;
                double t = std::max(std::max(mfma_s, lds_s), std::max(hbm_bytes / hbm, l2_bytes / l2));
                t += 3.0e-6 * (S > 1 ? 1 : 0);   // second launch
                if (t < best * 0.999) {
                    best = t;
                    bp.kind = kind;
                    bp.R = R;
                    bp.P = static_cast<int>(P);
                    bp.S = S;
                    bp.kb_per_split = static_cast<int>(kps);
                    bp.est_us = t * 1e6;
                }
            }
        }
    }
    if (best >= 1e30) return false;
    *out = bp;
    return true;
}

namespace {

template <int MW, int NB, bool DEEP>
hipError_t launch_panel_t(const GemmArgs& a, const PanelPlan& p, int32_t* partials, hipStream_t stream) {
    const int64_t cb = (a.N + 15) / 16;
    PanelParams pp;
    pp.M = static_cast<int>(a.M);
    pp.N = static_cast<int>(a.N);
    pp.K = static_cast<int>(a.K);
    pp.P = p.P;
    pp.cb_base = static_cast<int>(cb / p.P);
    pp.cb_extra = static_cast<int>(cb % p.P);
    pp.R = p.R;
    pp.rb_total = static_cast<int>((a.M + 15) / 16);
    pp.S = p.S;
    pp.kb_per_split = p.kb_per_split;
    const unsigned nblocks = static_cast<unsigned>(static_cast<int64_t>(p.P) * p.R * p.S);
    hipLaunchKernelGGL((gemm_panel<MW, NB, DEEP>), dim3(nblocks), dim3(PANEL_THREADS), 0, stream, a.xq, a.sx,
                       a.w, a.sw, a.residual, a.y, partials, pp);
    return hipGetLastError();
}

}  // namespace

bool panel_kind_shape(int kind, int* mw, int* nb) {
    if (kind < 0 || kind >= kNumPanelKinds) return false;
    *mw = kPanelKinds[kind].mw;
    *nb = kPanelKinds[kind].nb;
    return true;
}

bool panel_plan_valid(int64_t M, int64_t N, int64_t K, const PanelPlan& p) {
    if (p.kind < 0 || p.kind >= kNumPanelKinds || p.R < 1 || p.P < 1 || p.S < 1 || p.kb_per_split < 1)
        return false;
    const int64_t rb = (M + 15) / 16, cb = (N + 15) / 16, KB = K / 64;
    const int MW = kPanelKinds[p.kind].mw, NB = kPanelKinds[p.kind].nb;
    if (p.R > rb || p.P > cb) return false;
    if ((((rb + p.R - 1) / p.R) + 3) / 4 > MW) return false;   // rows per wave
    if ((cb + p.P - 1) / p.P > NB) return false;               // columns per panel
    if (p.kb_per_split % KBS != 0 && p.S > 1) return false;
    if (static_cast<int64_t>(p.kb_per_split) * p.S < KB) return false;   // K covered
    return true;
}

hipError_t launch_panel(const GemmArgs& a, const PanelPlan& p, void* workspace, hipStream_t stream) {
    if (!panel_plan_valid(a.M, a.N, a.K, p)) return hipErrorInvalidValue;
    int32_t* partials = a.acc_out ? a.acc_out : p.S > 1 ? static_cast<int32_t*>(workspace) : nullptr;
    if (a.acc_out && p.S > 1) return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    switch (p.kind) {
        case 0: e = launch_panel_t<1, 8, true>(a, p, partials, stream); break;
        case 1: e = launch_panel_t<2, 8, true>(a, p, partials, stream); break;
        case 2: e = launch_panel_t<2, 12, true>(a, p, partials, stream); break;
        case 3: e = launch_panel_t<3, 8, true>(a, p, partials, stream); break;
        case 4: e = launch_panel_t<4, 9, false>(a, p, partials, stream); break;
        case 5: e = launch_panel_t<6, 9, false>(a, p, partials, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.S <= 1 || a.acc_out) return e;
    return launch_reduce(a, p.S, partials, stream);
}

}  // namespace w8a8
