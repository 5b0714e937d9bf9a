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
//   - a stage is two 64-byte K-blocks of every row the workgroup touches:
//     its activation rows, then its weight rows.  Stages go HBM/L2 -> VGPR
//     -> LDS with loads that read 8 rows x 128 bytes per wave instruction
//     (whole cache lines: an instruction in MFMA fragment layout, 16 rows x
//     64 bytes, sustains about a third of the L2 bandwidth on MI355X), then
//     both operands' fragments are read from LDS.  NSET register sets keep
//     NSET stages in flight; NSLOT LDS slots (3 when they fit) let the next
//     stage's first fragments be read before the barrier;
//   - 16-byte chunks of a row are XOR-swizzled with the row index, so the 16
//     rows one fragment read touches hit distinct banks;
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
// own wait counts order them.  Only staging loads use the vector-memory
// counter in the main loop; it retires them in issue order, which is the
// order they are needed in.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int NXCD = 8;             // XCDs on MI355X
constexpr int PANEL_THREADS = 256;  // 4 waves, one per SIMD
constexpr int KBS = 2;              // 64-byte K-blocks per stage
constexpr int ROW_BYTES = 64 * KBS; // bytes of one row in a stage (8 chunks of 16)
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: raw 32-bit data
constexpr int kNonTemporal = 2;           // cache-policy operand of a buffer load: the nt bit

struct PanelParams {
    int M, N, K;
    int P, cb_base, cb_extra;   // panels; panel p has cb_base + (p < cb_extra) column blocks
    int R, rb_total;            // row splits over ceil(M/16) row blocks
    int S, kb_per_split;        // K splits (64-byte K-blocks per split)
};

// Chunk swizzle of a 128-byte LDS row. A 128-bit LDS read is served 32
// lanes at a time over a 512-byte window (four rows); the swizzle is constant
// on row pairs and steps through 0..7 over rows 0..15, so the 32 lanes of a
// fragment read (16 rows, two neighbouring logical chunks) hit 32 distinct
// 16-byte bank groups, and each 16 of them 16 distinct groups of 256 bytes.
__device__ __forceinline__ int panel_swz(int r) { return ((r >> 2) & 3) * 2 + ((r >> 1) & 1); }

// Smallest divisor of g that is at least `want` (the fragment ring's size:
// its phase must repeat every stage).
constexpr int ring_size(int g, int want) {
    for (int d = want; d <= g; ++d)
        if (g % d == 0) return d;
    return g;
}

// WNT: the weight loads are non-temporal (streamed past the caches).
template <int MW, int NB, int NSET, int NSLOT, bool WNT>
__global__ __launch_bounds__(PANEL_THREADS, 1) void gemm_panel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ B,
    const float* __restrict__ sw, const float* residual, float* y, int32_t* __restrict__ partials,
    PanelParams pp) {
    constexpr int AR = 64 * MW;                      // activation rows of a stage (4 waves)
    constexpr int BR = 16 * NB;                      // weight rows of a stage
    constexpr int RPAD = (AR + BR + 31) / 32 * 32;   // rows incl. padding: whole load instructions
    constexpr int QPT = RPAD / 32;                   // 16-byte pieces per thread per stage
    constexpr int QA = AR / 32;                      // of which activation pieces
    constexpr int STAGE_BYTES = RPAD * ROW_BYTES;
    static_assert(NSLOT == 2 || NSLOT == 3, "LDS slots");
    __shared__ __attribute__((aligned(1024))) int8_t smem[NSLOT * STAGE_BYTES];

    const int M = pp.M, N = pp.N, K = pp.K;
    // ---- block -> (panel, K split, row split); consecutive ids share an XCD,
    // so the row splits of one panel read its weights through the same L2,
    // and a K split's workgroups fill XCDs of their own, whose L2 then holds
    // that split's slice of the activations (short-request down projection
    // at split-K 4: 47.9 -> 44.5 us against all splits on every XCD)
    const int nblocks = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid % NXCD, slot = bid / NXCD;
    const int per = nblocks / NXCD, extra = nblocks % NXCD;
    const int lid = (xcd < extra) ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    const int r = lid % pp.R;
    const int p = (lid / pp.R) % pp.P;
    const int split = lid / (pp.R * pp.P);

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
    // (wave w owns row blocks [rs0 + w*nrb/4, rs0 + (w+1)*nrb/4), at most MW:
    // host-checked)
    const int row_end = min(16 * rs1, M);             // rows of this split: [16 rs0, row_end)
    const int row_first = min(16 * rs0, M - 1);

    // ---- staging.  Thread t's piece q is 16-byte chunk t % 8 (physical) of
    // stage row (t / 8) + 32 q, which holds logical chunk (t % 8) ^ swz(row)
    // (the swizzle depends on t alone).  Pieces q < QA are activation rows:
    // stage row w*16*MW + x is row 16*rbw(w) + x of the matrix; the others
    // are weight rows of the panel.  Every read is a raw buffer
    // load over exactly this panel's weight rows or this split's activation
    // rows: a fixed 32-bit per-lane offset plus a scalar stage offset, no
    // address arithmetic in the loop.
    const int t = threadIdx.x;
    const int st_pc = t & 7;
    const int st_lc = st_pc ^ panel_swz(t >> 3);
    const int b_rows = min(c0 + BR, N) - c0;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(B + static_cast<int64_t>(c0) * K), 0, b_rows * K, kBufferFlags);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A + static_cast<int64_t>(row_first) * K), 0, (row_end - row_first) * K, kBufferFlags);
    // Rows no result is stored from (a wave's row blocks past its mw, column
    // blocks past the panel, padding) get an offset past the buffer's range:
    // the hardware returns zeros without touching memory, so they cost no
    // bandwidth and the matrix cores multiply zeros (less power).
    constexpr int kOutOfRange = 0x40000000;   // beyond every buffer range here (< 2^31 with offsets)
    int q_off[QPT];
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
        const int sr = (t >> 3) + 32 * q;   // stage row
        if (q < QA) {
            const int w = sr / (16 * MW), x = sr % (16 * MW);
            const int rbw_w = rs0 + w * nrb / 4;
            const int mw_w = rs0 + (w + 1) * nrb / 4 - rbw_w;
            const int row = min(16 * rbw_w + x, row_end - 1);
            const bool own = x < 16 * mw_w && 16 * rbw_w + x < row_end;
            q_off[q] = own ? (row - row_first) * K + st_lc * 16 : kOutOfRange;
        } else {
            const int br = sr - AR;
            const int col = min(c0 + br, N - 1);
            q_off[q] = (br < 16 * ncb && c0 + br < N) ? (col - c0) * K + st_lc * 16 : kOutOfRange;
        }
    }
    // Piece q of stage st (clamped to the last stage).  In a short last stage
    // the chunks of its missing K-block re-read the stage's first K-block
    // (inside the matrix); those bytes are never multiplied.
    auto piece_load = [&](i32x4& dst, int st, int q) __attribute__((always_inline)) {
        st = min(st, nst - 1);
        const int lcd = ((st_lc >> 2) < nkb - st * KBS) ? 0 : -64;
        if (q < QA)
            dst = __builtin_amdgcn_raw_buffer_load_b128(ra, q_off[q] + lcd, (kb0 + st * KBS) * 64, 0);
        else
            dst = __builtin_amdgcn_raw_buffer_load_b128(rb, q_off[q] + lcd, (kb0 + st * KBS) * 64, WNT ? kNonTemporal : 0);
    };
    auto piece_store = [&](const i32x4& src, int slot_, int q) __attribute__((always_inline)) {
        *reinterpret_cast<i32x4*>(smem + slot_ * STAGE_BYTES + 16 * t + q * 32 * ROW_BYTES) = src;
    };
    auto stage_load = [&](i32x4* dst, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QPT; ++q) piece_load(dst[q], st, q);
    };
    auto stage_store = [&](const i32x4* src, int slot_) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QPT; ++q) piece_store(src[q], slot_, q);
    };

    // ---- fragment addresses: row x of a 16-row block, K-block u of the stage:
    // logical chunk 4u + l/16, physical chunk (4u + l/16) ^ swz(l % 16).
    const int f_row = lane & 15;
    int f_off[KBS];
#pragma unroll
    for (int u = 0; u < KBS; ++u) f_off[u] = f_row * ROW_BYTES + (((4 * u + (lane >> 4)) ^ panel_swz(f_row)) * 16);
    const int a_base = wave * 16 * MW * ROW_BYTES;   // this wave's activation rows in a stage

    i32x4 acc[MW][NB];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    // Every wave runs all MW x NB products: rows past its own (i >= mw) and
    // columns past the panel (j >= ncb) are zeros in LDS and are never
    // stored; in lockstep waves and panels the busiest one sets the time
    // anyway.
    //
    // Fragments: the activation fragments of a K-block (af[u]) are read
    // during the previous K-block; weight fragments go through a ring of RING
    // registers: a stage is G = KBS*NB groups (group g: K-block g / NB, column
    // block g % NB), group g runs MW MFMAs on ring register g % RING, and
    // right after its first MFMA the wave reads the fragment of group
    // g + RING - 1.
    constexpr int G = KBS * NB;
    constexpr int RING = ring_size(G, MW >= 3 ? 4 : 8);
    static_assert(G % RING == 0, "the ring phase must repeat every stage");
    i32x4 fr[RING];
    i32x4 af[KBS][MW];
    auto read_b = [&](int slot_, int g) __attribute__((always_inline)) {
        fr[g % RING] = *reinterpret_cast<const i32x4*>(smem + slot_ * STAGE_BYTES + f_off[g / NB] +
                                                       (AR + 16 * (g % NB)) * ROW_BYTES);
    };
    auto read_a = [&](int slot_, int u, int i) __attribute__((always_inline)) {
        af[u][i] = *reinterpret_cast<const i32x4*>(smem + slot_ * STAGE_BYTES + a_base + f_off[u] +
                                                   16 * i * ROW_BYTES);
    };

    i32x4 bs[NSET][QPT];
    constexpr bool PRE = NSLOT == 3;   // next stage readable before the barrier

    // ---- one stage; the instruction order is written out and pinned with
    // scheduling barriers (the compiler would otherwise sink every read to
    // its first use), and the compiler places the waits.
    //   - Stage st uses LDS slot st % NSLOT.  With 3 slots stage X is written
    //     during stage X-2 (into the slot stage X-3 used, free since the
    //     barrier at the top of stage X-2) and published by the barrier at the
    //     top of stage X-1, so the last K-block of a stage reads the first
    //     fragments of the next.  With 2 slots it is written during stage X-1
    //     and published at the top of stage X.
    //   - Staging set SET holds the stage to write (loaded NSET stages ago);
    //     piece by piece it goes to LDS and the piece of the stage NSET
    //     further on is loaded into its register.  Staging loads are the only
    //     vector-memory reads in the loop, and they are needed in issue order.
    //   - With one wave per SIMD, a memory instruction that has to wait for
    //     its queue stalls the matrix pipe, so after every MFMA the wave
    //     issues at most one weight-fragment read (right after the first MFMA
    //     of a column block) and one other memory instruction: the next
    //     K-block's activation fragments first, then this K-block's half of
    //     the staging stores and loads.
    // FULL: both K-blocks present (every stage but a short last one).
    auto run_stage = [&](int st, auto full_tag, auto set_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr int SET = decltype(set_tag)::value;
        if (st > 0) {
            __syncthreads();
            if constexpr (!PRE) {
                const int sl = st % NSLOT;
#pragma unroll
                for (int i = 0; i < MW; ++i) read_a(sl, 0, i);
#pragma unroll
                for (int g = 0; g < RING - 1; ++g) read_b(sl, g);
            }
        }
        const int slot_ = st % NSLOT;
        const int nslot = (st + 1) % NSLOT;
        const int kin = FULL ? KBS : nkb - st * KBS;
        const int wslot = (st + NSLOT - 1) % NSLOT;   // slot of the stage being written
        const int lst = st + NSLOT - 1 + NSET;        // stage being loaded
        constexpr int QH = (QPT + 1) / 2;             // staging pieces handled in K-block 0
#pragma unroll
        for (int u = 0; u < KBS; ++u) {
            if (!FULL && u >= kin) break;                // (uniform)
            // next K-block's activation fragments: the other K-block of this
            // stage, or (with PRE) K-block 0 of the next stage
            const bool a_next = u + 1 < KBS || PRE;
            const int a_slot = u + 1 < KBS ? slot_ : nslot;
            const int a_u = (u + 1) % KBS;
            const int na = a_next ? MW : 0;
            const int q0 = u == 0 ? 0 : QH, q1 = u == 0 ? QH : QPT;
            const int nsec = na + (FULL ? 2 * (q1 - q0) : 0);   // secondary memory instructions
            int sec = 0;
            auto secondary = [&]() __attribute__((always_inline)) {
                if (sec < na) {
                    read_a(a_slot, a_u, sec);
                } else {
                    const int k = sec - na, q = q0 + (k >> 1);
                    if ((k & 1) == 0) piece_store(bs[SET][q], wslot, q);
                    else piece_load(bs[SET][q], lst, q);
                }
                ++sec;
                __builtin_amdgcn_sched_barrier(0);
            };
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int g = u * NB + j;
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fr[g % RING], af[u][i], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (i == 0) {
                        const int gn = g + RING - 1;
                        if (gn < G || PRE) {
                            read_b(gn < G ? slot_ : nslot, gn < G ? gn : gn - G);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    if ((i != 0 || MW == 1) && sec < nsec) secondary();
                }
            }
#pragma unroll
            for (int k = 0; k < na + 2 * QPT; ++k)
                if (sec < nsec) secondary();
        }
    };

    // ---- prologue: the first NSLOT-1 stages into LDS (one memory latency),
    // the next NSET in flight, the first fragments in registers
    if (nst > 0) {   // (uniform) an empty K split multiplies nothing
        static_assert(NSET >= NSLOT - 1, "prologue staging space");
#pragma unroll
        for (int x = 0; x < NSLOT - 1; ++x) stage_load(bs[x], x);
#pragma unroll
        for (int x = 0; x < NSLOT - 1; ++x) stage_store(bs[x], x);
#pragma unroll
        for (int x = 0; x < NSET; ++x) stage_load(bs[x], NSLOT - 1 + x);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MW; ++i) read_a(0, 0, i);
#pragma unroll
        for (int g = 0; g < RING - 1; ++g) read_b(0, g);
    }
    using F = std::true_type;
    using T = std::false_type;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1 % NSET>;
    using S2 = std::integral_constant<int, 2 % NSET>;
    const int nfull = nkb / KBS;
    int st = 0;
    // staging sets rotate with the stage (set st % NSET): unrolled NSET-fold
    for (; st + NSET <= nfull; st += NSET) {
        run_stage(st, F{}, S0{});
        if constexpr (NSET > 1) run_stage(st + 1, F{}, S1{});
        if constexpr (NSET > 2) run_stage(st + 2, F{}, S2{});
    }
    // fewer than NSET full stages left (straight-line: a loop here would make
    // the compiler copy every register at its back edge), then a short one
    if (st < nfull) run_stage(st++, F{}, S0{});
    if constexpr (NSET > 2)
        if (st < nfull) run_stage(st++, F{}, S1{});
    if (st < nst) {
        const int set = st % NSET;
        if (set == 0) run_stage(st, T{}, S0{});
        if constexpr (NSET > 1) if (set == 1) run_stage(st, T{}, S1{});
        if constexpr (NSET > 2) if (set == 2) run_stage(st, T{}, S2{});
    }

    // ---- epilogue, in MW passes through LDS (the operand ring is free now).
    // Pass i: every wave parks row block i of its accumulators as int32
    // (16 rows x 16*NB columns, rows padded by 4 words); then all threads
    // sweep the 64 parked rows in 16-byte chunks along the rows: whole-line
    // output stores, the fixed epilogue in between.  An empty K split still
    // writes its zero partial.
    //
    // Loads and stores retire through one in-order counter, so a load issued
    // after a store cannot be waited for without waiting for that store too.
    // The sweep therefore issues no scale load after its first store: the
    // row and column scales of the workgroup are copied into LDS before the
    // passes, and the residual is loaded into registers ahead of the stores.
    constexpr int LDR = 16 * NB + 4;   // parked row pitch (int32)
    constexpr int CH = 4 * NB;         // 16-byte chunks per parked row
    constexpr int PER = 64 * CH / PANEL_THREADS;   // sweep chunks per thread and pass
    constexpr int SX_N = 64 * MW;      // rows of a split a workgroup can hold
    constexpr int SW_N = 16 * NB;
    static_assert(64 * LDR * 4 + (SX_N + SW_N) * 4 <= NSLOT * STAGE_BYTES, "epilogue staging fits the ring");
    static_assert((64 * CH) % PANEL_THREADS == 0, "whole sweep iterations");
    int32_t* park = reinterpret_cast<int32_t*>(smem);
    float* s_sw = reinterpret_cast<float*>(smem + 64 * LDR * 4);
    float* s_sx = s_sw + SW_N;
    const bool vec_ok = (N & 3) == 0 &&
                        (partials || ((reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                                      (reinterpret_cast<uintptr_t>(residual) & 15) == 0));
    int32_t* part = partials ? partials + static_cast<size_t>(split) * static_cast<size_t>(M) *
                                              static_cast<size_t>(N)
                             : nullptr;
    const int row_base = 16 * rs0;
    // chunk `it` of this thread in pass i: parked row rr, chunk cc, output (m, n)
    struct Chunk {
        int rr, cc, m, n;
        bool live;
    };
    auto chunk_at = [&](int i, int it) __attribute__((always_inline)) {
        Chunk c;
        const int q = t + it * PANEL_THREADS;
        c.rr = q / CH;
        c.cc = q % CH;
        const int w = c.rr >> 4, x = c.rr & 15;
        const int rbw_w = rs0 + w * nrb / 4;
        const int mw_w = rs0 + (w + 1) * nrb / 4 - rbw_w;
        c.m = 16 * (rbw_w + i) + x;
        c.n = c0 + 4 * c.cc;
        c.live = i < mw_w && c.m < M && 4 * c.cc < 16 * ncb && c.n < N;
        return c;
    };
    // Narrow kinds (the ones long-K residual layers run on) hold every
    // pass's residual in registers, loaded before the first store; wider
    // kinds load each pass's residual one pass ahead.
    constexpr bool RES_ALL = MW * NB <= 16;
    constexpr int RB = RES_ALL ? MW : 2;
    float4 rbuf[RB][PER];
    auto load_residual = [&](int i, float4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const Chunk c = chunk_at(i, it);
            if (c.live && vec_ok && c.n + 3 < N)
                dst[it] = *reinterpret_cast<const float4*>(
                    residual + static_cast<size_t>(c.m) * static_cast<size_t>(N) + static_cast<size_t>(c.n));
        }
    };
    __syncthreads();   // every wave is done with the operand ring
    if (!part) {
        for (int j = t; j < SW_N; j += PANEL_THREADS)
            if (j < 16 * ncb && c0 + j < N) s_sw[j] = sw[c0 + j];
        for (int j = t; j < SX_N; j += PANEL_THREADS)
            if (row_base + j < row_end) s_sx[j] = sx[row_base + j];
        if (residual) {
            if constexpr (RES_ALL) {
#pragma unroll
                for (int i = 0; i < MW; ++i) load_residual(i, rbuf[i]);
            } else {
                load_residual(0, rbuf[0]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MW; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
            *reinterpret_cast<i32x4*>(park + (wave * 16 + f_row) * LDR + 16 * j + 4 * (lane >> 4)) = acc[i][j];
        __syncthreads();
        if constexpr (!RES_ALL)
            if (!part && residual && i + 1 < MW) load_residual(i + 1, rbuf[(i + 1) & 1]);
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const Chunk c = chunk_at(i, it);
            if (!c.live) continue;
            const int m = c.m, n = c.n;
            const i32x4 a = *reinterpret_cast<const i32x4*>(park + c.rr * LDR + 4 * c.cc);
            const size_t o = static_cast<size_t>(m) * static_cast<size_t>(N) + static_cast<size_t>(n);
            if (vec_ok && n + 3 < N) {
                if (part) {
                    *reinterpret_cast<i32x4*>(part + o) = a;
                    continue;
                }
                const float sxm = s_sx[m - row_base];
                const float4 s4 = *reinterpret_cast<const float4*>(s_sw + 4 * c.cc);
                float4 v;
                if (residual) {
                    const float4 r4 = rbuf[RES_ALL ? i : (i & 1)][it];
                    v.x = scale_acc_residual(a[0], sxm, s4.x, r4.x);
                    v.y = scale_acc_residual(a[1], sxm, s4.y, r4.y);
                    v.z = scale_acc_residual(a[2], sxm, s4.z, r4.z);
                    v.w = scale_acc_residual(a[3], sxm, s4.w, r4.w);
                } else {
                    v.x = scale_acc(a[0], sxm, s4.x);
                    v.y = scale_acc(a[1], sxm, s4.y);
                    v.z = scale_acc(a[2], sxm, s4.z);
                    v.w = scale_acc(a[3], sxm, s4.w);
                }
                // non-temporal: every workgroup writes its outputs in the same
                // burst at the end, and streamed stores drain that burst 5-9%
                // faster (short-request gate+up 68 -> 62 us)
                store_out4(y + o, v, true);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e >= N) continue;
                    if (part) part[o + e] = a[e];
                    else y[o + e] = residual ? scale_acc_residual(a[e], s_sx[m - row_base], s_sw[4 * c.cc + e], residual[o + e])
                                             : scale_acc(a[e], s_sx[m - row_base], s_sw[4 * c.cc + e]);
                }
            }
        }
        __syncthreads();
    }
}

// Template configurations: MW row blocks per wave, NB column blocks per
// panel, NSET staging register sets, NSLOT LDS slots of (64*MW + 16*NB)
// rows x 128 bytes (within 160 KiB).  Registers per lane: 4*MW*NB
// accumulators, 4*NSET*(2*MW + NB/2) staging, 8*MW activation and 4 or 8
// weight fragments, within 512.
struct PanelKind {
    int mw, nb, nset, nslot;
};
// Wide panels for wide layers (N in the tens of thousands); narrow ones for
// N = 5120-like layers, where a wide kind would multiply columns past the
// panel and every wave would read all of their weight fragments.  The
// 6 x 9 kind (328-row batches) keeps one staging set: with two it needed
// more than 512 registers and spilled 276 bytes per lane inside the main
// loop; with one it spills nothing and measured 1% faster.
constexpr PanelKind kPanelKinds[] = {{1, 8, 3, 3}, {2, 8, 3, 3}, {2, 12, 3, 3}, {3, 8, 3, 3}, {4, 9, 3, 3},
                                     {6, 9, 1, 2}, {1, 4, 3, 3}, {2, 3, 3, 3}, {2, 4, 3, 3}, {2, 5, 3, 3},
                                     {4, 5, 3, 3}};
constexpr int kNumPanelKinds = sizeof(kPanelKinds) / sizeof(kPanelKinds[0]);

constexpr int NCU = 256;

}  // namespace

// Choose row splits R, column panels P and K splits S <= max_splitk for the
// panel kernel with a time model calibrated on MI355X: per round of
// workgroups, a fixed cost (prologue, the output write, launch) plus, per
// K-block, the larger of the MFMA issue time (MW*NB products of 16 cycles,
// times the measured 1.7 for interleaved memory instructions) and the LDS
// time (fragment reads of 4 waves and the staging writes at 110 B/clk);
// never below the HBM time of the weights, activations, output and
// partials; plus the split-K reduction when S > 1.  Returns false when no
// configuration holds the rows.
bool plan_panel(int64_t M, int64_t N, int64_t K, int max_splitk, bool residual, PanelPlan* out) {
    if (M <= 0 || N <= 0 || K <= 0) return false;
    const int64_t rb = (M + 15) / 16, cb = (N + 15) / 16, KB = K / 64;
    const double f = 1.8e9;          // clock under this kernel's MFMA load (Hz)
    const double hbm = 5.5e12;       // HBM bytes/s this kernel sustains
    const double fixed_s = 20e-6;    // per round: prologue, output write, launch
    const double lds_bpc = 110.0;    // LDS bytes per clock per CU it sustains
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
                const double mfma_cyc = 16.0 * MW * NB * 1.7;
                const double lds_cyc = (4.0 * (NB + MW) * 1024.0 + (64.0 * MW + 16.0 * NB) * 64.0) / lds_bpc;
                double t = static_cast<double>(rounds) *
                           (fixed_s + static_cast<double>(nkb) * std::max(mfma_cyc, lds_cyc) / f);
                double hbm_bytes = static_cast<double>(N) * K + static_cast<double>(M) * K +
                                   4.0 * M * N * (residual ? 2.0 : 1.0);
                if (S > 1) hbm_bytes += 4.0 * S * M * N;
                t = std::max(t, hbm_bytes / hbm + 8e-6);
                // reduction kernel: a second launch (about 5 us) and its stream.
                // Calibrated against every feasible plan of 40 mid-M shapes
                // timed on MI355X: with 3 us the planner split a 128 x 5120 x
                // 5120 product four ways (20 us) where one way takes 12.5 us
                if (S > 1) t += 5e-6 + (4.0 * S + 8.0) * M * N / 4.0e12;
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

template <int MW, int NB, int NSET, int NSLOT, bool WNT = false>
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
    hipLaunchKernelGGL((gemm_panel<MW, NB, NSET, NSLOT, WNT>), dim3(nblocks), dim3(PANEL_THREADS), 0, stream, a.xq, a.sx,
                       a.w, a.sw, a.residual, a.y, partials, pp);
    return hipGetLastError();
}

}  // namespace

bool panel_kind_shape(int kind, int* mw, int* nb, int* nset, int* nslot) {
    if (kind < 0 || kind >= kNumPanelKinds) return false;
    *mw = kPanelKinds[kind].mw;
    *nb = kPanelKinds[kind].nb;
    *nset = kPanelKinds[kind].nset;
    *nslot = kPanelKinds[kind].nslot;
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

bool make_panel_plan(int64_t M, int64_t N, int64_t K, int kind, int R, int P, int S, PanelPlan* out) {
    if (S < 1 || K < 64) return false;
    const int64_t KB = K / 64;
    int64_t kps = (KB + S - 1) / S;
    if (S > 1) kps = (kps + KBS - 1) / KBS * KBS;
    PanelPlan p{};
    p.kind = kind;
    p.R = R;
    p.P = P;
    p.S = S;
    p.kb_per_split = static_cast<int>(kps);
    p.est_us = 0.0;
    if (!panel_plan_valid(M, N, K, p)) return false;
    *out = p;
    return true;
}

hipError_t launch_panel(const GemmArgs& a, const PanelPlan& p, void* workspace, hipStream_t stream) {
    if (!panel_plan_valid(a.M, a.N, a.K, p)) return hipErrorInvalidValue;
    int32_t* partials = a.acc_out ? a.acc_out : p.S > 1 ? static_cast<int32_t*>(workspace) : nullptr;
    if (a.acc_out && p.S > 1) return hipErrorInvalidValue;
    // The wide kinds stream their weights past the caches when every weight
    // byte is read by one workgroup (no row or K splits) of a wide layer:
    // measured 3-5% faster at N = 34816, and slower where row splits read a
    // panel twice or N is narrow.
    const bool wnt = p.R == 1 && p.S == 1 && a.N >= 16384;
    hipError_t e = hipErrorInvalidValue;
    switch (p.kind) {
        case 0: e = launch_panel_t<1, 8, 3, 3>(a, p, partials, stream); break;
        case 1: e = launch_panel_t<2, 8, 3, 3>(a, p, partials, stream); break;
        case 2: e = wnt ? launch_panel_t<2, 12, 3, 3, true>(a, p, partials, stream)
                        : launch_panel_t<2, 12, 3, 3>(a, p, partials, stream); break;
        case 3: e = launch_panel_t<3, 8, 3, 3>(a, p, partials, stream); break;
        case 4: e = wnt ? launch_panel_t<4, 9, 3, 3, true>(a, p, partials, stream)
                        : launch_panel_t<4, 9, 3, 3>(a, p, partials, stream); break;
        case 5: e = wnt ? launch_panel_t<6, 9, 1, 2, true>(a, p, partials, stream)
                        : launch_panel_t<6, 9, 1, 2>(a, p, partials, stream); break;
        case 6: e = launch_panel_t<1, 4, 3, 3>(a, p, partials, stream); break;
        case 7: e = launch_panel_t<2, 3, 3, 3>(a, p, partials, stream); break;
        case 8: e = launch_panel_t<2, 4, 3, 3>(a, p, partials, stream); break;
        case 9: e = launch_panel_t<2, 5, 3, 3>(a, p, partials, stream); break;
        case 10: e = launch_panel_t<4, 5, 3, 3>(a, p, partials, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.S <= 1 || a.acc_out) return e;
    return launch_reduce(a, p.S, partials, stream);
}

}  // namespace w8a8
