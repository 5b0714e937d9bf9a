// C ABI of the W8A8 library: argument checks, then dispatch to the gfx950
// kernels.  Every check that the host can make runs before any launch, and
// a rejected call changes no output.  Per-entry semantics are documented in
// include/w8a8.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "w8a8.h"
#include "w8a8_diag.h"

namespace {

using w8a8::GemmArgs;
using w8a8::GemmPlan;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_k(int64_t K) {
    if (K <= 0 || (K % 64) != 0) return W8A8_ERR_SHAPE;
    if (K > W8A8_MAX_K) return W8A8_ERR_K_BOUND;
    return W8A8_OK;
}

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;  // grid and index limits of the kernels
// Entry points that launch a workgroup (of up to 1024 threads) per row take
// at most W8A8_MAX_ROWS rows, so that a launch stays below 2^32 work-items
// (the dispatch packet's grid size is 32 bits).
static_assert(int64_t{W8A8_MAX_ROWS} * 1024 < (int64_t{1} << 32), "per-row launches must fit 2^32 work-items");

int hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP; }

// Byte ranges [p, p+n) and [q, q+m) overlap.
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

int check_quantize_args(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                        const float* smooth, int64_t M, int64_t K, const int8_t* xq, const float* sx) {
    if (M < 0 || x_rows < 0) return W8A8_ERR_INVALID_ARG;
    if (const int kc = check_k(K)) return kc;
    if (M > W8A8_MAX_ROWS) return W8A8_ERR_SHAPE;
    if (ldx < K || (ldx % 4) != 0) return W8A8_ERR_INVALID_ARG;
    if (!row_idx && M > x_rows) return W8A8_ERR_SHAPE;
    if (M == 0) return W8A8_OK;
    if (!x || !smooth || !xq || !sx) return W8A8_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(smooth, 16) || !aligned(xq, 16) || !aligned(sx, 4))
        return W8A8_ERR_ALIGN;
    if (row_idx && !aligned(row_idx, 4)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

int check_readout_args(const int8_t* xq, const float* sx, int64_t M, int64_t K, const int8_t* w_vocab,
                       const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C,
                       const float* logits, const int32_t* err_flag);
int run_readout(const int8_t* xq, const float* sx, int64_t M, int64_t K, const int8_t* w_vocab,
                const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C, float* logits,
                int32_t* err_flag, hipStream_t s);
int check_softmax_args(const float* logits, int64_t M, int64_t C, const double* probs);

int check_gemm_args(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                    const float* residual, float* y, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0) return W8A8_ERR_INVALID_ARG;
    if (const int kc = check_k(K)) return kc;
    if (M > kMaxDim || N > kMaxDim) return W8A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!xq || !sx || !w || !sw || !y) return W8A8_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(w, 16) || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 4))
        return W8A8_ERR_ALIGN;
    if (residual) {
        if (!aligned(residual, 4)) return W8A8_ERR_ALIGN;
        const size_t bytes = static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float);
        if (residual != y && overlaps(residual, bytes, y, bytes)) return W8A8_ERR_INVALID_ARG;
    }
    return W8A8_OK;
}

// Kernel choice for a full product.  The column-panel kernel takes M up to
// kPanelOnlyM, up to kPanelCloseM unless the tiled kernel's time model is
// clearly faster, and up to kPanelMaxM where its own model is faster (see
// pick_panel), except full products with M <= SKINNY_MAX_M whose weights the
// skinny kernel streams through LDS (the full-vocabulary read-out), where
// the skinny kernel is faster; larger M takes the tiled kernel.  Measured:
// for M = 16..64 the panel kernel runs 1.5-3.2x faster than the skinny one
// (e.g. 64 x 34816 x 5120 in 43 against 139 us), while the 3 x 248000 x 5120
// read-out takes 189 us on the skinny kernel and 242 us on the panel one.
// The override can force a tiled configuration (0..TILE_KINDS-1), the panel
// kernel (PANEL_OVERRIDE, any M it fits) or the skinny kernel
// (SKINNY_OVERRIDE, every M <= SKINNY_MAX_M).
constexpr int64_t kPanelMaxM = 1536;
constexpr int64_t kPanelCloseM = 1024;   // past here the panel kernel needs the better estimate outright
constexpr int64_t kPanelOnlyM = 384;   // up to here no comparison: the panel kernel won on every measured shape
static_assert(W8A8_TILE_OVERRIDE_PANEL == w8a8::PANEL_OVERRIDE, "header and library disagree on the panel override");
static_assert(W8A8_TILE_OVERRIDE_SKINNY == w8a8::SKINNY_OVERRIDE, "header and library disagree on the skinny override");

bool pick_panel(int64_t M, int64_t N, int64_t K, int max_splitk, bool residual, w8a8::PanelPlan* pp) {
    const int ov = w8a8::tile_override_value();
    if (ov >= 0 && ov != w8a8::PANEL_OVERRIDE) return false;
    if (ov < 0 && M > kPanelMaxM) return false;
    if (!w8a8::plan_panel(M, N, K, max_splitk, residual, pp)) return false;
    // Past 384 rows the two kernels trade places by shape: the panels of a
    // wide layer no longer fit one round of workgroups (448 x 34816 x 5120:
    // two rounds, 106 us) while the tiled kernel still needs one (88 us);
    // narrow layers with long K stay far faster on panels (1024 x 5120 x
    // 17408: 110 against 193 us).  There the tiled kernel runs when its time
    // model is clearly below the panel's on a product that is not
    // launch-bound.  Calibrated on 30 shapes of 384-1024 rows (N from 4096
    // to 34816, K from 256 to 17408, split-K 1 and 8): the rule picks the
    // faster kernel on every one.
    if (ov < 0 && M > kPanelOnlyM) {
        const double tiled_us = w8a8::tiled_time_estimate_us(M, N, K, max_splitk);
        if (M <= kPanelCloseM && pp->est_us > 40.0 && tiled_us < 0.75 * pp->est_us) return false;
        // 1025-1536 rows: the panel kernel only where its estimate is the
        // lower one (long-K narrow layers: 1536 x 5120 x 17408 + residual,
        // 154 against 188 us); the same rule past 1536 rows would keep the
        // 2048-row down projection on panels, 7% slower than tiles
        if (M > kPanelCloseM && tiled_us <= pp->est_us) return false;
    }
    return true;
}

// The skinny kernel for a full product at split-K 1 (see above); otherwise
// *pp holds the panel plan when the panel kernel runs.
bool pick_skinny(int64_t M, int64_t N, int64_t K, bool residual, w8a8::PanelPlan* pp, bool* panel) {
    *panel = false;
    if (M > w8a8::SKINNY_MAX_M) return false;
    const int ov = w8a8::tile_override_value();
    if (ov == w8a8::SKINNY_OVERRIDE) return true;
    if (ov < 0 && w8a8::skinny_streams_lds(M, N, K)) return true;
    // Narrow layers of a few rows with a long K: the skinny kernel splits K
    // over the waves of each column tile, where the panel kernel's few panels
    // each run the whole K (1 x 1024 x 17408: 12 against 32 us; 8 x 5120 x
    // 17408: 30 against 34 us; 4 x 4096 x 5120: 13.0 against 14.7 us).
    // Measured over M = 1..16, N = 1024..15360 and K = 2048..17408: below
    // K = 4096 both are launch-bound, and past N = 8192 or M * N = 65536 the
    // panel kernel is as fast or faster.
    if (ov < 0 && K >= 4096 && N <= 8192 && M * N <= 65536) return true;
    *panel = pick_panel(M, N, K, 1, residual, pp);
    return !*panel;
}

int run_gemm(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
             const float* residual, float* y, int64_t M, int64_t N, int64_t K, int splitk,
             void* workspace, hipStream_t stream) {
    const GemmArgs a{xq, sx, w, sw, residual, y, M, N, K, nullptr};
    w8a8::PanelPlan pp;
    if (splitk == 1) {
        bool panel = false;
        if (pick_skinny(M, N, K, residual != nullptr, &pp, &panel)) {
            w8a8::SkinnyArgs s{xq, sx, w, sw, residual, y, M, N, K, N, nullptr, N, 0, nullptr};
            return hip_status(w8a8::launch_skinny(s, stream));
        }
        if (panel) return hip_status(w8a8::launch_panel(a, pp, workspace, stream));
    }
    if (pick_panel(M, N, K, splitk, residual != nullptr, &pp))
        return hip_status(w8a8::launch_panel(a, pp, workspace, stream));
    const GemmPlan plan = w8a8::plan_gemm(M, N, K, splitk);
    return hip_status(w8a8::launch_gemm_tiled(a, plan, workspace, stream));
}

// ---- split-K scratch of the allocation-free entry point.  One array per
// GPU the library runs on, held until the process ends.  In host code the
// array's name is only a stand-in for it: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.
static_assert(W8A8_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) static int8_t scratch[W8A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W8A8_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W8A8_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return W8A8_OK;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
    switch (status) {
        case W8A8_OK: return "ok";
        case W8A8_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad stride)";
        case W8A8_ERR_SHAPE: return "unsupported shape (K must be a positive multiple of 64; size limit)";
        case W8A8_ERR_ALIGN: return "misaligned pointer or stride";
        case W8A8_ERR_WORKSPACE: return "split-K workspace missing, misaligned or too small";
        case W8A8_ERR_K_BOUND: return "K above the int32 exactness bound";
        case W8A8_ERR_TOO_MANY_CANDIDATES: return "too many candidates; use the full-vocabulary GEMM";
        case W8A8_ERR_HIP: return "HIP runtime or launch error";
        default: return "unknown status";
    }
}

int w8a8_abi_version(void) { return 10000; }

int w8a8_set_tile_override(int kind) {
    if (kind < -1 || kind > w8a8::SKINNY_OVERRIDE) return W8A8_ERR_INVALID_ARG;
    w8a8::set_tile_override(kind);
    return W8A8_OK;
}

int w8a8_probe_stream_read(const void* buf, int64_t bytes, int32_t* sink, void* stream) {
    if (!buf || !aligned(buf, 16) || bytes <= 0 || (bytes & 15) || !sink || !aligned(sink, 4))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

int w8a8_probe_stream_narrow(const void* src, int64_t n, void* dst, void* stream) {
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || n <= 0 || (n & 3) ||
        overlaps(src, static_cast<size_t>(n) * 4, dst, static_cast<size_t>(n)))
        return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_stream_narrow(src, n, dst, static_cast<hipStream_t>(stream)));
}

int w8a8_probe_mfma_ceiling(int operand_kind, int64_t blocks, int64_t iters, int32_t* sink,
                            int64_t* ops, void* stream) {
    if (operand_kind < 0 || operand_kind > 3 || blocks <= 0 || blocks > kMaxDim || iters <= 0 ||
        !sink || !aligned(sink, 4))
        return W8A8_ERR_INVALID_ARG;
    if (ops) *ops = w8a8::mfma_ceiling_ops(blocks, iters);
    return hip_status(w8a8::launch_mfma_ceiling(operand_kind, blocks, iters, sink,
                                                static_cast<hipStream_t>(stream)));
}

int w8a8_quantize_act(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                      const float* smooth, int64_t M, int64_t K, int8_t* xq, float* sx,
                      void* stream) {
    if (const int rc = check_quantize_args(x, ldx, x_rows, row_idx, smooth, M, K, xq, sx)) return rc;
    if (M == 0) return W8A8_OK;
    const w8a8::QuantArgs a{x, ldx, x_rows, row_idx, smooth, M, K, xq, sx, nullptr};
    return hip_status(w8a8::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

int w8a8_gemm_plan(int64_t M, int64_t N, int64_t K, int splitk, int residual, int32_t* out) {
    if (!out || M <= 0 || N <= 0 || check_k(K) != W8A8_OK || splitk < 1 || splitk > W8A8_MAX_SPLITK ||
        M > kMaxDim || N > kMaxDim)
        return W8A8_ERR_INVALID_ARG;
    for (int i = 0; i < 10; ++i) out[i] = 0;
    w8a8::PanelPlan pp;
    bool panel = false;
    if (splitk == 1 && pick_skinny(M, N, K, residual != 0, &pp, &panel)) {
        out[0] = 0;
        return W8A8_OK;
    }
    if (panel || pick_panel(M, N, K, splitk, residual != 0, &pp)) {
        int mw = 0, nb = 0, nset = 0, nslot = 0;
        w8a8::panel_kind_shape(pp.kind, &mw, &nb, &nset, &nslot);
        const int32_t v[10] = {2, pp.kind, pp.R, pp.P, pp.S, pp.kb_per_split, mw, nb, nset, nslot};
        for (int i = 0; i < 10; ++i) out[i] = v[i];
        return W8A8_OK;
    }
    const GemmPlan plan = w8a8::plan_gemm(M, N, K, splitk);
    const int32_t v[10] = {1, static_cast<int32_t>(plan.kind), plan.bm, plan.bn, plan.splitk, 0, 0, 0, 0, 0};
    for (int i = 0; i < 10; ++i) out[i] = v[i];
    return W8A8_OK;
}

int w8a8_gemm_panel_forced(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                           const float* residual, float* y, int64_t M, int64_t N, int64_t K,
                           const int32_t* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return W8A8_ERR_INVALID_ARG;
    if (const int rc = check_gemm_args(xq, sx, w, sw, residual, y, M, N, K)) return rc;
    if (M == 0 || N == 0) return W8A8_OK;
    w8a8::PanelPlan pp;
    if (plan[3] < 1 || plan[3] > W8A8_MAX_SPLITK ||
        !w8a8::make_panel_plan(M, N, K, plan[0], plan[1], plan[2], plan[3], &pp))
        return W8A8_ERR_INVALID_ARG;
    if (pp.S > 1) {
        const size_t need = w8a8::gemm_workspace_bytes(M, N, pp.S);
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W8A8_ERR_WORKSPACE;
    }
    const GemmArgs a{xq, sx, w, sw, residual, y, M, N, K, nullptr};
    return hip_status(w8a8::launch_panel(a, pp, workspace, static_cast<hipStream_t>(stream)));
}

int w8a8_gemm(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
              const float* residual, float* y, int64_t M, int64_t N, int64_t K, void* stream) {
    if (const int rc = check_gemm_args(xq, sx, w, sw, residual, y, M, N, K)) return rc;
    if (M == 0 || N == 0) return W8A8_OK;
    return run_gemm(xq, sx, w, sw, residual, y, M, N, K, 1, nullptr, static_cast<hipStream_t>(stream));
}

size_t w8a8_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splitk) {
    if (M < 0 || N < 0 || check_k(K) != W8A8_OK || splitk < 1 || splitk > W8A8_MAX_SPLITK ||
        M > kMaxDim || N > kMaxDim)
        return static_cast<size_t>(-1);
    if (splitk == 1 || M == 0 || N == 0) return 0;
    return w8a8::gemm_workspace_bytes(M, N, splitk);
}

int w8a8_gemm_splitk(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                     const float* residual, float* y, int64_t M, int64_t N, int64_t K, int splitk,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (splitk < 1 || splitk > W8A8_MAX_SPLITK) return W8A8_ERR_INVALID_ARG;
    if (const int rc = check_gemm_args(xq, sx, w, sw, residual, y, M, N, K)) return rc;
    if (M == 0 || N == 0) return W8A8_OK;
    if (splitk > 1) {
        const size_t need = w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk);
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W8A8_ERR_WORKSPACE;
    }
    return run_gemm(xq, sx, w, sw, residual, y, M, N, K, splitk, workspace,
                    static_cast<hipStream_t>(stream));
}

int w8a8_gemm_splitk_noalloc(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                             const float* residual, float* y, int64_t M, int64_t N, int64_t K, int splitk,
                             void* stream) {
    if (splitk < 1 || splitk > W8A8_MAX_SPLITK) return W8A8_ERR_INVALID_ARG;
    if (const int rc = check_gemm_args(xq, sx, w, sw, residual, y, M, N, K)) return rc;
    if (M == 0 || N == 0) return W8A8_OK;
    void* ws = nullptr;
    if (splitk > 1) {
        if (w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk) > W8A8_NOALLOC_SCRATCH_BYTES)
            return W8A8_ERR_WORKSPACE;
        if (const int rc = scratch_address(&ws)) return rc;
    }
    return run_gemm(xq, sx, w, sw, residual, y, M, N, K, splitk, ws, static_cast<hipStream_t>(stream));
}

int w8a8_readout_candidates(const int8_t* xq, const float* sx, int64_t M, int64_t K,
                            const int8_t* w_vocab, const float* sw_vocab, int64_t V,
                            const int32_t* cand, int64_t C, float* logits, int32_t* err_flag,
                            void* stream) {
    if (const int rc = check_readout_args(xq, sx, M, K, w_vocab, sw_vocab, V, cand, C, logits, err_flag))
        return rc;
    if (M == 0 || C == 0) return W8A8_OK;
    return run_readout(xq, sx, M, K, w_vocab, sw_vocab, V, cand, C, logits, err_flag,
                       static_cast<hipStream_t>(stream));
}

int w8a8_row_absmax(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                    const float* smooth, int64_t M, int64_t K, int accumulate, float* amax,
                    void* stream) {
    if (!amax && M > 0) return W8A8_ERR_INVALID_ARG;
    // the same checks as quantisation, with amax standing in for xq and sx
    if (const int rc = check_quantize_args(x, ldx, x_rows, row_idx, smooth, M, K,
                                           reinterpret_cast<const int8_t*>(x), amax))
        return rc;
    if (M == 0) return W8A8_OK;
    const w8a8::QuantArgs a{x, ldx, x_rows, row_idx, smooth, M, K, nullptr, nullptr, nullptr};
    return hip_status(w8a8::launch_row_absmax(a, accumulate != 0, amax, static_cast<hipStream_t>(stream)));
}

int w8a8_quantize_act_amax(const float* x, int64_t ldx, int64_t x_rows, const int32_t* row_idx,
                           const float* smooth, const float* amax, int64_t M, int64_t K, int8_t* xq,
                           float* sx, void* stream) {
    if (const int rc = check_quantize_args(x, ldx, x_rows, row_idx, smooth, M, K, xq, sx)) return rc;
    if (M == 0) return W8A8_OK;
    if (!amax) return W8A8_ERR_INVALID_ARG;
    if (!aligned(amax, 4)) return W8A8_ERR_ALIGN;
    const w8a8::QuantArgs a{x, ldx, x_rows, row_idx, smooth, M, K, xq, sx, amax};
    return hip_status(w8a8::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

int w8a8_gemm_int32(const int8_t* xq, const int8_t* w, int64_t M, int64_t N, int64_t K, int32_t* acc,
                    void* stream) {
    if (M < 0 || N < 0) return W8A8_ERR_INVALID_ARG;
    if (const int kc = check_k(K)) return kc;
    if (M > kMaxDim || N > kMaxDim) return W8A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!xq || !w || !acc) return W8A8_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(w, 16) || !aligned(acc, 16)) return W8A8_ERR_ALIGN;
    const GemmArgs a{xq, nullptr, w, nullptr, nullptr, nullptr, M, N, K, acc};
    w8a8::PanelPlan pp;
    if (pick_panel(M, N, K, 1, false, &pp))
        return hip_status(w8a8::launch_panel(a, pp, nullptr, static_cast<hipStream_t>(stream)));
    const GemmPlan plan = w8a8::plan_gemm(M, N, K, 1);
    return hip_status(w8a8::launch_gemm_tiled(a, plan, nullptr, static_cast<hipStream_t>(stream)));
}

int w8a8_epilogue_int32(const int32_t* parts, int S, const float* sx, const float* sw,
                        const float* residual, float* y, int64_t M, int64_t N, void* stream) {
    if (M < 0 || N < 0 || S < 1 || S > W8A8_MAX_SPLITK) return W8A8_ERR_INVALID_ARG;
    if (M > kMaxDim || N > kMaxDim) return W8A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!parts || !sx || !sw || !y) return W8A8_ERR_INVALID_ARG;
    if (!aligned(parts, 4) || !aligned(sx, 4) || !aligned(sw, 4) || !aligned(y, 4)) return W8A8_ERR_ALIGN;
    const size_t out = static_cast<size_t>(M) * static_cast<size_t>(N) * 4;
    if (overlaps(parts, out * static_cast<size_t>(S), y, out)) return W8A8_ERR_INVALID_ARG;
    if (residual) {
        if (!aligned(residual, 4)) return W8A8_ERR_ALIGN;
        if (residual != y && overlaps(residual, out, y, out)) return W8A8_ERR_INVALID_ARG;
    }
    const GemmArgs a{nullptr, sx, nullptr, sw, residual, y, M, N, 0, nullptr};
    return hip_status(w8a8::launch_reduce(a, S, parts, static_cast<hipStream_t>(stream)));
}

int w8a8_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N, int64_t K,
                         int8_t* w, float* sw, void* stream) {
    if (N < 0) return W8A8_ERR_INVALID_ARG;
    if (const int kc = check_k(K)) return kc;
    if (N > W8A8_MAX_ROWS) return W8A8_ERR_SHAPE;
    if (N == 0) return W8A8_OK;
    if (!q || !d || !smooth || !w || !sw) return W8A8_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(d, 2) || !aligned(smooth, 16) || !aligned(w, 16) || !aligned(sw, 4))
        return W8A8_ERR_ALIGN;
    const size_t bytes = static_cast<size_t>(N) * static_cast<size_t>(K);
    if (overlaps(q, bytes, w, bytes) && q != w) return W8A8_ERR_INVALID_ARG;
    return hip_status(w8a8::launch_requantize_q8_0(q, d, smooth, N, K, w, sw, static_cast<hipStream_t>(stream)));
}

int w8a8_candidate_softmax(const float* logits, int64_t M, int64_t C, double* probs, void* stream) {
    if (const int rc = check_softmax_args(logits, M, C, probs)) return rc;
    return hip_status(w8a8::launch_candidate_softmax(logits, M, C, probs, static_cast<hipStream_t>(stream)));
}

int w8a8_answer_head(const float* h, int64_t ldh, int64_t h_rows, const int32_t* answer_rows,
                     int64_t M, const float* smooth, int64_t K, const int8_t* w_vocab,
                     const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C, int8_t* xq,
                     float* sx, float* logits, double* probs, int32_t* err_flag, void* stream) {
    if (!answer_rows && M > 0) return W8A8_ERR_INVALID_ARG;
    if (const int rc = check_quantize_args(h, ldh, h_rows, answer_rows, smooth, M, K, xq, sx)) return rc;
    if (const int rc = check_readout_args(xq, sx, M, K, w_vocab, sw_vocab, V, cand, C, logits, err_flag))
        return rc;
    if (const int rc = check_softmax_args(logits, M, C, probs)) return rc;
    if (M == 0) return W8A8_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (w8a8::answer_head_fused_fits(K)) {
        const w8a8::AnswerHeadArgs a{h, ldh, h_rows, answer_rows, M, smooth, K, w_vocab, sw_vocab, V,
                                     cand, C, xq, sx, logits, probs, err_flag};
        return hip_status(w8a8::launch_answer_head(a, s));
    }
    const w8a8::QuantArgs q{h, ldh, h_rows, answer_rows, smooth, M, K, xq, sx, nullptr};
    if (const int rc = hip_status(w8a8::launch_quantize(q, s))) return rc;
    if (C == 0) return W8A8_OK;
    if (const int rc = run_readout(xq, sx, M, K, w_vocab, sw_vocab, V, cand, C, logits, err_flag, s))
        return rc;
    return hip_status(w8a8::launch_candidate_softmax(logits, M, C, probs, s));
}

}  // extern "C"

namespace {

int check_readout_args(const int8_t* xq, const float* sx, int64_t M, int64_t K, const int8_t* w_vocab,
                       const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C,
                       const float* logits, const int32_t* err_flag) {
    if (M < 0 || C < 0 || V <= 0) return W8A8_ERR_INVALID_ARG;
    if (const int kc = check_k(K)) return kc;
    if (C > W8A8_MAX_CANDIDATES) return W8A8_ERR_TOO_MANY_CANDIDATES;
    if (M > W8A8_MAX_ROWS || V > kMaxDim) return W8A8_ERR_SHAPE;
    if (M == 0 || C == 0) return W8A8_OK;
    if (!xq || !sx || !w_vocab || !sw_vocab || !cand || !logits) return W8A8_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(w_vocab, 16) || !aligned(sx, 4) || !aligned(sw_vocab, 4) ||
        !aligned(cand, 4) || !aligned(logits, 4))
        return W8A8_ERR_ALIGN;
    if (err_flag && !aligned(err_flag, 4)) return W8A8_ERR_ALIGN;
    return W8A8_OK;
}

int run_readout(const int8_t* xq, const float* sx, int64_t M, int64_t K, const int8_t* w_vocab,
                const float* sw_vocab, int64_t V, const int32_t* cand, int64_t C, float* logits,
                int32_t* err_flag, hipStream_t s) {
    // One workgroup per row (the answer head's candidate scoring) where the
    // row fits its registers: 3 rows x 4 candidates of a 5120-wide lm_head
    // take 3.3 us per launch back to back against 4.9 us on the skinny
    // kernel, 64 rows x 16 candidates 6.9 against 16.3 us.
    if (w8a8::answer_head_fused_fits(K)) {
        const w8a8::ReadoutRowsArgs a{xq, sx, M, K, w_vocab, sw_vocab, V, cand, C, logits, err_flag};
        return hip_status(w8a8::launch_readout_rows(a, s));
    }
    // Otherwise the skinny kernel, 64 answer rows per launch; each launch
    // gathers M_chunk * C weight rows.
    for (int64_t m0 = 0; m0 < M; m0 += w8a8::SKINNY_MAX_M) {
        const int64_t mc = (M - m0 < w8a8::SKINNY_MAX_M) ? (M - m0) : w8a8::SKINNY_MAX_M;
        w8a8::SkinnyArgs a{xq + m0 * K, sx + m0, w_vocab, sw_vocab, nullptr, logits + m0 * C,
                           mc, mc * C, K, 0, cand + m0 * C, V, C, err_flag};
        if (const int rc = hip_status(w8a8::launch_skinny(a, s))) return rc;
    }
    return W8A8_OK;
}

int check_softmax_args(const float* logits, int64_t M, int64_t C, const double* probs) {
    if (M < 0 || C < 0) return W8A8_ERR_INVALID_ARG;
    if (C > W8A8_MAX_CANDIDATES) return W8A8_ERR_TOO_MANY_CANDIDATES;
    if (M > W8A8_MAX_ROWS) return W8A8_ERR_SHAPE;
    if (M == 0 || C == 0) return W8A8_OK;
    if (!logits || !probs) return W8A8_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(probs, 8)) return W8A8_ERR_ALIGN;
    // the read-out writes logits while the softmax reads them: no overlap
    // with the probabilities
    if (overlaps(logits, static_cast<size_t>(M * C) * 4, probs, static_cast<size_t>(M * C) * 8))
        return W8A8_ERR_INVALID_ARG;
    return W8A8_OK;
}

}  // namespace
