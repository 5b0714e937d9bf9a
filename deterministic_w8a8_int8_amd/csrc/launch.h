// Internal launchers behind the C ABI (host side).  Arguments are validated
// by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

struct QuantArgs {
    const float* x;
    int64_t ldx;
    int64_t x_rows;
    const int32_t* row_idx;
    const float* smooth;
    int64_t M;
    int64_t K;
    int8_t* xq;
    float* sx;
    const float* amax;   // given per-token maxima [M], or NULL: each row's own
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// amax_out[m] = exact max_k |fl(x/s)| of row m (max-combined with amax_out[m]
// when accumulate); xq, sx and amax of `a` are unused.
hipError_t launch_row_absmax(const QuantArgs& a, bool accumulate, float* amax_out, hipStream_t stream);

struct GemmArgs {
    const int8_t* xq;
    const float* sx;
    const int8_t* w;
    const float* sw;
    const float* residual;
    float* y;
    int64_t M;
    int64_t N;
    int64_t K;
    int32_t* acc_out;   // non-NULL: write the raw int32 accumulators [M,N] here
                        // instead of the epilogue (splitk 1; sx, sw, residual, y unused)
};

// Tiled MFMA GEMM.  Which tile shape runs depends only on (M, N, K, splitk);
// the workspace query and the launch use the same choice.
// Tile configurations of the tiled kernel (see gemm_tiled.hip):
//   0: 256x256, 4 waves, 128-byte K stages x2      1: 256x256, 8 waves, 64-byte x4
//   2: 256x128, 4 waves, 2 workgroups per CU        3: 128x128, 2 workgroups per CU
//   4: 256x256, 8 waves, 128-byte K stages x2
//   5: as 4, epilogue written straight from the accumulators
//   6: 256x320, 8 waves, 128-byte K stages x2, LDS-staged epilogue in two passes of rows
enum TileKind { TILE_KIND_0 = 0, TILE_KIND_1, TILE_KIND_2, TILE_KIND_3, TILE_KIND_4, TILE_KIND_5, TILE_KIND_6,
                TILE_KINDS };

struct GemmPlan {
    TileKind kind;
    int bm, bn;
    int64_t tiles_m, tiles_n;
    int splitk;
    int group_m;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int splitk);
// Time model of the tiled kernel (us) for routing against the column-panel
// kernel: rounds of full tiles at the per-CU rate measured for 256x320
// tiles, plus launch, prologue and epilogue, plus the split-K reduction.
double tiled_time_estimate_us(int64_t M, int64_t N, int64_t K, int splitk);
// Override of the kernel choice: -1 automatic, 0..TILE_KINDS-1 one tiled
// configuration, PANEL_OVERRIDE the column-panel kernel wherever it fits.
constexpr int PANEL_OVERRIDE = TILE_KINDS;
constexpr int SKINNY_OVERRIDE = TILE_KINDS + 1;   // the skinny kernel for every M <= SKINNY_MAX_M
void set_tile_override(int kind);
int tile_override_value();
size_t gemm_workspace_bytes(int64_t M, int64_t N, int splitk);
hipError_t launch_gemm_tiled(const GemmArgs& a, const GemmPlan& p, void* workspace,
                             hipStream_t stream);
// y = epilogue(P_0 + ... + P_{S-1}) for S int32 slices [S,M,N] (row-major).
hipError_t launch_reduce(const GemmArgs& a, int S, const int32_t* partials, hipStream_t stream);

// Column-panel GEMM for mid-sized M (gemm_panel.hip): R row splits, P column
// panels and S K splits (S > 1 writes int32 partials to the workspace, S
// slices of [M,N], then launch_reduce).  plan_panel picks the configuration
// from (M, N, K, max_splitk, residual) alone, with S <= max_splitk; it returns
// false when the kernel cannot hold the rows.
struct PanelPlan {
    int kind;          // template configuration (rows and columns per wave)
    int R, P, S;
    int kb_per_split;  // 64-byte K-blocks per K split
    double est_us;     // the model's time estimate
};
bool plan_panel(int64_t M, int64_t N, int64_t K, int max_splitk, bool residual, PanelPlan* out);
bool panel_plan_valid(int64_t M, int64_t N, int64_t K, const PanelPlan& p);
// A given plan (kind, R, P, S) with the K-blocks per split the planner would
// use for S; false when the kernel cannot run it on this shape.
bool make_panel_plan(int64_t M, int64_t N, int64_t K, int kind, int R, int P, int S, PanelPlan* out);
// Rows-per-wave and columns-per-panel limits (in blocks of 16), staging
// register sets and LDS slots of a panel kind.
bool panel_kind_shape(int kind, int* mw, int* nb, int* nset, int* nslot);
hipError_t launch_panel(const GemmArgs& a, const PanelPlan& p, void* workspace, hipStream_t stream);

// Skinny-M GEMM (M <= SKINNY_MAX_M): the weight is streamed from HBM once and
// every wave keeps 16 weight rows against all M activation rows.  With
// `gather` the weight row of output column j is gather[j]; with owner_c > 0
// only column j of row j / owner_c is written (the candidate read-out).
constexpr int64_t SKINNY_MAX_M = 64;
// True when a full product of this shape streams its weights through the
// skinny kernel's LDS rings (M <= 16 with many column tiles: the
// full-vocabulary read-out).  There it beats the column-panel kernel; for
// other M <= SKINNY_MAX_M the panel kernel is faster.
bool skinny_streams_lds(int64_t M, int64_t N, int64_t K);

struct SkinnyArgs {
    const int8_t* xq;
    const float* sx;
    const int8_t* w;
    const float* sw;
    const float* residual;
    float* y;
    int64_t M;
    int64_t N;       // output columns (gathered rows when gather != nullptr)
    int64_t K;
    int64_t ldy;
    const int32_t* gather;
    int64_t V;       // rows of w, for bounds checks of gather
    int64_t owner_c; // 0: plain GEMM; C > 0: read-out, column j belongs to row j / C
    int32_t* err_flag;
};

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t stream);

// Startup requantisation of Q8_0 weights with SmoothQuant (requant.hip):
// wq [N,K] and sw [N] from codes q [N,K], binary16 block scales d [N,K/32]
// and the smoothing vector [K]; K % 4 == 0 and K % 32 == 0.
hipError_t launch_requantize_q8_0(const int8_t* q, const uint16_t* d, const float* smooth, int64_t N,
                                  int64_t K, int8_t* wq, float* sw, hipStream_t stream);

// The answer head in one launch (answer_head.hip): quantise the hidden rows
// rows[0..M) of h, score the C candidates of each, candidate softmax; the
// same bits as launch_quantize + launch_readout_rows (or launch_skinny in
// gather/owner mode) + launch_candidate_softmax.  Needs K <= 18432 (answer_head_fused_fits).
struct AnswerHeadArgs {
    const float* h;
    int64_t ldh;
    int64_t h_rows;
    const int32_t* rows;
    int64_t M;
    const float* smooth;
    int64_t K;
    const int8_t* w;
    const float* sw;
    int64_t V;
    const int32_t* cand;
    int64_t C;
    int8_t* xq;
    float* sx;
    float* logits;
    double* probs;
    int32_t* err_flag;
};
bool answer_head_fused_fits(int64_t K);
hipError_t launch_answer_head(const AnswerHeadArgs& a, hipStream_t stream);

// The candidate read-out on given codes (answer_head.hip): one workgroup per
// row scores its C <= 64 candidates with the answer head's code; the same
// bits as launch_skinny in gather/owner mode.  Needs K <= 18432
// (answer_head_fused_fits).
struct ReadoutRowsArgs {
    const int8_t* xq;
    const float* sx;
    int64_t M;
    int64_t K;
    const int8_t* w;
    const float* sw;
    int64_t V;
    const int32_t* cand;
    int64_t C;
    float* logits;
    int32_t* err_flag;
};
hipError_t launch_readout_rows(const ReadoutRowsArgs& a, hipStream_t stream);

// Candidate softmax in binary64, one fixed operation sequence (softmax.hip):
// probs[m, c] for c < C <= 64; rows with a non-finite logit give NaN.
hipError_t launch_candidate_softmax(const float* logits, int64_t M, int64_t C, double* probs,
                                    hipStream_t stream);

// Diagnostic kernels (probes.hip): MFMA-only ceiling, streaming read and
// narrowing stream.
int64_t mfma_ceiling_ops(int64_t blocks, int64_t iters);
hipError_t launch_stream_read(const void* buf, int64_t bytes, int32_t* sink, hipStream_t stream);
hipError_t launch_stream_narrow(const void* src, int64_t n_floats, void* dst, hipStream_t stream);
hipError_t launch_mfma_ceiling(int kind, int64_t blocks, int64_t iters, int32_t* sink,
                               hipStream_t stream);

}  // namespace w8a8
