/*
 * w8a8_diag.h -- tuning and diagnostic calls of libw8a8.so (MI355X, gfx950).
 *
 * None of these is part of the W8A8 layer (include/w8a8.h).  They let tests
 * force a kernel choice, report which kernel a shape runs on, and measure
 * what the hardware sustains, so that measured kernel times can be related
 * to the chip's own ceilings.  No call here changes a result bit of the
 * layer.  Conventions (pointers, streams, status codes) are those of w8a8.h.
 */
#ifndef W8A8_DIAG_H
#define W8A8_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "w8a8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* w8a8_set_tile_override value that forces the column-panel kernel. */
#define W8A8_TILE_OVERRIDE_PANEL 7
/* w8a8_set_tile_override value that forces the skinny kernel for M <= 64. */
#define W8A8_TILE_OVERRIDE_SKINNY 8

/* Tuning and test hook (host, process-wide; the setting is one atomic
 * integer, so concurrent calls from several host threads are safe, and the
 * last one wins): force the tile configuration of the tiled GEMM for later
 * calls.  -1 = automatic (the default); 0..6 pick
 * one of the configurations of the tiled kernel (0: 256x256 with 4 waves on
 * 16x16x64 MFMAs, 1:
 * 256x256 with 8 waves and a 4-stage pipeline, 2: 256x128 with two
 * workgroups per CU, 3: 128x128, 4: 256x256 with 8 waves and 128-byte
 * stages, 5: as 4 with the epilogue stored straight from the accumulators,
 * 6: 256x320 with 8 waves);
 * W8A8_TILE_OVERRIDE_PANEL forces the column-panel kernel wherever it can
 * hold the rows (by default it runs for M <= 384, except the M <= 16 full
 * products whose weights the skinny kernel streams through LDS, and for
 * 385 <= M <= 1536 unless the time models put the tiled kernel ahead, as
 * for wide layers whose panels would need two rounds of workgroups);
 * W8A8_TILE_OVERRIDE_SKINNY forces the skinny kernel for every M <= 64 at
 * split-K 1.  It never changes a result bit, only speed.
 * Returns W8A8_ERR_INVALID_ARG for other values. */
int w8a8_set_tile_override(int kind);

/*
 * Diagnostic (host, no GPU call): which kernel w8a8_gemm_splitk would run
 * for this shape, split bound and residual flag (w8a8_gemm is splitk 1),
 * under the current tile override.  out: host int32[10], filled as
 *   out[0] = 0: skinny kernel (M <= 64: the full-vocabulary-style LDS stream,
 *              or when forced); rest 0.
 *   out[0] = 1: tiled kernel; out[1] tile configuration, out[2] and out[3]
 *            the tile's rows and columns, out[4] the K splits; rest 0.
 *   out[0] = 2: column-panel kernel; out[1] its configuration, out[2] row
 *            splits R, out[3] column panels P, out[4] K splits S (at most
 *            splitk), out[5] 64-byte K-blocks per split, out[6] row blocks
 *            of 16 per wave (limit), out[7] column blocks of 16 per panel
 *            (limit), out[8] staging register sets, out[9] LDS slots.
 * Returns W8A8_ERR_INVALID_ARG for an invalid shape or a NULL out.
 */
int w8a8_gemm_plan(int64_t M, int64_t N, int64_t K, int splitk, int residual, int32_t* out);

/*
 * Tuning hook: run w8a8_gemm_splitk's product on the column-panel kernel
 * with a given plan instead of the planner's.  plan: host int32[4] =
 * {configuration, row splits R, column panels P, K splits S}, the fields
 * out[1..4] of w8a8_gemm_plan for a panel plan; the K-blocks per split are
 * the planner's for that S.  The result bits are those of w8a8_gemm (the
 * plan changes only speed).  With S > 1, workspace (device, 256-byte
 * aligned, caller-owned) must hold w8a8_gemm_splitk_workspace_bytes(M, N,
 * K, S) bytes (S * M * N int32 partials, rounded up to 256).  Returns
 * W8A8_ERR_INVALID_ARG for a plan the kernel cannot run on this shape (rows
 * or columns beyond the configuration, S outside 1..W8A8_MAX_SPLITK),
 * W8A8_ERR_WORKSPACE for a missing or short workspace, and otherwise the
 * checks of w8a8_gemm.  Asynchronous on `stream`.
 */
int w8a8_gemm_panel_forced(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                           const float* residual, float* y, int64_t M, int64_t N, int64_t K,
                           const int32_t* plan, void* workspace, size_t workspace_bytes, void* stream);
/*
 * Diagnostic (not part of the layer): launch an MFMA-only kernel that runs
 * int8 MFMAs on register-resident operands, with no memory traffic, so the
 * caller can time the throughput the int8 matrix cores sustain on a given
 * kind of operand data.  operand_kind 0: v_mfma_i32_32x32x32_i8, A and B
 * uniform int8; 1: the same with A shaped like per-token-quantised
 * activations (mostly 0 and +-1), B uniform; 2 and 3: as 0 and 1 with
 * v_mfma_i32_16x16x64_i8 (two per 32x32x32 product, the same operations).
 * blocks x 512 threads run `iters` iterations.  *ops (host,
 * nullable) receives the number of int8 operations (2 per multiply-add)
 * launched.  sink: device int32, written only in the impossible case that
 * an xor of all accumulators equals a fixed constant (it keeps the work
 * alive).  Asynchronous on `stream`.
 */
int w8a8_probe_mfma_ceiling(int operand_kind, int64_t blocks, int64_t iters, int32_t* sink,
                            int64_t* ops, void* stream);

/*
 * Diagnostic (not part of the layer): read `bytes` of device memory at buf
 * once, each of up to 4096 workgroups of 256 threads streaming its own
 * contiguous chunk with 16-byte nontemporal loads (1 KiB per wave
 * instruction), so the caller can time the read bandwidth HBM sustains (use
 * a buffer much larger than the 256 MB last-level cache).  buf: device, 16-byte aligned,
 * bytes a positive multiple of 16.  sink: device int32, written only in the
 * impossible case that an xor of everything read equals a fixed constant.
 * Returns W8A8_ERR_INVALID_ARG for a bad argument.  Asynchronous on `stream`.
 */
int w8a8_probe_stream_read(const void* buf, int64_t bytes, int32_t* sink, void* stream);
/*
 * Diagnostic (not part of the layer): the activation quantizer's traffic
 * mix with none of its arithmetic.  Reads n 4-byte words at src (16-byte
 * nontemporal loads) and writes n bytes at dst (byte i = the top byte of
 * word i), each of up to 4096 workgroups of 256 threads streaming its own
 * contiguous chunk, so the caller can time the rate a 4-read/1-write stream
 * sustains (use buffers much larger than the 256 MB last-level cache).
 * src, dst: device, 16-byte aligned, not overlapping; n a positive multiple
 * of 4.  Returns W8A8_ERR_INVALID_ARG for a bad argument.  Asynchronous on
 * `stream`.
 */
int w8a8_probe_stream_narrow(const void* src, int64_t n, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_DIAG_H */
