"""Host-side checks of the column-panel GEMM's launch plans (no GPU).

The planner runs in the library (w8a8_gemm_plan reports its choice).  This
file mirrors, in Python, the index arithmetic the panel kernel does with a
plan: block -> (panel, K split, row split), the waves' row blocks, the
weight-staging chunks and the activation fragments.  For many shapes it
checks that every output element is produced exactly once per K split,
that the K splits tile [0, K) without overlap, that every global read stays
inside its matrix, that every LDS access stays inside the ring, and that
no wave or panel exceeds its kernel configuration's limits.  These are the
properties that keep the kernel in bounds and its integer sums complete.
"""
import itertools

import numpy as np
import pytest

from deterministic_w8a8_int8_amd import binding as B

NXCD, KBS, ROW_BYTES, THREADS, LDS_LIMIT = 8, 2, 128, 256, 160 * 1024
OUT_OF_RANGE = 0x40000000


def block_map(nblocks):
    """Hardware block id -> the kernel's XCD-contiguous linear id."""
    lids = []
    per, extra = divmod(nblocks, NXCD)
    for bid in range(nblocks):
        xcd, slot = bid % NXCD, bid // NXCD
        lid = xcd * (per + 1) + slot if xcd < extra else extra * (per + 1) + (xcd - extra) * per + slot
        lids.append(lid)
    return lids


def swz(r):
    return ((r >> 2) & 3) * 2 + ((r >> 1) & 1)


def check_plan(M, N, K, plan):
    path, kind, R, P, S, kps, MW, NB, NSET, NSLOT = plan
    assert path == 2
    assert NSLOT in (2, 3) and NSET >= NSLOT - 1
    rb_total, cb, KB = -(-M // 16), -(-N // 16), K // 64
    cb_base, cb_extra = divmod(cb, P)
    AR, BR = 64 * MW, 16 * NB
    RPAD = (AR + BR + 31) // 32 * 32
    QPT, QA = RPAD // 32, AR // 32
    STAGE = RPAD * ROW_BYTES
    assert NSLOT * STAGE <= LDS_LIMIT, "LDS ring"
    LDR = 16 * NB + 4
    assert 64 * LDR * 4 <= NSLOT * STAGE, "epilogue parking fits the ring"
    assert (64 * 4 * NB) % THREADS == 0
    assert 4 * MW * NB <= 256, "accumulators"
    nblocks = P * R * S
    lids = block_map(nblocks)
    assert sorted(lids) == list(range(nblocks)), "block renumbering is not a permutation"
    cover = np.zeros((S, rb_total, cb), dtype=np.int32)
    kcover = np.zeros(KB, dtype=np.int32)
    t = np.arange(THREADS)
    st_lc = (t & 7) ^ swz(t >> 3)
    lane = np.arange(64)
    for lid in lids:
        r, p, split = lid % R, (lid // R) % P, lid // (R * P)
        assert p < P and split < S
        cb0 = p * cb_base + min(p, cb_extra)
        ncb = cb_base + (1 if p < cb_extra else 0)
        assert 1 <= ncb <= NB, (ncb, NB)
        c0 = 16 * cb0
        kb0 = min(split * kps, KB)
        nkb = min(kb0 + kps, KB) - kb0
        nst = -(-nkb // KBS)
        if r == 0 and p == 0:
            kcover[kb0:kb0 + nkb] += 1
        rs0, rs1 = r * rb_total // R, (r + 1) * rb_total // R
        nrb = rs1 - rs0
        assert nrb >= 1
        row_end, row_first = min(16 * rs1, M), min(16 * rs0, M - 1)
        a_range, b_range = (row_end - row_first) * K, (min(c0 + BR, N) - c0) * K
        assert 0 < a_range < 2 ** 31 and 0 < b_range < 2 ** 31
        for wave in range(4):
            rbw = rs0 + wave * nrb // 4
            mw = rs0 + (wave + 1) * nrb // 4 - rbw
            assert 0 <= mw <= MW, (mw, MW)
            cover[split, rbw:rbw + mw, cb0:cb0 + ncb] += 1
        # staging loads: every in-range offset stays inside its buffer for every stage
        for q in range(QPT):
            sr = (t >> 3) + 32 * q
            if q < QA:
                w, x = sr // (16 * MW), sr % (16 * MW)
                rbw_w = rs0 + w * nrb // 4
                mw_w = rs0 + (w + 1) * nrb // 4 - rbw_w
                row = np.minimum(16 * rbw_w + x, row_end - 1)
                own = (x < 16 * mw_w) & (16 * rbw_w + x < row_end)
                off = np.where(own, (row - row_first) * K + st_lc * 16, OUT_OF_RANGE)
                rng = a_range
            else:
                br = sr - AR
                col = np.minimum(c0 + br, N - 1)
                own = (br < 16 * ncb) & (c0 + br < N)
                off = np.where(own, (col - c0) * K + st_lc * 16, OUT_OF_RANGE)
                rng = b_range
            for st in {0, max(nst - 1, 0)}:
                if nst == 0:
                    break
                lcd = np.where((st_lc >> 2) < nkb - st * KBS, 0, -64)
                soff = (kb0 + st * KBS) * 64
                full = off + lcd + soff
                inb = off != OUT_OF_RANGE
                assert (full[inb] >= 0).all() and (full[inb] + 16 <= rng).all(), (q, st)
                assert (full[~inb] >= rng).all() and (full[~inb] + 16 < 2 ** 31).all()
                # a multiplied chunk (its K-block inside the stage) belongs to this split
                used = inb & ((st_lc >> 2) < min(nkb - st * KBS, KBS))
                kbyte = (full[used] - st_lc[used] * 16 - lcd[used]) % K + st_lc[used] * 16 + lcd[used]
                assert ((kbyte >> 6) >= kb0).all() and ((kbyte >> 6) < kb0 + nkb).all()
            # LDS store offset of piece q inside the ring
            assert (NSLOT - 1) * STAGE + 16 * t.max() + q * 32 * ROW_BYTES + 16 <= NSLOT * STAGE
        # fragment reads inside the ring; 16 lanes of a read hit 16 distinct 16-byte bank groups
        for u in range(KBS):
            f_off = (lane & 15) * ROW_BYTES + (((4 * u + (lane >> 4)) ^ swz(lane & 15)) * 16)
            top_a = 3 * 16 * MW * ROW_BYTES + 16 * (MW - 1) * ROW_BYTES + f_off.max() + 16
            top_b = (AR + 16 * (NB - 1)) * ROW_BYTES + f_off.max() + 16
            assert max(top_a, top_b) <= STAGE
            for ph in range(4):
                b = ((lane[16 * ph:16 * ph + 16] & 15) * ROW_BYTES + f_off[16 * ph:16 * ph + 16] % ROW_BYTES)
                groups = (b % 256) // 16
                assert len(set(groups.tolist())) == 16
            # served 32 lanes at a time over a 512-byte window: 32 distinct groups
            for half in range(2):
                sl = slice(32 * half, 32 * half + 32)
                b = (lane[sl] & 15) * ROW_BYTES + f_off[sl] % ROW_BYTES
                assert len(set(((b % 512) // 16).tolist())) == 32
    assert (kcover == 1).all(), "K splits must tile the K-blocks exactly once"
    assert (cover == 1).all(), "every (row block, column block) once per K split"


SHAPES = [
    (256, 34816, 5120, 1, 0), (256, 5120, 17408, 1, 1), (256, 5120, 17408, 4, 1),
    (256, 5120, 17408, 8, 1), (328, 15360, 5120, 1, 0), (328, 34816, 5120, 1, 0),
    (65, 16, 64, 1, 0), (65, 1000, 128, 1, 0), (100, 333, 192, 2, 1), (127, 4097, 320, 3, 0),
    (200, 17, 64, 1, 1), (300, 50000, 704, 5, 0), (384, 640, 1024, 7, 1), (512, 34816, 5120, 1, 0),
    (97, 5120, 17408, 2, 1), (129, 15360, 5120, 1, 0), (448, 2048, 4096, 16, 0),
]


@pytest.mark.parametrize("M,N,K,S,res", SHAPES)
def test_panel_plan_in_bounds(M, N, K, S, res):
    """The panel plan of each shape (forced, so that shapes the router sends
    to the tiled kernel, like 512 x 34816 x 5120, are checked too)."""
    B.set_tile_override(B.W8A8_TILE_OVERRIDE_PANEL)
    try:
        plan = B.w8a8_gemm_plan(M, N, K, S, res)
    finally:
        B.set_tile_override(-1)
    assert plan[0] == 2, (M, N, K, S, plan)
    assert 1 <= plan[4] <= S
    check_plan(M, N, K, plan)


def test_panel_plan_forced_small_and_ragged():
    """With the panel kernel forced, small and ragged shapes still plan in bounds."""
    B.set_tile_override(B.W8A8_TILE_OVERRIDE_PANEL)
    try:
        for M, N, K, S in itertools.product([1, 15, 16, 17, 63, 64, 200], [1, 15, 17, 300], [64, 192, 1024], [1, 3]):
            plan = B.w8a8_gemm_plan(M, N, K, S, 0)
            assert plan[0] == 2, (M, N, K, S, plan)
            check_plan(M, N, K, plan)
    finally:
        B.set_tile_override(-1)


def test_panel_default_range():
    """By default the panel kernel takes M <= 384, except full products with
    M <= 16 whose weights the skinny kernel
    streams through LDS (the full-vocabulary read-out): at least 1024 column
    tiles and M rows of K + 16 bytes within 40 KiB; and narrow layers of a
    few rows with K >= 4096 (N <= 8192, M * N <= 65536), where the skinny
    kernel splits K over its waves.  From 385 to 1024 rows
    the two kernels' time models decide (the decisions below are the faster
    kernel as measured on MI355X); from 1025 to 1536 rows the panel kernel
    runs only where its estimate is the lower one; past 1536 rows the tiled
    kernel runs."""
    assert B.w8a8_gemm_plan(1, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(64, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(3, 248000, 5120, 1, 0)[0] == 0
    assert B.w8a8_gemm_plan(7, 16384, 5120, 1, 0)[0] == 0    # 7 rows of K + 16 bytes fit 40 KiB of LDS
    assert B.w8a8_gemm_plan(8, 16384, 5120, 1, 0)[0] == 2    # 8 do not
    assert B.w8a8_gemm_plan(7, 16368, 5120, 1, 0)[0] == 2    # 1023 column tiles
    assert B.w8a8_gemm_plan(3, 248000, 5120, 2, 0)[0] == 2   # split-K: not the skinny kernel
    # narrow long-K layers of a few rows: the skinny kernel splits K over waves
    assert B.w8a8_gemm_plan(1, 1024, 17408, 1, 1)[0] == 0
    assert B.w8a8_gemm_plan(8, 5120, 17408, 1, 1)[0] == 0
    assert B.w8a8_gemm_plan(12, 5120, 5120, 1, 0)[0] == 0
    assert B.w8a8_gemm_plan(16, 4096, 17408, 1, 0)[0] == 0
    assert B.w8a8_gemm_plan(16, 5120, 17408, 1, 1)[0] == 2   # M * N past 65536
    assert B.w8a8_gemm_plan(4, 10240, 5120, 1, 0)[0] == 2    # N past 8192
    assert B.w8a8_gemm_plan(1, 4096, 2048, 1, 0)[0] == 2     # K below 4096: launch-bound either way
    assert B.w8a8_gemm_plan(65, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(512, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(513, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(1025, 4096, 1024, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(640, 34816, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(768, 15360, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(896, 34816, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(896, 15360, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(1024, 5120, 17408, 1, 1)[0] == 2
    assert B.w8a8_gemm_plan(1024, 5120, 17408, 8, 1)[0] == 2
    assert B.w8a8_gemm_plan(1024, 5120, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(1280, 5120, 17408, 1, 1)[0] == 2   # 1025-1536 rows: the panel estimate must win
    assert B.w8a8_gemm_plan(1536, 5120, 17408, 1, 1)[0] == 2
    assert B.w8a8_gemm_plan(1280, 34816, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(1536, 15360, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(1536, 5120, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(1537, 5120, 17408, 1, 1)[0] == 1
    assert B.w8a8_gemm_plan(2048, 5120, 17408, 1, 1)[0] == 1
    assert B.w8a8_gemm_plan(384, 34816, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(385, 34816, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(512, 34816, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(480, 25000, 5120, 1, 0)[0] == 1
    assert B.w8a8_gemm_plan(512, 20000, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(512, 15360, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(448, 5120, 5120, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(512, 5120, 17408, 8, 1)[0] == 2
    assert B.w8a8_gemm_plan(500, 4096, 256, 1, 0)[0] == 2    # a few microseconds: launch-bound
    B.set_tile_override(B.W8A8_TILE_OVERRIDE_PANEL)
    try:
        assert B.w8a8_gemm_plan(448, 34816, 5120, 1, 0)[0] == 2
    finally:
        B.set_tile_override(-1)
    for kind in range(B.W8A8_TILE_OVERRIDE_PANEL):
        B.set_tile_override(kind)
        try:
            assert B.w8a8_gemm_plan(256, 34816, 5120, 1, 0)[0] == 1
        finally:
            B.set_tile_override(-1)
    B.set_tile_override(B.W8A8_TILE_OVERRIDE_SKINNY)
    try:
        assert B.w8a8_gemm_plan(64, 4096, 1024, 1, 0)[0] == 0
        assert B.w8a8_gemm_plan(65, 4096, 1024, 1, 0)[0] == 1
    finally:
        B.set_tile_override(-1)


def test_forced_plan_sample_in_bounds():
    """Every forced plan the GPU parity test runs (panel_cases.sample_plans)
    keeps the kernel's reads, writes and LDS accesses in bounds."""
    from panel_cases import SHAPES, sample_plans
    n = 0
    for M, N, K, _ in SHAPES:
        good, bad = sample_plans(M, N, K)
        assert len(good) >= 6 and bad, (M, N, K)
        for _, t in good:
            check_plan(M, N, K, t)
            n += 1
    assert n >= 24
