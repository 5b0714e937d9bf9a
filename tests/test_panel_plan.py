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

NXCD, KBS, NSTB, ROW_BYTES = 8, 4, 3, 256


def block_map(nblocks):
    """Hardware block id -> the kernel's XCD-contiguous linear id."""
    lids = []
    per, extra = divmod(nblocks, NXCD)
    for bid in range(nblocks):
        xcd, slot = bid % NXCD, bid // NXCD
        lid = xcd * (per + 1) + slot if xcd < extra else extra * (per + 1) + (xcd - extra) * per + slot
        lids.append(lid)
    return lids


def check_plan(M, N, K, plan):
    path, kind, R, P, S, kps, MW, NB = plan
    assert path == 2
    rb_total, cb, KB = -(-M // 16), -(-N // 16), K // 64
    cb_base, cb_extra = divmod(cb, P)
    nblocks = P * R * S
    lids = block_map(nblocks)
    assert sorted(lids) == list(range(nblocks)), "block renumbering is not a permutation"
    cover = np.zeros((S, rb_total, cb), dtype=np.int32)
    kcover = np.zeros(KB, dtype=np.int32)
    lds_bytes = NSTB * NB * 16 * ROW_BYTES
    for lid in lids:
        r, split, p = lid % R, (lid // R) % S, lid // (R * S)
        assert p < P
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
        for wave in range(4):
            rbw = rs0 + wave * nrb // 4
            mw = rs0 + (wave + 1) * nrb // 4 - rbw
            assert 0 <= mw <= MW, (mw, MW)
            cover[split, rbw:rbw + mw, cb0:cb0 + ncb] += 1
            # activation fragments: rows clamped to M-1, bytes 64*kb + 16*grp .. +16
            for i in range(mw):
                rows = np.minimum(16 * (rbw + i) + np.arange(16), M - 1)
                assert rows.min() >= 0 and rows.max() < M
            if nkb:
                assert (kb0 + nkb - 1) * 64 + 48 + 16 <= K
        # weight staging: thread t, row t/16 + 16q (clamped), logical chunk lc
        t = np.arange(256)
        st_lc = (t & 15) ^ (t >> 4)
        for st in range(nst):
            kin = nkb - st * KBS
            lc = np.where((st_lc >> 2) < kin, st_lc, st_lc & 3)
            kbyte = kb0 * 64 + st * ROW_BYTES + lc * 16
            assert kbyte.min() >= 0 and (kbyte + 16).max() <= K
            # the chunk's K-block lies inside this split whenever it is multiplied
            used = (lc >> 2) < min(kin, KBS)
            assert ((kbyte[used] >> 6) < kb0 + nkb).all()
        for q in range(ncb):
            col = np.minimum(c0 + 16 * q + (t >> 4), N - 1)
            assert col.max() < N
            assert (col - c0).max() * K < 2 ** 32
            # LDS store and fragment-read offsets inside the ring
            assert (NSTB - 1) * NB * 16 * ROW_BYTES + 16 * 255 + q * 16 * ROW_BYTES + 16 <= lds_bytes
        lane = np.arange(64)
        for u in range(KBS):
            f_off = (lane & 15) * ROW_BYTES + (((4 * u + (lane >> 4)) ^ (lane & 15)) * 16)
            assert f_off.max() + (ncb - 1) * 16 * ROW_BYTES + (NSTB - 1) * NB * 16 * ROW_BYTES + 16 <= lds_bytes
            # bank spread: 16 lanes of one read phase hit 16 distinct 16-byte slots of 256 bytes
            for ph in range(4):
                slots = (f_off[16 * ph:16 * ph + 16] % 256) // 16
                assert len(set(slots.tolist())) == 16
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
    plan = B.w8a8_gemm_plan(M, N, K, S, res)
    if plan[0] != 2:
        pytest.skip("shape not on the panel kernel")
    assert 1 <= plan[4] <= S
    check_plan(M, N, K, plan)


def test_panel_plan_forced_small_and_ragged():
    """With the panel kernel forced, small and ragged shapes still plan in bounds."""
    B.set_tile_override(6)
    try:
        for M, N, K, S in itertools.product([1, 15, 16, 17, 63, 64, 200], [1, 15, 17, 300], [64, 192, 1024], [1, 3]):
            plan = B.w8a8_gemm_plan(M, N, K, S, 0)
            if S == 1 and M <= 64:
                assert plan[0] == 0   # the skinny kernel keeps M <= 64 without split-K
                continue
            assert plan[0] == 2, (M, N, K, S, plan)
            check_plan(M, N, K, plan)
    finally:
        B.set_tile_override(-1)


def test_panel_default_range():
    """By default the panel kernel takes 64 < M <= 512 and nothing else."""
    assert B.w8a8_gemm_plan(64, 4096, 1024, 1, 0)[0] == 0
    assert B.w8a8_gemm_plan(65, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(512, 4096, 1024, 1, 0)[0] == 2
    assert B.w8a8_gemm_plan(513, 4096, 1024, 1, 0)[0] == 1
    for kind in range(6):
        B.set_tile_override(kind)
        try:
            assert B.w8a8_gemm_plan(256, 34816, 5120, 1, 0)[0] == 1
        finally:
            B.set_tile_override(-1)
