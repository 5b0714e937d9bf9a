"""Forced column-panel plans shared by a CPU test (every plan's index
arithmetic in bounds, test_panel_plan.py) and a GPU test (every plan's
output against the oracle, test_gpu_panel_plans.py): the GPU runs only plans
the CPU mirror has checked."""
import numpy as np

# Template configurations of the panel kernel: rows of 16 per wave (MW),
# columns of 16 per panel (NB), staging register sets, LDS slots.
KINDS = [(1, 8, 3, 3), (2, 8, 3, 3), (2, 12, 3, 3), (3, 8, 3, 3), (4, 9, 3, 3), (6, 9, 1, 2),
         (1, 4, 3, 3), (2, 3, 3, 3), (2, 4, 3, 3), (2, 5, 3, 3), (4, 5, 3, 3)]
KBS = 2   # 64-byte K-blocks per stage

# (M, N, K, residual): ragged M and N, 65 K-blocks (a short last stage)
SHAPES = [(100, 1000, 2048, False), (257, 2056, 1152, True), (328, 520, 4160, True), (16, 3000, 1024, False)]


def plan_tuple(M, N, K, kind, R, P, S):
    """The w8a8_gemm_plan-style tuple of a forced plan (K-blocks per split as
    the planner computes them), or None when the kernel cannot run it."""
    if not 0 <= kind < len(KINDS) or R < 1 or P < 1 or S < 1:
        return None
    MW, NB, NSET, NSLOT = KINDS[kind]
    rb, cb, KB = (M + 15) // 16, (N + 15) // 16, K // 64
    kps = -(-KB // S)
    if S > 1:
        kps = -(-kps // KBS) * KBS
    if R > rb or P > cb or -(-(-(-rb // R)) // 4) > MW or -(-cb // P) > NB or kps * S < KB:
        return None
    return (2, kind, R, P, S, kps, MW, NB, NSET, NSLOT)


def sample_plans(M, N, K, count=12, seed=0):
    """A seeded sample of up to `count` runnable plans and a few rejected ones."""
    rng = np.random.default_rng(seed + M * 131 + N * 7 + K)
    rb, cb = (M + 15) // 16, (N + 15) // 16
    cand = []
    for kind in range(len(KINDS)):
        for R in range(1, min(rb, 6) + 1):
            for S in (1, 2, 3, 5):
                for P in sorted({1, 2, 3, 7, cb // 4, cb // 2, cb} - {0}):
                    if P <= cb and P * R * S <= 1024:
                        cand.append((kind, R, P, S))
    order = rng.permutation(len(cand))
    good, bad = [], []
    for i in order:
        p = cand[i]
        t = plan_tuple(M, N, K, *p)
        if t is not None and len(good) < count:
            good.append((p, t))
        elif t is None and len(bad) < 3:
            bad.append(p)
    return good, bad
