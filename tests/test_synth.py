"""Host checks of the seeded input helpers that the GPU tests rely on."""
import numpy as np
import pytest

from deterministic_w8a8_int8_amd import synth


@pytest.mark.parametrize("M,N,b", [(256, 34816, 16), (328, 15360, 16), (1000, 1000, 32), (17, 33, 16), (1, 5, 16)])
def test_block_points_touch_every_block_once(M, N, b):
    mi, ni = synth.block_points(np.random.default_rng(0), M, N, b, b)
    assert mi.min() >= 0 and mi.max() < M and ni.min() >= 0 and ni.max() < N
    blocks = set(zip((mi // b).tolist(), (ni // b).tolist()))
    assert len(blocks) == mi.size == (-(-M // b)) * (-(-N // b))


def test_sample_points_include_corners():
    mi, ni = synth.sample_points(np.random.default_rng(1), 40, 70, 10)
    pts = set(zip(mi.tolist(), ni.tolist()))
    assert {(0, 0), (0, 69), (39, 0), (39, 69)} <= pts
