"""The test-side conversion to the stored block layout matches the documented formula."""
import numpy as np

from tests.gpu_util import blocks_from_panels, blocks_to_panels


def test_panel_layout_formula_and_roundtrip():
    r = np.random.default_rng(0)
    B = r.integers(0, 1000, (3, 64, 64))
    P = blocks_to_panels(B)
    flat = P.reshape(3, -1)
    for i in (0, 5, 63):
        for j in (0, 15, 16, 47, 63):
            assert flat[1, (j // 16) * 1024 + i * 16 + j % 16] == B[1, i, j]
    assert np.array_equal(blocks_from_panels(P), B)
