"""The GPU tests' row sampler covers every row tile of the launch shapes."""
import numpy as np
import pytest

from parity_util import tile_rows


@pytest.mark.parametrize("m", [8, 255, 256, 257, 4096, 5120, 14336, 17920, 18944])
def test_tile_rows_cover_every_tile(m):
    rows = tile_rows(m, 3)
    assert rows.min() >= 0 and rows.max() == m - 1 and np.all(np.diff(rows) > 0)
    for tile in (128, 256, 512):
        covered = set((rows // tile).tolist())
        assert covered == set(range((m + tile - 1) // tile))
