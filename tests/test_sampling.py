"""The stratified sampling of the full-size parity tests reaches every output tile (host only)."""
import numpy as np
import pytest

from sampling import strata


@pytest.mark.parametrize("n", [1, 31, 33, 255, 256, 257, 4097, 4352, 8191, 8192, 32768, 131072])
def test_every_tile_and_band_is_reached(n):
    s = strata(n)
    assert s.min() == 0 and s.max() == n - 1 and np.all(np.diff(s) > 0)
    for tile in (64, 128, 256):
        assert len(set((s // tile).tolist())) == -(-n // tile), tile          # every tile row / column
    assert len(set((s // 32).tolist())) == -(-n // 32)                       # every 32-wide band
    full_bands = s[s < (n // 32) * 32]
    if n >= 32 * 32:
        assert len(set((full_bands % 32).tolist())) == 32                     # every lane row of a block
    if n >= 1024:
        # every (wave row of a 256 tile, band inside the wave tile) pair, i.e. every band offset of a tile
        assert len(set(((s % 256) // 32).tolist())) == 8


def test_tile_edges_both_sides():
    s = set(strata(8192).tolist())
    for e in range(128, 8192, 128):
        assert e - 1 in s and e in s


def test_size_stays_small():
    """At 8192 about 384 rows and columns: 2 x 384 x 8192^2 multiply-adds for the oracle."""
    assert len(strata(8192)) <= 8192 // 32 + 2 * (8192 // 128) + 2
