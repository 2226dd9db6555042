"""Which rows and columns of a large result the parity tests compare with the oracle (test helper).

``strata(n)`` picks indices along an extent of n so that every part of every output tile is
reached, whatever the tile (64, 128 or 256 wide) and the launch split:

- one index in every 32-wide band -- a 32 x 32 MFMA block and one band of the epilogue -- with
  its offset inside the band stepping by 13 (coprime to 32), so over the bands every one of the
  32 lane rows (columns) of a block is compared;
- both sides of every multiple of 128 (the edges of 128-wide wave tiles and tiles, which include
  every 256 edge);
- the first and the last index.

Compared along full rows and full columns, the union reaches every output tile, every 32-row band
of each tile and every (wave row, band) pair.  tests/test_sampling.py checks these properties.
"""
from __future__ import annotations

import numpy as np

BAND = 32
STEP = 13


def strata(n: int) -> np.ndarray:
    if n <= 0:
        return np.zeros(0, np.int64)
    idx = {0, n - 1}
    for b in range(-(-n // BAND)):
        idx.add(min(b * BAND + (b * STEP) % BAND, n - 1))
    for e in range(128, n, 128):
        idx.update((e - 1, e))
    return np.array(sorted(idx), dtype=np.int64)
