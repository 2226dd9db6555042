"""Host-side launch and traffic arithmetic for the tiled product (analysis only; no GPU work).

- ``tile_count`` / ``wave_utilization``: an output grid of ceil-divided tiles, run one tile per
  compute unit at a time, takes ceil(tiles / units) waves; the last wave may leave units idle, so
  the utilisation is tiles / (waves x units) (02_gpu_execution_model.py, CS336 lecture 5, part 5
  "wave quantization").
- ``tile_order``: program id -> (tile row, tile column) under row-major or grouped order
  (06_triton_style.py, CS349E lecture 10, demo 2: bands of GROUP_M tile rows, walked down one
  tile column at a time inside a band).  Built here by enumerating that definition; the GPU
  library exports its own closed-form device mapping (``gemm_f16_f32_tile_order``), and the tests
  check one against the other.
- ``dram_bytes_tiled``: the pages' wave model of DRAM traffic (04_tensor_cores.py demo 3 and
  06_triton_style.py demo 2): the tiles of one wave advance through K together and share the
  cache, so each wave reads every distinct tile-row of A and tile-column of B it touches once;
  the C write is added once.  The pages name this model without printing it; this reading is
  the one that reproduces every figure they print (see tests/test_model.py).
- ``l2_bytes``: the per-program read volume (M.K.N/BN + K.N.M/BM) x element size
  (06_triton_style.py demo 1).
- ``softmax_traffic``: element loads and stores of the row softmax as five separate kernels
  (max, subtract, exp, sum, divide) or as one fused program per row (06_triton_style.py demo 3).
"""
from __future__ import annotations

import math


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def tile_count(m: int, n: int, bm: int, bn: int) -> int:
    """Output tiles of an m x n result in bm x bn tiles (partial tiles at the edges count)."""
    return cdiv(m, bm) * cdiv(n, bn)


def wave_utilization(tiles: int, units: int) -> tuple[int, float]:
    """(waves, utilisation) for `tiles` equal tiles on `units` compute units, one at a time each."""
    waves = cdiv(tiles, units)
    return waves, (tiles / (waves * units) if waves else 0.0)


def tile_order(tiles_m: int, tiles_n: int, group_m: int | None = None):
    """Lists (pm, pn) indexed by program id; group_m None (or 1) is row-major order.

    Enumerates the definition directly: bands of group_m consecutive tile rows, in order; inside a
    band, every tile column from left to right, and inside a column the band's rows from the top."""
    g = 1 if group_m is None else group_m
    order = []
    if g == 1:
        order = [(r, c) for r in range(tiles_m) for c in range(tiles_n)]
    else:
        for top in range(0, tiles_m, g):
            band = range(top, min(top + g, tiles_m))
            order.extend((r, c) for c in range(tiles_n) for r in band)
    return [r for r, _ in order], [c for _, c in order]


def dram_bytes_tiled(n: int, bm: int, bn: int, per_unit: int, units: int, elem: int = 2,
                     group: int | None = None) -> int:
    """Wave-model DRAM bytes for an n x n x n product in bm x bn tiles, per_unit tiles per unit."""
    tm, tn = cdiv(n, bm), cdiv(n, bn)
    pm, pn = tile_order(tm, tn, group)
    per_wave = per_unit * units
    total = 0
    for w0 in range(0, tm * tn, per_wave):
        rows = set(pm[w0:w0 + per_wave])
        cols = set(pn[w0:w0 + per_wave])
        total += (len(rows) * bm + len(cols) * bn) * n * elem
    return total + n * n * elem


def l2_bytes(M: int, N: int, K: int, bm: int, bn: int, elem: int = 2) -> int:
    """Bytes the programs read from the cache level above LDS: A once per tile column, B once per
    tile row (ceil-divided for ragged edges)."""
    return (M * K * cdiv(N, bn) + K * N * cdiv(M, bm)) * elem


def softmax_traffic(M: int, N: int, fused: bool) -> tuple[int, int]:
    """(elements loaded, elements stored) for the row softmax of an M x N matrix.

    Operator by operator, each kernel reads its whole input from memory and writes its whole
    output back: the row maximum reads MN and writes M; the subtraction reads MN plus one
    maximum per row and writes MN; exp reads and writes MN; the row sum reads MN and writes M;
    the division reads MN plus one sum per row and writes MN.  Fused, one program reads its row
    once and writes it once."""
    if fused:
        return M * N, M * N
    kernels = [(M * N, M), (M * N + M, M * N), (M * N, M * N), (M * N, M), (M * N + M, M * N)]
    return sum(k[0] for k in kernels), sum(k[1] for k in kernels)
