"""Host-side launch and traffic arithmetic for the tiled product (analysis only; no GPU work).

- ``wave_utilization``: tiles, waves and utilisation when a grid of output tiles runs on a number
  of compute units, one tile per unit at a time (02_gpu_execution_model.py, CS336 lecture 5,
  part 5 "wave quantization": ceil-divided tile counts, ceil-divided waves, utilisation = tiles /
  (waves x units)).
- ``tile_order``: program id -> (tile row, tile column) under row-major or grouped order
  (06_triton_style.py, CS349E lecture 10, the matmul kernel's program-id mapping).  The GPU library
  exports its own device-side mapping (``gemm_f16_f32_tile_order``); this is the plain-Python one
  for the traffic model below.
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


def wave_utilization(n: int, tile_m: int, tile_n: int, units: int, m: int | None = None):
    """(tiles, waves, utilisation) for an m x n output (m defaults to n) in tile_m x tile_n tiles."""
    m = n if m is None else m
    tiles = cdiv(m, tile_m) * cdiv(n, tile_n)
    waves = cdiv(tiles, units)
    return tiles, waves, tiles / (waves * units)


def tile_order(tiles_m: int, tiles_n: int, group_m: int | None = None):
    """Lists (pm, pn) indexed by program id; group_m None (or 1) is row-major order."""
    pm, pn = [], []
    for pid in range(tiles_m * tiles_n):
        if group_m is None:
            pm.append(pid // tiles_n)
            pn.append(pid % tiles_n)
            continue
        per_group = group_m * tiles_n
        group = pid // per_group
        first = group * group_m
        rows = min(tiles_m - first, group_m)
        pm.append(first + (pid % per_group) % rows)
        pn.append((pid % per_group) // rows)
    return pm, pn


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
