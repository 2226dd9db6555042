"""Host-side checks of the autotuner: search space, traffic prior, cache (no GPU)."""
import pytest

import dense_tiled_gemm_f16_amd as g
from dense_tiled_gemm_f16_amd import autotune, model


def test_every_candidate_is_a_valid_launch():
    cs = autotune.candidates()
    assert len(cs) == len(autotune.TILES) * len(autotune.GROUP_MS) * len(autotune.XCD_REMAPS)
    for c in cs:
        rc, p = g.gemm_f16_f32_plan(1000, 900, 700, 256, 704, 256, 904, 256, 904, c.opts())
        assert rc == 0, c
        assert (p["bm"], p["bn"]) == autotune.TILES[c.tile] and p["group_m"] == c.group_m


@pytest.mark.parametrize("n,bm,bn,group", [(4096, 128, 128, None), (4096, 128, 128, 8), (4096, 256, 128, 16),
                                           (2048, 256, 256, 4), (1792, 128, 128, 8)])
def test_wave_bytes_generalises_the_pages_model(n, bm, bn, group):
    """On square problems the M x N wave model equals the pages' square model, whose FP16 C term
    (n^2 x 2 bytes) becomes the FP32 C write here."""
    got = autotune._wave_bytes(n, n, n, bm, bn, group or 1)
    pages = model.dram_bytes_tiled(n, bm, bn, 1, autotune.UNITS, elem=2, group=group)
    assert got == pages - n * n * 2 + n * n * 4


def test_prior_orders_tiles_like_the_measurements():
    top = autotune.ranked(8192, 8192, 8192)[0]
    assert top.tile == 1
    r1792 = autotune.ranked(1792, 1792, 1792)
    assert r1792[0].tile == 5          # the 256x256 grid leaves 207 of 256 CUs idle at 1792
    small = autotune.ranked(256, 256, 256)[0]
    assert small.tile in (2, 3, 5)


def test_cache_round_trip(tmp_path):
    path = str(tmp_path / "sub" / "tune.json")
    c = autotune.Cache(path)
    key = autotune.problem_key(1024, 1024, 1024, 0.0, 1024, 1024, 1024, True)
    assert c.get(key) is None
    c.put(key, {"tile": 5, "group_m": 8, "xcd_remap": 1}, 12.5, 14.0)
    c2 = autotune.Cache(path)
    assert c2.get(key) == {"tile": 5, "group_m": 8, "xcd_remap": 1}
    assert autotune.problem_key(1024, 1024, 1024, 1.0, 1024, 1024, 1024, True) != key
