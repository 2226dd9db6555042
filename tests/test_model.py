"""Host-side launch/traffic arithmetic pinned to the counts the pages print."""
import pytest

from dense_tiled_gemm_f16_amd import model


def test_wave_quantization_page_example(golden):
    """02_gpu_execution_model.py part 5: A100 (108 SMs), 256x128 tiles: 1792 -> 98 tiles in one
    wave; 1793 -> 120 tiles in two waves."""
    g = golden["page_launch_counts"]["wave_quantization"]
    t = model.tile_count(1792, 1792, 256, 128)
    w, _ = model.wave_utilization(t, 108)
    assert (t, w) == (g["n_1792"]["tiles"], g["n_1792"]["waves"])
    t = model.tile_count(1793, 1793, 256, 128)
    w, u = model.wave_utilization(t, 108)
    assert (t, w) == (g["n_1793"]["tiles"], g["n_1793"]["waves"])
    assert abs(u - 120 / 216) < 1e-12


@pytest.mark.parametrize("tile,tiles1792,tiles1793", [((256, 256), 49, 64), ((256, 128), 98, 120),
                                                      ((128, 128), 196, 225)])
def test_wave_quantization_on_256_cus(tile, tiles1792, tiles1793):
    """The same arithmetic for MI355X's 256 compute units: every tile size fits one wave."""
    for n, tiles in ((1792, tiles1792), (1793, tiles1793)):
        t = model.tile_count(n, n, tile[0], tile[1])
        assert (t, model.wave_utilization(t, 256)[0]) == (tiles, 1)


def test_grouped_order_page_example(golden):
    g = golden["page_launch_counts"]["grouped_order_9x9"]
    pm, pn = model.tile_order(9, 9, 3)
    assert [[a, b] for a, b in zip(pm[:9], pn[:9])] == g["group_m_3_first_nine"]
    assert len(set(pm[:9])) * 9 + len(set(pn[:9])) * 9 == g["group_m_3_blocks_read"]
    pm, pn = model.tile_order(9, 9, None)
    assert len(set(pm[:9])) * 9 + len(set(pn[:9])) * 9 == g["row_major_blocks_read"]


def test_library_launch_order_matches_model():
    """The GPU library's exported closed-form mapping equals the enumeration of the grouped order's
    definition, for full and short last bands and bands taller than the grid."""
    import dense_tiled_gemm_f16_amd as g
    for tm, tn, gm in ((32, 32, 8), (15, 17, 3), (9, 9, 3), (7, 5, 1), (33, 7, 4), (5, 9, 8), (1, 40, 4),
                       (40, 1, 16), (17, 17, 17)):
        rc, pm, pn = g.gemm_f16_f32_tile_order(tm, tn, gm, 0)
        assert rc == 0
        assert (pm, pn) == model.tile_order(tm, tn, None if gm == 1 else gm)


def test_dram_wave_model_h100_times(golden):
    """04_tensor_cores.py demo 3: 4096^3 FP16 on H100 (132 SMs, one tile per SM, 3.35 TB/s): about
    340 / 100 / 60 us of DRAM time for 64x64 / 128x128 / 128x256 tiles (rounded on the page)."""
    g = golden["page_launch_counts"]["dram_time_h100_4096"]
    for (bm, bn), key in (((64, 64), "64x64"), ((128, 128), "128x128"), ((128, 256), "128x256")):
        us = model.dram_bytes_tiled(4096, bm, bn, 1, 132, elem=2) / 3.35e12 * 1e6
        assert abs(us - g["approx_us"][key]) <= 0.1 * g["approx_us"][key], (key, us)
    assert abs(2 * 4096 ** 3 / 989e12 * 1e6 - g["compute_us_at_989TF"]) <= 0.02 * g["compute_us_at_989TF"]


def test_dram_wave_model_grouped_order_ratios(golden):
    """06_triton_style.py demo 2: relative to row-major order, 128x128 tiles with GROUP_M = 8 read
    69-77% of the DRAM bytes, 128x256 tiles with GROUP_M = 16 read 87-89%, and GROUP_M = 4 can read
    more than row-major (A100 108 SMs and H100 132 SMs, 4096^3 FP16)."""
    g = golden["page_launch_counts"]["grouped_order_traffic_4096"]
    r8, r16, r4 = [], [], []
    for sms in (108, 132):
        base = model.dram_bytes_tiled(4096, 128, 128, 1, sms, elem=2)
        r8.append(100 * model.dram_bytes_tiled(4096, 128, 128, 1, sms, elem=2, group=8) / base)
        base2 = model.dram_bytes_tiled(4096, 128, 256, 1, sms, elem=2)
        r16.append(100 * model.dram_bytes_tiled(4096, 128, 256, 1, sms, elem=2, group=16) / base2)
        for bm, bn in ((128, 128), (128, 256)):
            b = model.dram_bytes_tiled(4096, bm, bn, 1, sms, elem=2)
            r4.append(100 * model.dram_bytes_tiled(4096, bm, bn, 1, sms, elem=2, group=4) / b)
    lo, hi = g["tile_128x128_group_8_pct_range"]
    assert all(lo - 0.5 <= x <= hi + 0.5 for x in r8), r8
    assert round(min(r8)) == lo and round(max(r8)) == hi
    lo, hi = g["tile_128x256_group_16_pct_range"]
    assert all(lo - 0.5 <= x <= hi + 0.5 for x in r16), r16
    assert g["group_4_can_exceed_row_major"] == (max(r4) > 100)


def test_l2_bytes_formula_page_512():
    """06_triton_style.py demo 1: at 512^3 in FP32 the block sizes 16x16 .. 128x256 give from 4 to
    about 43 FLOP per byte read (2MNK / ((MKN/BN + KNM/BM) x 4))."""
    f = 2 * 512 ** 3
    assert f / model.l2_bytes(512, 512, 512, 16, 16, elem=4) == 4
    assert round(f / model.l2_bytes(512, 512, 512, 128, 256, elem=4)) == 43
    # the same tiles in FP16 give twice the intensity; 256x256 gives 128 FLOP/byte
    assert f / model.l2_bytes(512, 512, 512, 256, 256, elem=2) == 128
