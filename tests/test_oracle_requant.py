"""Pins for the oracle's NVFP4 dequant and NVFP4 -> MXFP4 requant (CPU only).

Page: "radiance_nvfp4.py" -- dequant_nvfp4 (W = e2m1 * e4m3 / divisor),
requant_rows (passes of ROW_CHUNK rows, relative RMS error),
RadianceNvfp4ToMxfp4.process_weights_after_loading (each partition of a merged
linear with its own divisor, outputs concatenated in row order).

Independent checks: hand-worked dequant values (golden), lossless round trip
of power-of-two NVFP4 blocks, exact divisor-doubling behaviour, partition and
row-chunk independence, and the statistics recomputed from decoded outputs.
"""
import os

import numpy as np

from w4a8_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def test_dequant_nvfp4_golden(orc):
    for sb, gd, code, expect in _rows("nvfp4_layout.txt"):
        c = int(code)
        packed = np.full((1, 16), c | (c << 4), np.uint8)
        scale = np.full((1, 2), int(sb, 16), np.uint8)
        w = orc.dequant_nvfp4(packed, scale, float(gd))
        assert (w == np.float32(expect)).all(), (sb, gd, code, w[0, :4])


def _e4m3_exact(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


def test_dequant_golden_rows_fix_the_rounding_order():
    """The golden rows separate the page's order (divide the scale by the
    divisor, then multiply by the code) from the two other fp32 orders: an
    oracle that multiplied first, or multiplied by the divisor's reciprocal,
    would fail at least one row of test_dequant_nvfp4_golden."""
    f = np.float32
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    orders = {
        "divide_first": lambda c, s, g: f(f(c) * f(f(s) / f(g))),
        "multiply_first": lambda c, s, g: f(f(f(c) * f(s)) / f(g)),
        "reciprocal": lambda c, s, g: f(f(c) * f(f(s) * f(f(1.0) / f(g)))),
    }
    fails = {k: 0 for k in orders}
    for sb, gd, code, expect in _rows("nvfp4_layout.txt"):
        c = int(code)
        cv = -grid[c & 7] if c & 8 else grid[c & 7]
        for name, fn in orders.items():
            if fn(cv, _e4m3_exact(int(sb, 16)), float(gd)) != np.float32(expect):
                fails[name] += 1
    assert fails["divide_first"] == 0
    assert fails["multiply_first"] >= 1 and fails["reciprocal"] >= 1, fails


def test_dequant_nvfp4_nibble_order_and_scale_index(orc):
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x07 | (0x02 << 4)          # k=0: code 7 (6.0), k=1: code 2 (1.0)
    packed[0, 8] = 0x0B                        # k=16: code 11 (-1.5)
    scale = np.array([[0x38, 0x40]], np.uint8)  # 1.0 for k < 16, 2.0 for k >= 16
    w = orc.dequant_nvfp4(packed, scale, 1.0)
    assert w[0, 0] == 6.0 and w[0, 1] == 1.0 and w[0, 16] == -3.0
    assert np.count_nonzero(w) == 3


def _pow2_nvfp4(g, rows, K):
    """NVFP4 whose e4m3 scale is one power of two per 32-block."""
    codes = g.integers(0, 16, (rows, K))
    e = g.integers(-6, 7, (rows, K // 32))
    sbyte = ((e + 7) << 3).astype(np.uint8)      # e4m3 2^e, normal range
    scale = np.repeat(sbyte, 2, axis=1)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale


def test_power_of_two_blocks_round_trip_losslessly(orc):
    g = np.random.default_rng(5)
    packed, scale = _pow2_nvfp4(g, 32, 256)
    for gd in (1.0, 8.0, 0.25):
        w = orc.dequant_nvfp4(packed, scale, gd)
        for mode in ("ocp", "noclip", "mse"):
            mp, me, st = orc.requant_nvfp4_to_mxfp4(packed, scale, [32], [gd], mode)
            back = orc.dequant_mxfp4(mp, me)
            assert np.array_equal(back, w), (gd, mode)
            assert st[0, 0] == 0.0


def test_divisor_doubling_shifts_exponent_only(orc):
    t = synth.tiny()
    gd = float(t["part_divisor"][0])
    a = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"], [gd], "mse")
    b = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"], [2 * gd], "mse")
    assert np.array_equal(a[0], b[0])
    ea = a[1].astype(int)
    eb = b[1].astype(int)
    nz = a[0].reshape(a[0].shape[0], -1, 16).any(-1)       # blocks that are not all zero
    assert np.array_equal(eb[nz], ea[nz] - 1)
    assert abs(b[2][0, 0] * 4 - a[2][0, 0]) <= 1e-6 * a[2][0, 0]


def test_partitions_are_independent(orc):
    g = np.random.default_rng(6)
    codes = g.integers(0, 16, (96, 128))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scale = g.integers(0x20, 0x50, (96, 8)).astype(np.uint8)
    rows, divs = [40, 56], [3.0, 0.7]
    mp, me, st = orc.requant_nvfp4_to_mxfp4(packed, scale, rows, divs, "mse")
    r0 = 0
    for i, (n, d) in enumerate(zip(rows, divs)):
        p1, e1, s1 = orc.requant_nvfp4_to_mxfp4(packed[r0:r0 + n], scale[r0:r0 + n], [n], [d], "mse")
        assert np.array_equal(mp[r0:r0 + n], p1) and np.array_equal(me[r0:r0 + n], e1)
        assert st[i, 0] == s1[0, 0] and st[i, 1] == s1[0, 1]
        r0 += n
    # a merged layer that used one divisor (the stock scheme's max) differs
    mp2, me2, _ = orc.requant_nvfp4_to_mxfp4(packed, scale, [96], [3.0], "mse")
    assert not np.array_equal(me2[40:], me[40:])


def test_row_chunk_does_not_change_results(orc):
    t = synth.tiny()
    ref = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"], t["part_divisor"], "mse", 0)
    for chunk in (1, 3, 100, 4096):
        out = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"],
                                         t["part_divisor"], "mse", chunk)
        assert np.array_equal(out[0], ref[0]) and np.array_equal(out[1], ref[1])
        assert np.allclose(out[2], ref[2], rtol=1e-12)


def test_stats_match_decoded_error(orc):
    t = synth.tiny()
    for mode in ("ocp", "noclip", "mse"):
        mp, me, st = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"],
                                                t["part_divisor"], mode, 64)
        w = orc.dequant_nvfp4(t["nv_packed"], t["nv_scale"], t["part_divisor"][0]).astype(np.float64)
        d = orc.dequant_mxfp4(mp, me).astype(np.float64)
        err = ((d - w) ** 2).sum()
        assert abs(st[0, 0] - err) <= 1e-5 * err
        assert abs(st[0, 1] - (w ** 2).sum()) <= 1e-9 * st[0, 1]
    # mse never has more error than noclip (it takes the better of noclip and noclip-1)
    e_nc = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"], t["part_divisor"], "noclip")[2][0, 0]
    e_ms = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"], t["part_divisor"], "mse")[2][0, 0]
    assert e_ms <= e_nc


def test_rejects_bad_arguments(orc):
    import pytest
    t = synth.tiny()
    with pytest.raises(ValueError):
        orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], [256], [0.0])
    with pytest.raises(ValueError):
        orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], [256], [float("nan")])
