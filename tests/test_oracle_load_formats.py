"""Pins for the oracle's bf16 and fp8-per-channel -> MXFP4 load-time encoders
(CPU only).

Page: "radiance_nvfp4.py" -- RadianceBf16ToMxfp4.process_weights_after_loading
(requant_rows on the bf16 weight) and RadianceFp8ChannelToMxfp4
.process_weights_after_loading (the e4m3 weight widened to fp32 times its
row's fp32 scale, then quant_mxfp4).

Independent checks: blocks on the MXFP4 grid round-trip losslessly from bf16
under every rule; fp8 with unit scales agrees bit for bit with bf16 holding the
same values (torch's exact casts); per-row power-of-two scales leave the codes
alone and move each row's exponents by exactly that power (a wrong row, a
division instead of a product or a column index would not); the statistics
recomputed from decoded outputs; bad inputs rejected.
"""
import numpy as np
import pytest
import torch


def _bf16_bits(a_f32):
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _grid_blocks(g, rows, K):
    """fp32 values on the MXFP4 grid: random codes times 2^e per 32-block."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    idx = g.integers(0, 8, (rows, K))
    sgn = np.where(g.integers(0, 2, (rows, K)) == 1, -1.0, 1.0).astype(np.float32)
    e = g.integers(-20, 12, (rows, K // 32)).astype(np.float32)
    return grid[idx] * sgn * np.repeat(np.exp2(e), 32, axis=1)


def _e4m3_codes(g, rows, K):
    c = g.integers(0, 256, (rows, K)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E            # no NaN codes
    return c


def _e4m3_as_f32(c):
    return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_bf16_grid_blocks_round_trip_losslessly(orc):
    g = np.random.default_rng(11)
    w = _grid_blocks(g, 24, 256)
    bits = _bf16_bits(w)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), w)
    for mode in ("ocp", "noclip", "mse"):
        mp, me, st = orc.quant_bf16_to_mxfp4(bits, mode)
        assert np.array_equal(orc.dequant_mxfp4(mp, me), w), mode
        assert st[0] == 0.0 and abs(st[1] - (w.astype(np.float64) ** 2).sum()) <= 1e-12 * st[1]


def test_fp8_unit_scale_matches_bf16_path(orc):
    g = np.random.default_rng(12)
    c = _e4m3_codes(g, 40, 512)
    v = _e4m3_as_f32(c)                       # every e4m3 value is exact in bf16
    for mode in ("ocp", "noclip", "mse"):
        a = orc.quant_fp8ch_to_mxfp4(c, np.ones(40, np.float32), mode)
        b = orc.quant_bf16_to_mxfp4(_bf16_bits(v), mode)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), mode
        assert np.allclose(a[2], b[2], rtol=1e-12)


def test_fp8_power_of_two_row_scales_move_exponents_only(orc):
    g = np.random.default_rng(13)
    rows, K = 48, 384
    c = _e4m3_codes(g, rows, K)
    p = g.integers(-6, 7, rows)
    base = orc.quant_fp8ch_to_mxfp4(c, np.ones(rows, np.float32), "mse")
    out = orc.quant_fp8ch_to_mxfp4(c, np.exp2(p).astype(np.float32), "mse")
    assert np.array_equal(out[0], base[0])
    nz = base[0].reshape(rows, -1, 16).any(-1)            # blocks that are not all zero
    shift = out[1].astype(int) - base[1].astype(int)
    assert np.array_equal(shift[nz], np.broadcast_to(p[:, None], shift.shape)[nz])
    # the sums scale row by row with 4^p: check the total of squares directly
    w = _e4m3_as_f32(c).astype(np.float64) * np.exp2(p)[:, None]
    assert abs(out[2][1] - (w ** 2).sum()) <= 1e-12 * out[2][1]


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_load_stats_match_decoded_error(orc, kind):
    g = np.random.default_rng(14)
    rows, K = 32, 256
    for mode in ("ocp", "noclip", "mse"):
        if kind == "bf16":
            bits = _bf16_bits(g.standard_normal((rows, K)).astype(np.float32) * 0.02)
            w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
            mp, me, st = orc.quant_bf16_to_mxfp4(bits, mode)
        else:
            c = _e4m3_codes(g, rows, K)
            s = (g.random(rows) * 0.01 + 1e-4).astype(np.float32)
            w = (_e4m3_as_f32(c) * s[:, None]).astype(np.float64)   # one fp32 product each
            mp, me, st = orc.quant_fp8ch_to_mxfp4(c, s, mode)
        d = orc.dequant_mxfp4(mp, me).astype(np.float64)
        err = ((d - w) ** 2).sum()
        assert abs(st[0] - err) <= 1e-5 * err, (kind, mode)
        assert abs(st[1] - (w ** 2).sum()) <= 1e-9 * st[1], (kind, mode)


def test_load_encoders_reject_bad_inputs(orc):
    with pytest.raises(ValueError):
        orc.quant_bf16_to_mxfp4(np.zeros((2, 48), np.uint16))              # K % 32
    with pytest.raises(ValueError):
        orc.quant_bf16_to_mxfp4(np.full((1, 32), 0x7F80, np.uint16))       # +inf
    c = np.zeros((2, 64), np.uint8)
    c[1, 5] = 0x7F                                                          # NaN code
    with pytest.raises(ValueError):
        orc.quant_fp8ch_to_mxfp4(c, np.ones(2, np.float32))
    with pytest.raises(ValueError):
        orc.quant_fp8ch_to_mxfp4(np.zeros((2, 64), np.uint8), np.array([1.0, np.inf], np.float32))
