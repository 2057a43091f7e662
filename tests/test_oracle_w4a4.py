"""Pins for the oracle's W4A4 (MXFP4 activations x MXFP4 weights) reference.

Page: "vllm-radiance (MXFP4)" -- the Quark MXFP4 checkpoints declare MXFP4
weights AND activations (group 32, e8m0 scales); the W4A8 kernel departs from
that.  The activation quantizer is not printed on the pages; the reading taken
is the OCP MX rule, the page's "ocp" exponent (floor(log2 amax) - 2) with
nearest-even e2m1 codes saturating at 6.

Independent checks: equality with the (separately pinned) W4A8 reference when
a token's blocks share one exponent (e2m1 values are exact in e4m3); a one-hot
closed form; agreement with a dequantize-then-fp64-matmul computation; the
activation quantizer's blocks land in the OCP range [4, 8) and every code is a
nearest grid point (brute force).
"""
import numpy as np
import torch

GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _codes(g, rows, K):
    return g.integers(0, 16, (rows, K)).astype(np.uint8)


def _pack(c):
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _value(c):
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def test_w4a4_equals_w4a8_when_blocks_share_an_exponent(orc):
    g = np.random.default_rng(31)
    M, N, K = 5, 7, 256
    xc = _codes(g, M, K)
    ex_row = g.integers(110, 140, M).astype(np.uint8)
    xe = np.repeat(ex_row[:, None], K // 32, axis=1)
    wc = _codes(g, N, K)
    we = g.integers(100, 150, (N, K // 32)).astype(np.uint8)
    # the same activations as e4m3 codes with one fp32 token scale
    x8 = torch.from_numpy(_value(xc).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    xs = np.exp2(ex_row.astype(np.float64) - 127).astype(np.float32)
    a = orc.w4a4_gemm(_pack(xc), xe, _pack(wc), we)
    b = orc.mxfp4_gemm(x8, xs, _pack(wc), we)
    assert np.array_equal(a, b)


def test_w4a4_one_hot(orc):
    M, N, K = 2, 3, 96
    xc = np.zeros((M, K), np.uint8)
    wc = np.zeros((N, K), np.uint8)
    xc[1, 70] = 0xD           # -3
    wc[2, 70] = 0x7           # 6
    xe = np.full((M, K // 32), 127, np.uint8)
    we = np.full((N, K // 32), 127, np.uint8)
    xe[1, 2] = 130            # 2^3
    we[2, 2] = 120            # 2^-7
    out = orc.w4a4_gemm(_pack(xc), xe, _pack(wc), we)
    want = np.zeros((M, N))
    want[1, 2] = -3 * 6 * 2.0 ** (3 - 7)
    assert np.array_equal(out, want)


def test_w4a4_matches_dequantized_matmul(orc):
    g = np.random.default_rng(32)
    M, N, K = 9, 11, 320
    xp, wp = _pack(_codes(g, M, K)), _pack(_codes(g, N, K))
    xe = g.integers(90, 160, (M, K // 32)).astype(np.uint8)
    we = g.integers(90, 160, (N, K // 32)).astype(np.uint8)
    ref = orc.dequant_mxfp4(xp, xe).astype(np.float64) @ orc.dequant_mxfp4(wp, we).astype(np.float64).T
    out = orc.w4a4_gemm(xp, xe, wp, we)
    assert np.allclose(out, ref, rtol=1e-12, atol=0)
    mi, ni = g.integers(0, M, 40), g.integers(0, N, 40)
    assert np.array_equal(orc.w4a4_gemm(xp, xe, wp, we, mi=mi, ni=ni), out[mi, ni])


def test_act_quant_is_the_ocp_rule(orc):
    g = np.random.default_rng(33)
    x = (g.standard_normal((16, 256)) * np.exp2(g.integers(-8, 8, (16, 1)))).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    p, e = orc.quant_act_mxfp4(bits)
    d = orc.dequant_mxfp4(p, e).astype(np.float64)
    for r in range(16):
        for b in range(256 // 32):
            blk = xb[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            s = 2.0 ** (int(e[r, b]) - 127)
            assert 4 <= amax / s < 8                      # floor(log2 amax) - 2
            cand = np.sign(blk)[:, None] * GRID[None, :] * s
            best = np.abs(cand - blk[:, None]).min(1)
            assert np.array_equal(np.abs(d[r, 32 * b:32 * b + 32] - blk), best)
