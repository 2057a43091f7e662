"""Pins of the oracle's fused linear (per-token e4m3 quant of bf16 activations,
then the MXFP4 GEMM) against what the arithmetic fixes, independently of how
the oracle composes it: a one-hot token, exact power-of-two rescaling, a zero
token, and lossless tokens against a plain dequantize-then-matmul."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _bf16_bits(a):
    """fp64 values exactly representable in bf16 -> bf16 bit patterns."""
    f = np.asarray(a, np.float32)
    bits = f.view(np.uint32)
    assert (bits & 0xFFFF == 0).all(), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _weights(N, K, seed):
    g = np.random.default_rng(seed)
    wp = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    we = g.integers(118, 136, (N, K // 32), dtype=np.uint8)
    return wp, we


def test_one_hot_token():
    # x = v e_k with v = 448 * 2^j: the token scale is 2^j exactly, the code is
    # e4m3(+-448) = +-448, so out[n] = v * w[n, k] with no rounding anywhere
    N, K = 24, 256
    wp, we = _weights(N, K, 1)
    wd = oracle.dequant_mxfp4(wp, we)
    for j, k, sign in [(0, 0, 1), (-5, 77, -1), (3, 255, 1)]:
        x = np.zeros((1, K))
        x[0, k] = sign * 448.0 * 2.0 ** j
        out = oracle.linear_bf16(_bf16_bits(x), wp, we)
        assert np.array_equal(out[0], x[0, k] * wd[:, k]), (j, k)


def test_power_of_two_rescaling():
    # scaling a token by 2^j (exact in bf16 and far from its range limits)
    # scales its token scale by 2^j and leaves the codes alone
    N, K = 40, 384
    wp, we = _weights(N, K, 2)
    g = np.random.default_rng(3)
    x = np.round(g.normal(size=(3, K)) * 64) / 64
    base = oracle.linear_bf16(_bf16_bits(x), wp, we)
    for j in (-7, 4):
        out = oracle.linear_bf16(_bf16_bits(x * 2.0 ** j), wp, we)
        assert np.array_equal(out, base * 2.0 ** j), j


def test_zero_token_rows():
    N, K = 16, 128
    wp, we = _weights(N, K, 4)
    x = np.zeros((2, K))
    x[1, 5] = 3.0
    out = oracle.linear_bf16(_bf16_bits(x), wp, we)
    assert (out[0] == 0).all() and (out[1] != 0).any()


def test_lossless_tokens_match_dequantized_matmul():
    # tokens whose values are s * (e4m3 grid values) with row amax exactly
    # 448 s quantize without loss: the fused linear is then x @ W^T for the
    # dequantized weight, exactly (every product and partial sum of these
    # small integers times powers of two is exact in fp64)
    N, K = 33, 512
    wp, we = _weights(N, K, 5)
    wd = oracle.dequant_mxfp4(wp, we)
    g = np.random.default_rng(6)
    grid = np.array([oracle.e4m3_value(b) for b in range(0x7F)])   # non-negative finite e4m3
    grid = grid[grid <= 448]
    rows = []
    for m, j in enumerate((-3, 0, 2)):
        v = g.choice(grid[grid >= 2.0 ** -3], size=K) * g.choice([-1.0, 1.0], size=K)
        v[g.integers(0, K)] = 448.0 * (1 if m % 2 == 0 else -1)
        rows.append(v * 2.0 ** j)
    x = np.array(rows)
    out = oracle.linear_bf16(_bf16_bits(x), wp, we)
    assert np.array_equal(out, x @ wd.T)


def test_sampled_outputs_match_full():
    N, K = 50, 256
    wp, we = _weights(N, K, 7)
    g = np.random.default_rng(8)
    x = np.round(g.normal(size=(4, K)) * 16) / 16
    bits = _bf16_bits(x)
    full = oracle.linear_bf16(bits, wp, we)
    mi = g.integers(0, 4, 30)
    ni = g.integers(0, N, 30)
    assert np.array_equal(oracle.linear_bf16(bits, wp, we, mi=mi, ni=ni), full[mi, ni])
