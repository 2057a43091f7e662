"""Pins of the oracle's asymmetric int4 g128 GEMM (zero point per group and
column, stored minus one) against what the definition fixes, independently of
how the oracle computes it: the symmetric case against the symmetric
reference, a one-hot activation, invariance under shifting a group's codes and
zero together, and a plain fp64 dequantize-then-matmul."""
import numpy as np

import oracle
from w4a8_gemm_amd import synth


def _acts(M, K, seed):
    g = np.random.default_rng(seed)
    x8 = g.integers(0, 256, (M, K), dtype=np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x38                       # no NaN codes
    s = g.uniform(0.5, 2.0, M).astype(np.float32)
    return x8, s


def _codes(qw_kn):
    """[K/8, N] int32 -> codes [N, K]"""
    w = qw_kn.view(np.uint32)
    K8, N = w.shape
    c = np.stack([(w >> (4 * j)) & 15 for j in range(8)], axis=1)       # [K/8, 8, N]
    return c.reshape(K8 * 8, N).T.astype(np.int64)


def _zeros(qz, N):
    """[K/128, N/8] int32 -> z [K/128, N] (stored + 1)"""
    w = qz.view(np.uint32)
    z = np.stack([(w >> (4 * j)) & 15 for j in range(8)], axis=2)       # [G, N/8, 8]
    return z.reshape(w.shape[0], N).astype(np.int64) + 1


def _f16(bits):
    return bits.view(np.float16).astype(np.float64)


def test_uniform_zeros_equal_symmetric():
    q = synth.int4_random(64, 384, seed=31)
    x8, s = _acts(3, 384, 32)
    nk, bad = oracle.int4_prepare(q["qweight_kn"], q["qzeros"], 64, 384)
    assert bad == 0
    ref = oracle.int4_gemm(x8, s, nk, q["scales"])
    assert np.array_equal(oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"]), ref)


def test_one_hot_activation():
    N, K = 40, 256
    q = synth.int4_zp(N, K, seed=33)
    c, z, sc = _codes(q["qweight_kn"]), _zeros(q["qzeros"], N), _f16(q["scales"])
    for k, code, val in [(0, 0x38, 1.0), (129, 0xD0, -8.0), (255, 0x7E, 448.0)]:
        x8 = np.zeros((1, K), np.uint8)
        x8[0, k] = code
        out = oracle.int4_zp_gemm(x8, np.ones(1, np.float32), q["qweight_kn"], q["qzeros"], q["scales"])
        want = val * (c[:, k] - z[k // 128]) * sc[k // 128]
        assert np.array_equal(out[0], want), k


def _pack(c, z):
    """codes [N, K], zero points [K/128, N] -> (qweight [K/8, N], qzeros [K/128, N/8]) int32"""
    N, K = c.shape
    qw = np.zeros((K // 8, N), np.uint32)
    ck = c.T.reshape(K // 8, 8, N)
    for j in range(8):
        qw |= ck[:, j, :].astype(np.uint32) << (4 * j)
    qz = np.zeros((K // 128, N // 8), np.uint32)
    zz = (z - 1).reshape(K // 128, N // 8, 8)
    for j in range(8):
        qz |= zz[:, :, j].astype(np.uint32) << (4 * j)
    return qw.view(np.int32), qz.view(np.int32)


def test_shifting_codes_and_zero_together():
    # (c + 1) - (z + 1) = c - z: group 1's codes limited to 0..14 and zeros to
    # 1..15, then every code and zero of that group raised by one
    N, K = 32, 256
    q = synth.int4_zp(N, K, seed=34)
    c, z = _codes(q["qweight_kn"]), _zeros(q["qzeros"], N)
    c[:, 128:] = np.minimum(c[:, 128:], 14)
    z[1] = np.minimum(z[1], 15)
    x8, s = _acts(2, K, 35)
    qw, qz = _pack(c, z)
    assert np.array_equal(_codes(qw), c) and np.array_equal(_zeros(qz, N), z)
    base = oracle.int4_zp_gemm(x8, s, qw, qz, q["scales"])
    c[:, 128:] += 1
    z[1] += 1
    qw, qz = _pack(c, z)
    assert np.array_equal(oracle.int4_zp_gemm(x8, s, qw, qz, q["scales"]), base)
    # and a planted error (one zero moved alone) shows
    z[1, 3] -= 1
    qw, qz = _pack(c, z)
    assert not np.array_equal(oracle.int4_zp_gemm(x8, s, qw, qz, q["scales"]), base)


def test_matches_dequantized_matmul():
    N, K = 48, 512
    q = synth.int4_zp(N, K, seed=36)
    c, z, sc = _codes(q["qweight_kn"]), _zeros(q["qzeros"], N), _f16(q["scales"])
    w = (c - np.repeat(z.T, 128, axis=1)) * np.repeat(sc.T, 128, axis=1)     # [N, K]
    x8, s = _acts(4, K, 37)
    xv = np.vectorize(oracle.e4m3_value)(x8).astype(np.float64)
    want = s.astype(np.float64)[:, None] * (xv @ w.T)
    got = oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_sampled_outputs_match_full():
    N, K = 24, 256
    q = synth.int4_zp(N, K, seed=38)
    x8, s = _acts(5, K, 39)
    full = oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"])
    g = np.random.default_rng(40)
    mi, ni = g.integers(0, 5, 25), g.integers(0, N, 25)
    got = oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"], mi=mi, ni=ni)
    assert np.array_equal(got, full[mi, ni])
