"""Pins of the oracle's int5 g128 GEMM (low four bits in the int4 word layout,
the fifth bit in a plane of its own, zero points stored minus one) against
what the definition fixes: int4 when every fifth bit is clear, a one-hot
activation, shifting a group's codes and zero together, and a plain fp64
dequantize-then-matmul."""
import numpy as np

import oracle
from w4a8_gemm_amd import synth


def _acts(M, K, seed):
    g = np.random.default_rng(seed)
    x8 = g.integers(0, 256, (M, K), dtype=np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x38
    s = g.uniform(0.5, 2.0, M).astype(np.float32)
    return x8, s


def _codes(q):
    """-> codes [N, K] in 0..31"""
    lo = q["qweight_kn"].view(np.uint32)
    hi = q["qweight_hi"].view(np.uint32)
    K8, N = lo.shape
    c = np.stack([(lo >> (4 * j)) & 15 for j in range(8)], axis=1).reshape(K8 * 8, N)
    b = np.stack([(hi >> j) & 1 for j in range(32)], axis=1).reshape(K8 * 8, N)
    return (c | (b << 4)).T.astype(np.int64)


def _pack(c, zm1, q):
    N, K = c.shape
    lo = np.zeros((K // 8, N), np.uint32)
    hi = np.zeros((K // 32, N), np.uint32)
    ck = c.T
    for j in range(8):
        lo |= (ck.reshape(K // 8, 8, N)[:, j, :] & 15).astype(np.uint32) << (4 * j)
    for j in range(32):
        hi |= ((ck.reshape(K // 32, 32, N)[:, j, :] >> 4) & 1).astype(np.uint32) << j
    return dict(q, qweight_kn=lo.view(np.int32), qweight_hi=hi.view(np.int32), qzeros=zm1.astype(np.uint8))


def _run(q, x8, s, **kw):
    return oracle.int5_gemm(x8, s, q["qweight_kn"], q["qweight_hi"], q["qzeros"], q["scales"], **kw)


def test_fifth_bits_clear_is_int4():
    # codes below 16 and z = 8 (stored 7): the symmetric int4 weight with the same low bits
    N, K = 40, 256
    q = synth.int5(N, K, seed=51)
    c = _codes(q) & 15
    q = _pack(c, np.full((K // 128, N), 7), q)
    x8, s = _acts(3, K, 52)
    qz4 = np.full((K // 128, N // 8), 0x77777777, np.uint32).view(np.int32)
    nk, bad = oracle.int4_prepare(q["qweight_kn"], qz4, N, K)
    assert bad == 0
    assert np.array_equal(_run(q, x8, s), oracle.int4_gemm(x8, s, nk, q["scales"]))


def test_one_hot_activation():
    N, K = 32, 384
    q = synth.int5(N, K, seed=53)
    c = _codes(q)
    z = q["qzeros"].astype(np.int64) + 1
    sc = q["scales"].view(np.float16).astype(np.float64)
    for k, code, val in [(5, 0x38, 1.0), (200, 0xC4, -3.0), (383, 0x7E, 448.0)]:
        x8 = np.zeros((1, K), np.uint8)
        x8[0, k] = code
        out = _run(q, x8, np.ones(1, np.float32))
        assert np.array_equal(out[0], val * (c[:, k] - z[k // 128]) * sc[k // 128]), k


def test_shifting_codes_and_zero_together():
    N, K = 24, 256
    q = synth.int5(N, K, seed=54)
    c, zm1 = _codes(q), q["qzeros"].astype(np.int64)
    c[:, :128] = np.minimum(c[:, :128], 30)
    zm1[0] = np.minimum(zm1[0], 30)
    x8, s = _acts(2, K, 55)
    base = _run(_pack(c, zm1, q), x8, s)
    c[:, :128] += 1
    zm1[0] += 1
    assert np.array_equal(_run(_pack(c, zm1, q), x8, s), base)
    zm1[0, 5] += 1 if zm1[0, 5] < 31 else -1
    assert not np.array_equal(_run(_pack(c, zm1, q), x8, s), base)


def test_matches_dequantized_matmul():
    N, K = 48, 512
    q = synth.int5(N, K, seed=56)
    c = _codes(q)
    z = q["qzeros"].astype(np.int64) + 1
    sc = q["scales"].view(np.float16).astype(np.float64)
    w = (c - np.repeat(z.T, 128, axis=1)) * np.repeat(sc.T, 128, axis=1)
    x8, s = _acts(4, K, 57)
    xv = np.vectorize(oracle.e4m3_value)(x8).astype(np.float64)
    want = s.astype(np.float64)[:, None] * (xv @ w.T)
    got = _run(q, x8, s)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_sampled_outputs_match_full():
    N, K = 16, 256
    q = synth.int5(N, K, seed=58)
    x8, s = _acts(5, K, 59)
    full = _run(q, x8, s)
    g = np.random.default_rng(60)
    mi, ni = g.integers(0, 5, 25), g.integers(0, N, 25)
    assert np.array_equal(_run(q, x8, s, mi=mi, ni=ni), full[mi, ni])
