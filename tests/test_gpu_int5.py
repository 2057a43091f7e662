"""GPU parity: int5 g128 (W5A8) against the oracle, on the split-K decode
kernel (M <= 32) and the tile kernel (M > 32: 64-, 128- and 256-row tiles,
K split across workgroups when the tiles are few)."""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_f16, dev_f32, dev_i32, dev_u8, host_bf16_as_f64, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _prep(q):
    return w4.int5g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qweight_hi"]), dev_u8(q["qzeros"]),
                                         dev_f16(q["scales"]))


def _case(name, q, M, seed, sample=None, spread=10.0):
    N, K = q["N"], q["K"]
    say("int5", name, (M, N, K))
    pw = _prep(q)
    x8, s = oracle.quant_act_fp8(synth.acts(M, K, seed=seed, spread=spread))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.int5g128_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, host_bf16_as_f64(w4.int5g128_gemm_prepared(dx, ds, pw))), name
    args = (x8, s, q["qweight_kn"], q["qweight_hi"], q["qzeros"], q["scales"])
    if sample is None:
        assert_gemm_close(got, oracle.int5_gemm(*args), name)
    else:
        g = np.random.default_rng(M + N)
        mi = np.concatenate([np.arange(M), g.integers(0, M, sample), np.full(64, M - 1)])
        ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, sample), N - 1 - np.arange(64)])
        assert_gemm_close(got[mi, ni], oracle.int5_gemm(*args, mi=mi, ni=ni), name)
    return got


# decode: one and two activation tiles, K split across workgroups, ragged N
# (not a multiple of 16 or 4), K ending inside a 4-step chunk; tiles: 64 rows
# (M 33..64), 128 rows (65..128) and 256 rows, each with and without a K
# split, ragged M, N and chunks
INT5 = [(1, 64, 128), (3, 130, 640), (16, 200, 1152), (17, 1000, 4096), (32, 522, 17408), (5, 20000, 512),
        (33, 96, 384), (40, 300, 4096), (64, 20000, 512), (70, 300, 1024), (100, 1000, 17408),
        (129, 1000, 2176), (300, 520, 1152), (513, 4100, 640)]


@pytest.mark.parametrize("M,N,K", INT5)
def test_int5_ragged(M, N, K):
    _case(f"{M}x{N}x{K}", synth.int5(N, K, seed=(M, N, K, 61)), M, (M, K, 61))


# the spread tiles (wide layers, 9 <= M <= 64): one to four activation tiles,
# one or two weight tiles per wave, odd chunk counts (the last trip past the
# padded steps: after padding steps, K = 1152, and after a real step, K = 1536)
INT5_SPREAD = [(9, 24576, 640, None), (33, 30000, 2048, None), (64, 65536, 512, None), (40, 24576, 1152, None),
               (24, 24576, 1536, None), (64, 24600, 4608, 4096), (17, 24602, 896, None), (12, 24576, 128, None)]


@pytest.mark.parametrize("M,N,K,sample", INT5_SPREAD)
def test_int5_spread(M, N, K, sample):
    _case(f"spread {M}x{N}x{K}", synth.int5(N, K, seed=(M, N, K, 65)), M, (M, K, 65), sample=sample)


@pytest.mark.parametrize("M", [1, 16, 64, 2048])
def test_int5_full_size(M):
    _case(f"int5 M={M}", synth.int5(), M, (62, M), sample=4096 if M > 64 else None)


@pytest.mark.parametrize("M", [8, 200])
def test_int5_symmetric(M):
    q = synth.int5(520, 2048, seed=63, symmetric=True)
    _case(f"symmetric M={M}", q, M, 64)


def _transposed(h):
    # bit pair (8 i + 2 q, +1) of a checkpoint word -> bits (8 q + 2 i, +1)
    o = np.zeros_like(h)
    for i in range(4):
        for q in range(4):
            o |= ((h >> np.uint32(8 * i + 2 * q)) & np.uint32(3)) << np.uint32(8 * q + 2 * i)
    return o


def test_int5_prepared_planes():
    N, K = 20, 640
    q = synth.int5(N, K, seed=65)
    pw = _prep(q)
    s_pad = 4 * ((K // 128 + 3) // 4)
    w5 = pw.w5.cpu().numpy().view(np.uint32).reshape(2, s_pad // 4, 64, 4)     # tile, chunk, lane, step
    hi = _transposed(q["qweight_hi"].view(np.uint32))
    for t in range(2):
        for s_ in range(s_pad):
            for L in range(64):
                row, g = 16 * t + (L & 15), L >> 4
                want = hi[4 * s_ + g, row] if row < N and s_ < K // 128 else 0
                assert w5[t, s_ // 4, L, s_ % 4] == want
    st = pw.s.cpu().numpy()
    c_pad = s_pad // 4
    for t in range(2):
        for c in range(c_pad):
            rec = st[(t * c_pad + c) * 256:(t * c_pad + c + 1) * 256]
            zb = rec[128:192].view(np.int8).reshape(4, 4, 4).transpose(1, 0, 2).reshape(4, 16)   # [step][row]
            for u in range(4):
                for r in range(16):
                    n, s_ = 16 * t + r, 4 * c + u
                    want = 15 - int(q["qzeros"][s_, n]) if n < N and s_ < K // 128 else 0
                    assert zb[u, r] == want
