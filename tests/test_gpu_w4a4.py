"""GPU parity: W4A4 (MXFP4 activations x prepared MXFP4 weights) against the
oracle.  The activation quantizer (OCP rule) is a bit-exact contract; the GEMM
is a tolerance contract on bf16 outputs against the exact fp64 result."""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_bf16, dev_u8, host, host_bf16_as_f64, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _case(name, wp, we, M, seed, spread=1.0, sample=None):
    N, K = wp.shape[0], 2 * wp.shape[1]
    bits = synth.acts(M, K, seed=seed, spread=spread)
    say("w4a4", name, (M, N, K))
    xp, xe = w4.quant_act_mxfp4(dev_bf16(bits))
    rp, re_ = oracle.quant_act_mxfp4(bits)
    assert np.array_equal(host(xp), rp) and np.array_equal(host(xe), re_), name
    pw = w4.mxfp4_prepare(dev_u8(wp), dev_u8(we))
    got = host_bf16_as_f64(w4.w4a4_gemm_prepared(xp, xe, pw))
    again = host_bf16_as_f64(w4.w4a4_gemm_prepared(xp, xe, pw))
    assert np.array_equal(got, again), name
    if sample is None:
        ref = oracle.w4a4_gemm(rp, re_, wp, we)
        assert_gemm_close(got, ref, name)
    else:
        g = np.random.default_rng(M + N)
        mi = np.concatenate([np.arange(M), g.integers(0, M, sample), np.full(64, M - 1)])
        ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, sample), N - 1 - np.arange(64)])
        ref = oracle.w4a4_gemm(rp, re_, wp, we, mi=mi, ni=ni)
        assert_gemm_close(got[mi, ni], ref, name)


# 128- and 256-row tiles, ragged M and N (N % 4 != 0: scalar stores), K of one
# to many steps, few tiles with K split across workgroups
W4A4 = [(1, 64, 128), (5, 300, 384), (33, 1000, 1152), (100, 520, 4096), (129, 1026, 640),
        (300, 700, 2048), (513, 260, 768), (64, 20000, 512)]


@pytest.mark.parametrize("M,N,K", W4A4)
def test_w4a4_ragged(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 7))
    _case(f"{M}x{N}x{K}", w["w_packed"], w["w_e8m0"], M, (M, K, 7), spread=10.0)


# the split-K decode kernel (M <= 12 on wide layers, <= 32 on narrow ones):
# one and two 16-row activation tiles, ragged N, K ending inside a 4-step
# chunk (partial e8m0 chunk), a long K split across workgroups, and the first
# M past the wide-layer bound (tile kernel)
W4A4_DECODE = [(12, 20000, 640), (13, 20000, 640), (16, 4100, 2560), (17, 36, 4736), (32, 520, 17408),
               (3, 1001, 17408)]


@pytest.mark.parametrize("M,N,K", W4A4_DECODE)
def test_w4a4_decode(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 11))
    _case(f"decode {M}x{N}x{K}", w["w_packed"], w["w_e8m0"], M, (M, K, 11), spread=10.0)


# the spread tiles (wide layers, M <= 64): one to four 16-row activation tiles
# with ragged M, one or two weight tiles per wave, N not a multiple of 8 (row
# stores by the products' lanes) or of 4 (scalar stores), K ending inside a
# 4-step chunk, and an odd number of 4-step chunks, where the last trip of 8
# steps runs past the padded steps (weights of the last padded step repeated,
# activation codes zero): after padding steps (K = 1152) and after a real step
# (K = 512, 1536)
W4A4_SPREAD = [(3, 25001, 640, None), (17, 24602, 896, None), (33, 30000, 2048, None), (64, 65536, 512, None),
               (47, 40000, 5120, 2048), (2, 24576, 1152, None), (40, 24576, 1152, None), (24, 24576, 1536, None),
               (1, 30000, 512, None), (64, 24600, 4608, 2048), (5, 24576, 128, None), (50, 24576, 256, None)]


@pytest.mark.parametrize("M,N,K,sample", W4A4_SPREAD)
def test_w4a4_spread(M, N, K, sample):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 13))
    _case(f"spread {M}x{N}x{K}", w["w_packed"], w["w_e8m0"], M, (M, K, 13), spread=10.0, sample=sample)


@pytest.mark.parametrize("M", [1, 8, 12, 13, 16, 32, 48, 64, 4096])
def test_w4a4_gate_up(gate_up_mx, M):
    _case(f"gate_up M={M}", gate_up_mx[0], gate_up_mx[1], M, (8, M), sample=4096 if M > 64 else None)


@pytest.mark.parametrize("M", [1, 16, 32, 4096])
def test_w4a4_down_proj(M):
    d = synth.down_proj()
    _case(f"down_proj M={M}", d["w_packed"], d["w_e8m0"], M, (9, M), sample=4096 if M > 64 else None)


def test_w4a4_rejects_bad_shapes():
    w = synth.mxfp4_random(64, 256, seed=3)
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    xp = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        w4.w4a4_gemm_prepared(xp, torch.zeros((4, 8), dtype=torch.uint8, device="cuda"), pw)   # K = 128 != 256
