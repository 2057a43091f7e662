"""GPU parity: the linear on bf16 activations (per-token fp8 quantization fused
into the split-K decode kernel where it fits, else quant kernel + GEMM)
against the oracle.  The codes and token scales it writes are a bit-exact
contract (the standalone quantizer's); the output is a tolerance contract
against the exact fp64 result, and bit-identical to the unfused GPU path
(quant kernel, then the GEMM), whose plan the fused kernel keeps."""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_bf16, dev_f16, dev_i32, dev_u8, host, host_bf16_as_f64, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _run(name, bits, pw, unfused, x_view=None, sample=None, ref_fn=None):
    """bits: bf16 bits [M, K] (host); x_view: the device tensor to pass (a
    strided or offset view holding the same values), else a fresh copy."""
    M, K = bits.shape
    say("linear", name, (M, pw.N, K))
    x = dev_bf16(bits) if x_view is None else x_view
    out, x8, xs = unfused["linear"](x, pw)
    again, _, _ = unfused["linear"](x, pw)
    got = host_bf16_as_f64(out)
    assert np.array_equal(got, host_bf16_as_f64(again)), name
    r8, rs = oracle.quant_act_fp8(bits)
    assert np.array_equal(host(x8), r8), name
    assert np.array_equal(host(xs), rs), name
    # the unfused GPU path on the same codes and scales: the same kernel plan,
    # so the same bits
    ref_gpu = host_bf16_as_f64(unfused["gemm"](dev_u8(r8), torch.from_numpy(rs).cuda(), pw))
    assert np.array_equal(got, ref_gpu), name + " vs unfused"
    if sample is None:
        ref = ref_fn(bits)
        assert_gemm_close(got, ref, name)
    else:
        g = np.random.default_rng(M + pw.N)
        mi = np.concatenate([np.arange(M), g.integers(0, M, sample), np.full(64, M - 1)])
        ni = np.concatenate([g.integers(0, pw.N, M), g.integers(0, pw.N, sample), pw.N - 1 - np.arange(64)])
        assert_gemm_close(got[mi, ni], ref_fn(bits, mi, ni), name)
    return got, ref_gpu


MX = {"linear": w4.mxfp4_linear_prepared, "gemm": w4.mxfp4_gemm_prepared}
I4 = {"linear": w4.int4g128_linear_prepared, "gemm": w4.int4g128_gemm_prepared}


def _mx(N, K, seed):
    w = synth.mxfp4_random(N, K, seed=seed)
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    return pw, lambda b, mi=None, ni=None: oracle.linear_bf16(b, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni)


# fused (one launch) for small M with K unsplit; the quant kernel + GEMM
# otherwise (M = 17, long K, M = 40 tiled); ragged N, K of one step to many;
# one token on a wide layer (K a multiple of 1024 up to 8192): fused into the
# spread tiles, ragged N and the longest K
LINEAR = [(1, 64, 128), (1, 300, 640), (2, 1000, 4736), (5, 257, 1024), (8, 520, 2048), (16, 130, 512),
          (17, 600, 1152), (3, 1001, 17408), (40, 700, 384), (1, 20000, 5120), (12, 20000, 640),
          (1, 25001, 1024), (1, 30000, 8192)]


@pytest.mark.parametrize("M,N,K", LINEAR)
def test_mxfp4_linear_ragged(M, N, K):
    pw, ref = _mx(N, K, (M, N, K, 21))
    bits = synth.acts(M, K, seed=(M, K, 21), spread=10.0)
    _run(f"{M}x{N}x{K}", bits, pw, MX, ref_fn=ref)


def test_mxfp4_linear_special_rows():
    # a zero token (scale 1, all codes 0), a token with one huge value, a
    # token of one repeated value, tiny values
    N, K = 96, 640
    pw, ref = _mx(N, K, 22)
    x = np.zeros((4, K), np.float32)
    x[1, 7] = 1.0e30
    x[1, 100:110] = -1.0
    x[2, :] = -0.375
    x[3, ::3] = 1.0e-30
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    _run("special rows", bits, pw, MX, ref_fn=ref)


def test_mxfp4_linear_special_token_wide():
    # one token on a wide layer (the spread tiles with the quantization fused):
    # a zero token (scale 1, codes 0), then one huge value among small ones
    N, K = 24576, 2048
    pw, ref = _mx(N, K, 26)
    for i, x in enumerate((np.zeros((1, K), np.float32), np.full((1, K), 1.0e-3, np.float32))):
        if i == 1:
            x[0, 5] = -1.0e30
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        _run(f"special token {i}", bits, pw, MX, ref_fn=ref, sample=4096)


def test_mxfp4_linear_strided_and_unaligned_rows():
    N, K = 300, 1024
    pw, ref = _mx(N, K, 23)
    bits = synth.acts(4, K, seed=24, spread=4.0)
    # rows 1040 elements apart (16-byte multiple): fused
    big = np.zeros((4, 1040), np.uint16)
    big[:, :K] = bits
    xb = dev_bf16(big)[:, :K]
    _run("strided", bits, pw, MX, x_view=xb, ref_fn=ref)
    # rows 1027 elements apart, and a start 2 bytes past alignment: the quant
    # kernel + GEMM
    odd = np.zeros((4, 1027 + 1), np.uint16)
    odd[:, 1:K + 1] = bits
    xo = dev_bf16(odd)[:, 1:K + 1]
    _run("unaligned", bits, pw, MX, x_view=xo, ref_fn=ref)


class _NoWorkspace:
    """A workspace argument of no bytes: the linear's codes stay row-major."""

    def args(self):
        return None, 0


# more than 16 rows on a wide layer: the quant kernel also writes the codes
# step-major into the workspace and the spread tiles stage from that copy;
# without room in the workspace the same call reads the row-major codes.
# Ragged N, K of 5 steps (no e8m0 chunk slots), 9 and 16; both outputs the
# GEMM's on the written codes bit for bit (M = 3: the row-major path both times)
@pytest.mark.parametrize("M,N,K", [(3, 25001, 640), (17, 25001, 640), (33, 24600, 2048), (64, 30000, 1152)])
def test_mxfp4_linear_wide_step_major(M, N, K):
    pw, ref = _mx(N, K, (M, N, K, 28))
    bits = synth.acts(M, K, seed=(M, K, 28), spread=10.0)
    got, ref_gpu = _run(f"wide {M}x{N}x{K}", bits, pw, MX, ref_fn=ref, sample=4096)
    out, _, _ = w4.mxfp4_linear_prepared(dev_bf16(bits), pw, workspace=_NoWorkspace())
    assert np.array_equal(host_bf16_as_f64(out), ref_gpu), "row-major codes"


@pytest.fixture(scope="module")
def gate_up_pw(gate_up_mx):
    return w4.mxfp4_prepare(dev_u8(gate_up_mx[0]), dev_u8(gate_up_mx[1]))


# the headline decode step's four calls (M = 1, 8, 16, 64) and M = 2: every
# output against the oracle
@pytest.mark.parametrize("M", [1, 2, 8, 16, 64])
def test_mxfp4_linear_gate_up(gate_up_mx, gate_up_pw, M):
    wp, we = gate_up_mx[:2]
    bits = synth.acts(M, synth.HIDDEN, seed=(25, M), spread=10.0)
    _run(f"gate_up M={M}", bits, gate_up_pw, MX,
         ref_fn=lambda b, mi=None, ni=None: oracle.linear_bf16(b, wp, we, mi=mi, ni=ni))


@pytest.mark.parametrize("M", [1, 16, 64])
def test_mxfp4_linear_down_proj(M):
    d = synth.down_proj()
    pw = w4.mxfp4_prepare(dev_u8(d["w_packed"]), dev_u8(d["w_e8m0"]))
    bits = synth.acts(M, synth.INTERMEDIATE, seed=(26, M), spread=10.0)
    _run(f"down_proj M={M}", bits, pw, MX,
         ref_fn=lambda b, mi=None, ni=None: oracle.linear_bf16(b, d["w_packed"], d["w_e8m0"], mi=mi, ni=ni))


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (4, 136, 1152), (9, 520, 2048), (24, 200, 640)])
def test_int4_linear(M, N, K):
    q = synth.int4_random(N, K, seed=(M, N, K, 27))
    ref_nk, bad = oracle.int4_prepare(q["qweight_kn"], q["qzeros"], N, K)
    assert bad == 0
    pw = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))

    def ref(b):
        x8, s = oracle.quant_act_fp8(b)
        return oracle.int4_gemm(x8, s, ref_nk, q["scales"])
    bits = synth.acts(M, K, seed=(M, K, 27), spread=10.0)
    _run(f"int4 {M}x{N}x{K}", bits, pw, I4, ref_fn=ref)
