"""GPU parity: the decode band with explicit plans (w4a8_decode_with_plan, the
entry point for tile sweeps) against the oracle, over the plan space each
weight kind accepts: row-major MXFP4 and transposed int4 (tiles per wave,
K steps per chunk, K splits) and fragment-order MXFP4 (ring depth, K parts per
tile).  Every plan computes the same GEMM; only the summation order moves."""
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


def _acts(M, K, seed):
    return oracle.quant_act_fp8(synth.acts(M, K, seed=seed, spread=10.0))


@pytest.mark.parametrize("M,N,K", [(1, 300, 1152), (5, 1000, 4096), (20, 136, 2048)])
@pytest.mark.parametrize("u", [2, 3, 4])
@pytest.mark.parametrize("ks", [1, 2, 4, 8])
def test_prepared_plans(M, N, K, u, ks):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 71))
    x8, s = _acts(M, K, (M, K, 71))
    say("decode plan prepared", (M, N, K), "depth", u, "parts", ks)
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.decode_with_plan(dev_u8(x8), dev_f32(s), pw.w, pw.s, 0, u, ks, kind="prepared", N=N))
    assert_gemm_close(got, oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"]), f"prepared u={u} ks={ks}")


@pytest.mark.parametrize("M,N,K", [(1, 300, 1152), (7, 520, 4096), (40, 64, 640)])
@pytest.mark.parametrize("rt", [1, 2, 4])
@pytest.mark.parametrize("u", [1, 2, 4])
@pytest.mark.parametrize("ks", [1, 3])
def test_rowmajor_plans(M, N, K, rt, u, ks):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 72))
    x8, s = _acts(M, K, (M, K, 72))
    say("decode plan mxfp4", (M, N, K), rt, u, ks)
    got = host_bf16_as_f64(w4.decode_with_plan(dev_u8(x8), dev_f32(s), dev_u8(w["w_packed"]),
                                               dev_u8(w["w_e8m0"]), rt, u, ks))
    assert_gemm_close(got, oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"]), f"mxfp4 {rt} {u} {ks}")


@pytest.mark.parametrize("M,N,K", [(1, 136, 1152), (9, 1000, 4096)])
@pytest.mark.parametrize("rt", [1, 2, 4])
@pytest.mark.parametrize("u", [1, 2, 4])
@pytest.mark.parametrize("ks", [1, 3])
def test_int4_plans(M, N, K, rt, u, ks):
    q = synth.int4_random(N, K, seed=(M, N, K, 73))
    ref_nk, bad = oracle.int4_prepare(q["qweight_kn"], q["qzeros"], N, K)
    assert bad == 0
    x8, s = _acts(M, K, (M, K, 73))
    say("decode plan int4", (M, N, K), rt, u, ks)
    nk = w4.int4g128_prepare(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]))
    got = host_bf16_as_f64(w4.decode_with_plan(dev_u8(x8), dev_f32(s), nk, dev_f16(q["scales"]), rt, u, ks,
                                               kind="int4"))
    assert_gemm_close(got, oracle.int4_gemm(x8, s, ref_nk, q["scales"]), f"int4 {rt} {u} {ks}")
