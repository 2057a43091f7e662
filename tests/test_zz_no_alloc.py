"""GPU: the prepared MXFP4 GEMM that allocates nothing
(w4a8_mxfp4_gemm_prepared_noalloc: split-K partials in the library's static
device array) against the entry point that takes a workspace, through the C
ABI.  Two calls in a row on the down_proj shape, both splitting K (the 64-row
tiles at M = 64, the register-streamed tiles at M = 16), the second smaller:
outputs bit-identical to the workspace entry point's, and within the GEMM bar
of the oracle on sampled outputs.  A call whose partials exceed the array is
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_f32, dev_u8, host_bf16_as_f64, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu

N, K = synth.HIDDEN, synth.INTERMEDIATE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _call(L, dx, ds, pw, out, M):
    v = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.w4a8_mxfp4_gemm_prepared_noalloc(v(dx), v(ds), v(pw.w), v(pw.s), v(out), M, N, K, None)


def test_noalloc_matches_workspace_entry_point():
    L = w4.lib()
    cap = int(L.w4a8_mxfp4_gemm_prepared_noalloc_max_scratch())
    w = synth.mxfp4_random(N, K, seed=91)
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    for M in (64, 16):
        assert 0 < w4.gemm_workspace_bytes(M, N, K, "prepared") <= cap
        x8, s = oracle.quant_act_fp8(synth.acts(M, K, seed=(91, M), spread=10.0))
        dx, ds = dev_u8(x8), dev_f32(s)
        say("noalloc gemm", (M, N, K))
        ref = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert _call(L, dx, ds, pw, out, M) == w4.binding.OK
        got = host_bf16_as_f64(out)
        assert np.array_equal(got, ref), M
        g = np.random.default_rng(M)
        mi = np.concatenate([np.arange(M), g.integers(0, M, 2048)])
        ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, 2048)])
        assert_gemm_close(got[mi, ni], oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni), M)


def test_noalloc_refuses_partials_beyond_the_array():
    # M = 385 on the down_proj shape needs about 23.7 MB of partials; every
    # smaller M fits the 16 MiB array
    L = w4.lib()
    cap = int(L.w4a8_mxfp4_gemm_prepared_noalloc_max_scratch())
    M = 385
    assert w4.gemm_workspace_bytes(M, N, K, "prepared") > cap >= w4.gemm_workspace_bytes(M - 1, N, K, "prepared")
    w = synth.mxfp4_random(N, K, seed=92)
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    x8 = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.ones((M,), dtype=torch.float32, device="cuda")
    out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    say("noalloc refusal", (M, N, K))
    assert _call(L, x8, xs, pw, out, M) == w4.binding.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()
