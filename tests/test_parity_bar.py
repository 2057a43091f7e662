"""The GEMM parity bar itself (host only): correctly rounded bf16 outputs pass
at any output count, an output two bf16 ulps off fails, a systematic bias over
many outputs fails the rel_F part."""
import numpy as np
import pytest
import torch

from gpu_util import GEMM_REL_F_MIN_OUTPUTS, assert_gemm_close


def _bf16(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("n", [64, 4096])
def test_correctly_rounded_passes(n):
    for seed in range(20):
        ref = np.random.default_rng(seed).standard_normal(n)
        assert_gemm_close(_bf16(ref), ref)


def test_two_ulps_off_fails():
    ref = np.random.default_rng(1).standard_normal(64)
    got = _bf16(ref)
    i = int(np.argmax(np.abs(ref)))
    ulp = 2.0 ** (np.floor(np.log2(abs(got[i]))) - 7)
    got[i] += np.sign(got[i]) * 2 * ulp          # >= 1.5 ulp from the exact value
    with pytest.raises(AssertionError):
        assert_gemm_close(got, ref)


def test_bias_fails_rel_f():
    # every output 2^-8 relative high: inside the per-element bound (the
    # rounding half-ulp), but rel_F ~ 3.9e-3 over many outputs
    n = 4 * GEMM_REL_F_MIN_OUTPUTS
    ref = np.random.default_rng(2).standard_normal(n)
    got = ref * (1 + 2.0 ** -8)
    with pytest.raises(AssertionError):
        assert_gemm_close(got, ref)
