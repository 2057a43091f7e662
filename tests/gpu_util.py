"""Helpers shared by the GPU parity tests: device upload/download of raw bit
arrays and the GEMM error metric.  No arithmetic of the method lives here."""
import sys

import numpy as np
import torch


def say(*msg):
    """Name the case before a GPU step (flushed, so a lost box still shows it)."""
    print("[gpu-case]", *msg, file=sys.stderr, flush=True)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> a cuda bfloat16 tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.float16).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host_bf16_as_f64(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def rel_frobenius(out, ref):
    """||out - ref||_F / ||ref||_F in fp64 (the pages' CHECKALL metric)."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(out - ref) / den) if den > 0 else float(np.linalg.norm(out))


# rel_F bar for bf16 outputs of the W4A8 GEMM (bf16 rounding alone is ~1.66e-3)
GEMM_REL_F = 2e-3

# fewest compared outputs at which the rel_F statistic is stable enough to gate on
GEMM_REL_F_MIN_OUTPUTS = 1024


def assert_gemm_close(got, ref, name=""):
    """The GEMM bar on bf16 outputs against the exact (fp64, unrounded) result:
    every output within bf16 rounding of it (half an ulp, at most 2^-8 relative)
    plus 1e-3 of the outputs' RMS for fp32 accumulation order; and rel_F <=
    GEMM_REL_F over the compared outputs.  bf16 rounding alone puts rel_F near
    1.5e-3 in expectation, so over a few dozen outputs its sampling spread
    passes the bar's headroom even when every output is correctly rounded:
    below GEMM_REL_F_MIN_OUTPUTS outputs the per-element bound decides."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    slack = np.abs(ref) * 2.0 ** -8 + 1e-3 * np.sqrt(np.mean(ref * ref))
    bad = np.abs(got - ref) > slack
    assert not bad.any(), (name, int(bad.sum()), float(np.max(np.abs(got - ref) - slack)))
    if ref.size >= GEMM_REL_F_MIN_OUTPUTS:
        err = rel_frobenius(got, ref)
        assert err <= GEMM_REL_F, (name, err)
