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
