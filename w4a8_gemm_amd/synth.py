"""Seeded synthetic inputs for the MXFP4 W4A8 linear layer.

This module makes *inputs* only.  It holds none of the layer's own arithmetic
(no NVFP4 dequant, no MXFP4 encoding, no fp8 activation quant, no GEMM), so it
can feed both the library and the CPU oracle without tying them together.
Random draws come from torch's seeded CPU generator; bf16, fp16 and e4m3 values
come from torch's own round-to-nearest-even casts.

Workload shapes follow the pages: hidden size 5120, MLP intermediate 17408,
a merged gate_up projection of two 17408-row partitions ("radiance_nvfp4.py",
RadianceNvfp4ToMxfp4: per-partition global scales; "vllm-radiance (MXFP4)",
How the MXFP4 path works: the gate_up 17408x5120 measurement), and the
AutoGPTQ int4 layout of "radiance_autoround.py" (module docstring).

Generators (all arrays are numpy, on the host):
  tiny()              NVFP4 256x512, uniform codes, scales 2^U(-4,2), M=4 acts
  gate_up()           NVFP4 2x17408 x 5120 from N(0, 0.02^2) with 0.1% x20
                      outliers, partition amax ratio 1.7
  down_proj()         MXFP4 5120 x 17408 drawn in the encoded domain with a
                      heavy-tailed (Student-t, 4 dof) per-row exponent
  int4()              int4 g128 symmetric, qweight [K/8, N], fp16 scales
  acts(M, K, seed)    bf16 N(0,1) activations, optional per-token spread
"""
from __future__ import annotations

import functools

import numpy as np
import torch

HIDDEN = 5120
INTERMEDIATE = 17408
# "radiance_nvfp4.py": compressed-tensors stores the global scale as 6*448/amax.
NVFP4_GLOBAL_NUM = 6.0 * 448.0


def _gen(seed) -> torch.Generator:
    if isinstance(seed, (tuple, list)):
        s = 0
        for v in seed:
            s = (s * 1000003 + int(v)) & 0x7FFFFFFFFFFFFFFF
        seed = s
    return torch.Generator().manual_seed(int(seed))


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """fp32 -> bf16 (torch RNE cast) -> raw uint16 bits."""
    return x.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_bits(x: torch.Tensor) -> np.ndarray:
    """fp32 -> float8_e4m3fn (torch RNE cast; inputs kept in range) -> uint8 bits."""
    return x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pack_nibbles(codes: torch.Tensor) -> np.ndarray:
    """[rows, K] codes 0..15 -> [rows, K/2] bytes, even k in the low nibble."""
    c = codes.to(torch.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous().numpy()


def acts(M: int, K: int, seed, spread: float = 1.0) -> np.ndarray:
    """bf16 bits [M, K] of N(0,1); row m scaled by spread^(m/(M-1)) (1 for M=1)."""
    g = _gen(seed)
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    if spread != 1.0 and M > 1:
        f = torch.tensor([spread ** (m / (M - 1)) for m in range(M)], dtype=torch.float32)
        x = x * f[:, None]
    return bf16_bits(x)


def tiny(seed: int = 0, N: int = 256, K: int = 512, M: int = 4) -> dict:
    """NVFP4 weight N x K: codes uniform over 0..15, e4m3 scales per 16 drawn as
    2^U(-4,2), one partition whose global divisor is 6*448 over the nominal
    amax 6 * max(scale); bf16 N(0,1) activations M x K."""
    g = _gen(seed)
    codes = torch.randint(0, 16, (N, K), generator=g)
    sval = torch.exp2(torch.rand((N, K // 16), generator=g) * 6.0 - 4.0)
    scale = e4m3_bits(sval)
    smax = float(torch.from_numpy(scale).view(torch.float8_e4m3fn).to(torch.float32).max())
    gd = np.float32(NVFP4_GLOBAL_NUM / (6.0 * smax))
    x = bf16_bits(torch.randn((M, K), generator=g, dtype=torch.float32))
    return dict(nv_packed=pack_nibbles(codes), nv_scale=scale,
                part_rows=np.array([N], np.int64), part_divisor=np.array([gd], np.float32),
                x=x, N=N, K=K, M=M)


# e2m1 magnitudes and the midpoints between them, used only to build NVFP4
# test inputs (the forward NVFP4 quantizer is not part of the layer: the pages
# start from an NVFP4 checkpoint).
_NV_GRID_MID = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=torch.float32)


def _nvfp4_encode(w: torch.Tensor, gd: float, rows_per_step: int = 2048):
    """Standard NVFP4 recipe for building inputs: per 16-block e4m3 scale
    amax16 * gd / 6, codes = nearest e2m1 magnitude of |w| * gd / scale."""
    n, K = w.shape
    packed = np.empty((n, K // 2), np.uint8)
    scale = np.empty((n, K // 16), np.uint8)
    gdt = torch.tensor(gd, dtype=torch.float32)
    for a in range(0, n, rows_per_step):
        wb = w[a:a + rows_per_step].reshape(-1, K // 16, 16)
        amax16 = wb.abs().amax(-1)
        s8 = (amax16 * gdt / 6.0).to(torch.float8_e4m3fn)
        scale[a:a + rows_per_step] = s8.view(torch.uint8).numpy()
        sdec = s8.to(torch.float32)
        mag = torch.where(sdec[..., None] > 0, wb.abs() * gdt / sdec[..., None],
                          torch.zeros_like(wb))
        idx = torch.bucketize(mag, _NV_GRID_MID)
        code = idx | ((wb < 0) & (idx > 0)).to(idx.dtype) << 3
        packed[a:a + rows_per_step] = pack_nibbles(code.reshape(-1, K))
    return packed, scale


def _gate_up_partitions(seed, rows, K, ratio):
    """The two fp32 partitions of the gate_up weight, in order, each with its
    NVFP4 global divisor 6*448/amax."""
    g = _gen(seed)
    amax_gate = None
    for p in range(2):
        w = torch.randn((rows, K), generator=g, dtype=torch.float32) * 0.02
        out = torch.rand((rows, K), generator=g) < 0.001
        w = torch.where(out, w * 20.0, w)
        del out
        amax = float(w.abs().max())
        if p == 0:
            amax_gate = amax
        else:
            w = w * np.float32(amax_gate / ratio / amax)
            amax = float(w.abs().max())
        yield w, float(np.float32(NVFP4_GLOBAL_NUM / amax))


@functools.lru_cache(maxsize=4)
def gate_up(seed: int = 1, rows: int = INTERMEDIATE, K: int = HIDDEN, ratio: float = 1.7) -> dict:
    """Merged gate_up projection, two partitions of `rows` rows each.  Each is
    N(0, 0.02^2) with 0.1% of entries (Bernoulli) multiplied by 20; the up
    partition is rescaled so amax_gate / amax_up = ratio; each partition is
    NVFP4-encoded with its own divisor 6*448/amax."""
    parts, divs = [], []
    for w, gd in _gate_up_partitions(seed, rows, K, ratio):
        parts.append(_nvfp4_encode(w, gd))
        divs.append(gd)
        del w
    return dict(nv_packed=np.concatenate([parts[0][0], parts[1][0]]),
                nv_scale=np.concatenate([parts[0][1], parts[1][1]]),
                part_rows=np.array([rows, rows], np.int64),
                part_divisor=np.array(divs, np.float32), N=2 * rows, K=K)


def gate_up_original(seed: int = 1, rows: int = INTERMEDIATE, K: int = HIDDEN, ratio: float = 1.7) -> torch.Tensor:
    """The unquantized fp32 weight [2 rows, K] that gate_up() encodes to NVFP4
    (same draws), for accuracy reports against the original."""
    return torch.cat([w for w, _ in _gate_up_partitions(seed, rows, K, ratio)])


# Magnitude-index frequencies for synthetic MXFP4 codes (shaped like a
# Gaussian block at its no-clip scale; index 0 also takes the zeros).
_MX_IDX_P = torch.tensor([0.10, 0.16, 0.16, 0.14, 0.16, 0.15, 0.09, 0.04])


@functools.lru_cache(maxsize=4)
def down_proj(seed: int = 2, N: int = HIDDEN, K: int = INTERMEDIATE) -> dict:
    """MXFP4 weight N x K sampled directly in the encoded domain: per row an
    exponent offset floor(log2|t|) (t ~ Student-t, 4 dof, clipped to [-3, 5])
    gives heavy-tailed rows; per block e8m0 = 127 - 7 + offset + U{-1, 0};
    codes: magnitude index from a fixed categorical, random sign when
    nonzero."""
    g = _gen(seed)
    z = torch.randn((N,), generator=g, dtype=torch.float64)
    chi = torch.randn((N, 4), generator=g, dtype=torch.float64).pow(2).sum(-1)
    t = z / torch.sqrt(chi / 4.0)
    off = torch.floor(torch.log2(t.abs().clamp_min(1e-30))).clamp(-3, 5).to(torch.int32)
    jit = torch.randint(-1, 1, (N, K // 32), generator=g, dtype=torch.int32)
    e8m0 = (127 - 7 + off[:, None] + jit).to(torch.uint8).numpy()
    idx = torch.multinomial(_MX_IDX_P, N * K, replacement=True, generator=g).reshape(N, K)
    neg = torch.randint(0, 2, (N, K), generator=g).bool() & (idx > 0)
    codes = idx | (neg.to(idx.dtype) << 3)
    return dict(w_packed=pack_nibbles(codes), w_e8m0=e8m0, N=N, K=K)


@functools.lru_cache(maxsize=4)
def int4(seed: int = 4, N: int = HIDDEN, K: int = INTERMEDIATE) -> dict:
    """AutoGPTQ int4 g128 symmetric: qweight [K/8, N] int32 of uniform codes
    (nibble j of word i is k = 8i + j), fp16 scales [K/128, N] = |N(0, 0.01^2)|,
    qzeros [K/128, N/8] all 0x77777777."""
    g = _gen(seed)
    qw = torch.randint(-(2 ** 31), 2 ** 31, (K // 8, N), generator=g, dtype=torch.int64)
    qweight = qw.to(torch.int32).numpy()
    sc = (torch.randn((K // 128, N), generator=g, dtype=torch.float32) * 0.01).abs()
    scales = sc.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    qzeros = np.full((K // 128, N // 8), 0x77777777, dtype=np.uint32).view(np.int32)
    return dict(qweight_kn=qweight, scales=scales, qzeros=qzeros, N=N, K=K)


def mxfp4_random(N: int, K: int, seed, e_lo: int = 120, e_hi: int = 130) -> dict:
    """MXFP4 weight drawn directly in the encoded domain (for ragged-shape parity
    cases): uniform 4-bit codes, e8m0 bytes uniform in [e_lo, e_hi]."""
    g = _gen(seed)
    codes = torch.randint(0, 16, (N, K), generator=g)
    e8m0 = torch.randint(e_lo, e_hi + 1, (N, K // 32), generator=g).to(torch.uint8).numpy()
    return dict(w_packed=pack_nibbles(codes), w_e8m0=e8m0, N=N, K=K)


def int4_random(N: int, K: int, seed) -> dict:
    """int4 g128 weight of any (N % 8 == 0, K % 128 == 0) shape, same recipe as int4()."""
    return int4.__wrapped__(seed=seed, N=N, K=K)


def int4_zp(N: int = HIDDEN, K: int = INTERMEDIATE, seed=11) -> dict:
    """int4 g128 asymmetric in the same checkpoint layout: codes and fp16 scales
    as int4(), qzeros [K/128, N/8] with every nibble (the zero point minus one)
    uniform in 0..15, so zero points 1..16 all occur."""
    d = dict(int4.__wrapped__(seed=seed, N=N, K=K))
    g = _gen((*seed, 1) if isinstance(seed, (tuple, list)) else (seed, 1))
    qz = torch.randint(-(2 ** 31), 2 ** 31, (K // 128, N // 8), generator=g, dtype=torch.int64)
    d["qzeros"] = qz.to(torch.int32).numpy()
    return d


def int5(N: int = HIDDEN, K: int = INTERMEDIATE, seed=12, symmetric: bool = False) -> dict:
    """int5 g128: uniform 5-bit codes split into the int4 word layout (low four
    bits, qweight [K/8, N]) and a fifth-bit plane (qweight_hi [K/32, N], bit
    k % 32 of word [k/32, n]); zero points minus one [K/128, N] uint8 uniform
    in 0..31 (15, i.e. z = 16, when symmetric); fp16 scales |N(0, 0.005^2)|."""
    g = _gen((*seed, 2) if isinstance(seed, (tuple, list)) else (seed, 2))
    lo = torch.randint(-(2 ** 31), 2 ** 31, (K // 8, N), generator=g, dtype=torch.int64)
    hi = torch.randint(-(2 ** 31), 2 ** 31, (K // 32, N), generator=g, dtype=torch.int64)
    sc = (torch.randn((K // 128, N), generator=g, dtype=torch.float32) * 0.005).abs()
    if symmetric:
        qz = np.full((K // 128, N), 15, np.uint8)
    else:
        qz = torch.randint(0, 32, (K // 128, N), generator=g).to(torch.uint8).numpy()
    return dict(qweight_kn=lo.to(torch.int32).numpy(), qweight_hi=hi.to(torch.int32).numpy(), qzeros=qz,
                scales=sc.to(torch.float16).view(torch.int16).numpy().view(np.uint16), N=N, K=K)


def bf16_weight(N: int = 2 * INTERMEDIATE, K: int = HIDDEN, seed=5) -> np.ndarray:
    """An unquantized bf16 linear [N, K] (bf16 bits, uint16): N(0, 0.02^2) with
    0.1% of entries multiplied by 20, cast to bf16 (RNE)."""
    g = _gen(seed)
    w = torch.randn((N, K), generator=g, dtype=torch.float32) * 0.02
    w = torch.where(torch.rand((N, K), generator=g) < 0.001, w * 20.0, w)
    return bf16_bits(w)


def fp8ch_weight(N: int = 2 * INTERMEDIATE, K: int = HIDDEN, seed=6) -> dict:
    """An fp8 per-channel linear as such checkpoints store it: the weight of
    bf16_weight's recipe, one fp32 scale per row s = amax_row / 448, codes
    e4m3(w / s) (torch's RNE cast).  -> dict(w8 [N, K] u8, row_scale [N] f32)."""
    g = _gen(seed)
    w = torch.randn((N, K), generator=g, dtype=torch.float32) * 0.02
    w = torch.where(torch.rand((N, K), generator=g) < 0.001, w * 20.0, w)
    s = (w.abs().amax(1) / 448.0).clamp(min=1e-12)
    w8 = (w / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return dict(w8=w8, row_scale=s.numpy().astype(np.float32), N=N, K=K)
