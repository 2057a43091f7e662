"""Pins for the oracle's number formats (CPU only).

e2m1: the page's grid ("radiance_nvfp4.py", unpack_e2m1) from tests/golden.
e4m3 / fp16 / bf16 decode and the e4m3 RNE encode: checked against torch's and
numpy's own casts (library routines), over all codes, every rounding boundary,
saturation and signed-zero cases, and a random sample.
"""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def test_e2m1_grid_golden(orc):
    grid = {int(i): float(v) for i, v in _rows("e2m1_grid.txt")}
    assert len(grid) == 8
    for c in range(16):
        v = orc.e2m1_value(c)
        expect = grid[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == expect, (c, v, expect)
    # code 8 is negative zero
    assert np.signbit(orc.e2m1_value(8)) and orc.e2m1_value(8) == 0.0
    assert not np.signbit(orc.e2m1_value(0))


def test_e4m3_decode_all_codes_vs_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = orc.e4m3_value(b)
        if b in (0x7F, 0xFF):
            assert np.isnan(v) and np.isnan(ref[b])
        else:
            assert v == ref[b], (hex(b), v, ref[b])
            assert np.signbit(v) == bool(b & 0x80)
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9


def test_f16_decode_all_codes_vs_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for h in range(0, 65536, 7):  # stride: ~9.4k codes, all exponents
        v = orc.f16_value(h)
        if np.isnan(ref[h]):
            assert np.isnan(v)
        else:
            assert v == ref[h], (hex(h), v, ref[h])


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_every_boundary_vs_torch(orc):
    pos = np.array([orc.e4m3_value(b) for b in range(0x7F)], np.float64)  # 0 .. 448
    ys = []
    for i in range(len(pos) - 1):
        mid = np.float32((pos[i] + pos[i + 1]) / 2)  # exact in fp32
        assert float(mid) == (pos[i] + pos[i + 1]) / 2
        u = int(mid.view(np.uint32))
        for d in range(-8, 9):
            ys.append(np.uint32(max(u + d, 0)).view(np.float32))
        ys.append(np.float32(pos[i]))
    ys = np.array(ys, np.float32)
    ys = ys[(ys >= 0) & (ys <= 448)]
    ys = np.concatenate([ys, -ys])
    got = orc.e4m3_encode_array(ys)
    ref = _torch_e4m3(ys)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(ys[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_random_vs_torch(orc):
    g = np.random.default_rng(123)
    y = np.concatenate([
        g.uniform(-448, 448, 1 << 20),
        np.ldexp(g.uniform(-1, 1, 1 << 20), g.integers(-12, 9, 1 << 20)),
    ]).astype(np.float32)
    y = y[np.abs(y) <= 448]
    got = orc.e4m3_encode_array(y)
    assert np.array_equal(got, _torch_e4m3(y))


def test_e4m3_encode_saturation_and_sign(orc):
    for y in [448.0, 448.5, 463.99, 464.0, 464.01, 479.0, 480.0, 1e6, 3.0e38]:
        assert orc.e4m3_encode(y) == 0x7E, y
        assert orc.e4m3_encode(-y) == 0xFE, y
    assert orc.e4m3_encode(0.0) == 0x00
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(-1e-30) == 0x80          # rounds to zero, keeps the sign
    assert orc.e4m3_encode(2.0 ** -10) == 0x00       # tie between 0 and 2^-9 -> even code 0
    assert orc.e4m3_encode(3 * 2.0 ** -10) == 0x02   # tie between codes 1 and 2 -> 2
    assert orc.e4m3_encode(-(2.0 ** -9)) == 0x81


def test_bf16_decode_sample_vs_torch(orc):
    bits = np.arange(0, 65536, 3, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([orc.bf16_value(int(b)) for b in bits], np.float32)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
