"""Pins for the oracle's per-token fp8 quant and GEMM references (CPU only).

fp8 activations ("radiance_autoround.py", autoround_linear: per-token dynamic
e4m3 with an fp32 scale per row): a hand-worked row, the invariants that fix
the scale (every nonzero row reaches +-448), the half-ulp reconstruction bound,
the all-zero row, and agreement with torch's e4m3 cast of x/s.

GEMM ("radiance_autoround.py", _exact_ref; MXFP4 dequant from
"radiance_nvfp4.py", dequant_mxfp4): one-hot weights against the closed form,
all-ones weights against a library sum, nibble order, per-block scale index,
sign flip, a torch fp64 matmul of library-decoded operands, and the int4
code map (c - 8, exact in e4m3) including int4 == MXFP4 on shared values.
"""
import os

import numpy as np
import torch

from w4a8_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = int(v, 0)
    return out


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dec_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- activations

def test_act_hand_worked_row(orc):
    x = _bf16([[448.0, -224.0, 1.0, 0.0, -0.0, 0.001]])
    x8, s = orc.quant_act_fp8(x)
    assert s[0] == 1.0
    # 448 = 1.75*2^8 -> 0x7E; -224 = -1.75*2^7 -> 0xF6; 1.0 -> 0x38; 0 -> 0x00; -0 -> 0x80
    assert list(x8[0, :5]) == [0x7E, 0xF6, 0x38, 0x00, 0x80]
    x = _bf16([[896.0, 1.0]])          # s = 2: 896 -> 448, 1 -> 0.5 = 0x30
    x8, s = orc.quant_act_fp8(x)
    assert s[0] == 2.0 and list(x8[0]) == [0x7E, 0x30]


def test_act_invariants(orc):
    x = synth.acts(64, 1024, 11, spread=10.0)
    x[5] = 0
    x8, s = orc.quant_act_fp8(x)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    dec = _dec_e4m3(x8)
    for m in range(64):
        if m == 5:
            assert s[m] == 1.0 and not (x8[m] & 0x7F).any()
            continue
        assert ((x8[m] & 0x7F) == 0x7E).any()          # the row max lands on 448
        assert s[m] == np.float32(np.float32(np.abs(xf[m]).max()) / np.float32(448.0))
        err = np.abs(dec[m] * s[m] - xf[m])
        # half an e4m3 ulp of the scaled value (3 mantissa bits), times s, plus
        # the subnormal floor 2^-10 * s, plus the rounding of x/s itself
        y = np.abs(xf[m]) / s[m]
        ulp = np.where(y >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 1e-300))).astype(int) - 3), 2.0 ** -9)
        assert (err <= (ulp / 2 + 1e-6 * y) * s[m] + 1e-30).all()
        assert ((x8[m] >> 7) == np.signbit(xf[m])).all()


def test_act_codes_match_torch_cast(orc):
    x = synth.acts(32, 4096, 12, spread=100.0)
    x8, s = orc.quant_act_fp8(x)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    y = xt / torch.from_numpy(s)[:, None]              # IEEE fp32 division
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(x8, ref)


def test_act_strided_rows(orc):
    x = synth.acts(8, 300, 13)
    x8a, sa = orc.quant_act_fp8(x[:, :256], K=256)
    x8b, sb = orc.quant_act_fp8(x, K=256, ldx=300)
    assert np.array_equal(x8a, x8b) and np.array_equal(sa, sb)


# ---------------------------------------------------------------- MXFP4 GEMM

def test_gemm_one_hot_weights(orc):
    g = np.random.default_rng(20)
    M, N, K = 3, 4, 128
    x8 = g.integers(0, 256, (M, K)).astype(np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x11
    xs = np.array([0.5, 3.0, 1e-3], np.float32)
    for kstar in (0, 1, 31, 32, 33, 127):
        for code in (1, 7, 10, 15):
            wp = np.zeros((N, K // 2), np.uint8)
            we = np.full((N, K // 32), 127, np.uint8)
            n = 2
            wp[n, kstar // 2] = code if kstar % 2 == 0 else code << 4
            we[n, kstar // 32] = 127 + 5
            ref = orc.mxfp4_gemm(x8, xs, wp, we)
            val = orc.e2m1_value(code) * 2.0 ** 5
            expect = xs.astype(np.float64) * _dec_e4m3(x8[:, kstar]) * val
            assert np.array_equal(ref[:, n], expect), (kstar, code)
            assert not ref[:, [0, 1, 3]].any()


def test_gemm_all_ones_is_row_sum(orc):
    g = np.random.default_rng(21)
    M, N, K = 4, 3, 256
    x8 = g.integers(0, 256, (M, K)).astype(np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x22
    xs = np.array([1.0, 0.25, 7.0, 2.0], np.float32)
    wp = np.full((N, K // 2), 0x22, np.uint8)            # code 2 = 1.0 in both nibbles
    we = np.full((N, K // 32), 127, np.uint8)
    ref = orc.mxfp4_gemm(x8, xs, wp, we)
    rs = torch.from_numpy(_dec_e4m3(x8)).sum(1).numpy() * xs
    assert np.allclose(ref, rs[:, None], rtol=1e-15, atol=0)


def test_gemm_sign_flip_and_block_scale(orc):
    g = np.random.default_rng(22)
    M, N, K = 2, 5, 192
    x8 = synth_fp8(g, M, K)
    xs = np.array([0.3, 1.7], np.float32)
    codes = g.integers(0, 16, (N, K))
    codes[codes == 8] = 0
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    we = g.integers(120, 135, (N, K // 32)).astype(np.uint8)
    ref = orc.mxfp4_gemm(x8, xs, wp, we)
    flip = np.where(codes > 0, codes ^ 8, 0)
    wpf = (flip[:, 0::2] | (flip[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(orc.mxfp4_gemm(x8, xs, wpf, we), -ref)
    # raising block b's exponent by one doubles exactly that block's share
    b = 3
    we2 = we.copy()
    we2[:, b] += 1
    wp_b = np.zeros_like(wp)
    wp_b[:, b * 16:(b + 1) * 16] = wp[:, b * 16:(b + 1) * 16]
    share = orc.mxfp4_gemm(x8, xs, wp_b, we)
    assert np.allclose(orc.mxfp4_gemm(x8, xs, wp, we2), ref + share, rtol=1e-14, atol=1e-300)


def synth_fp8(g, M, K):
    x8 = g.integers(0, 256, (M, K)).astype(np.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x33
    return x8


def test_gemm_matches_library_matmul_and_sampling(orc):
    g = np.random.default_rng(23)
    M, N, K = 5, 48, 512
    x8 = synth_fp8(g, M, K)
    xs = g.uniform(0.01, 2, M).astype(np.float32)
    codes = g.integers(0, 16, (N, K))
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    we = g.integers(110, 140, (N, K // 32)).astype(np.uint8)
    ref = orc.mxfp4_gemm(x8, xs, wp, we)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    wd = grid[codes & 7] * np.where(codes & 8, -1.0, 1.0) * np.repeat(np.ldexp(1.0, we.astype(int) - 127), 32, 1)
    lib = (torch.from_numpy(_dec_e4m3(x8)) @ torch.from_numpy(wd).T).numpy() * xs[:, None]
    assert np.allclose(ref, lib, rtol=1e-12, atol=1e-300)
    mi = g.integers(0, M, 50)
    ni = g.integers(0, N, 50)
    assert np.array_equal(orc.mxfp4_gemm(x8, xs, wp, we, mi, ni), ref[mi, ni])


# ---------------------------------------------------------------- int4 g128

def test_int4_code_map_exact_in_e4m3(orc):
    kv = _kv("int4_symmetric.txt")
    assert kv["zero_point"] == ((kv["qzeros_word"] & 0xF) + 1)
    for c in range(16):
        v = c - kv["zero_point"]
        assert kv["code_min_value"] <= v <= kv["code_max_value"]
        assert orc.e4m3_value(orc.e4m3_encode(float(v))) == v


def test_int4_prepare_checks_symmetry_and_transposes(orc):
    kv = _kv("int4_symmetric.txt")
    d = synth.int4(seed=9, N=64, K=256)
    out, bad = orc.int4_prepare(d["qweight_kn"], d["qzeros"], 64, 256)
    assert bad == 0 and np.array_equal(out, d["qweight_kn"].T)
    qz = d["qzeros"].copy()
    assert (qz.view(np.uint32) == kv["qzeros_word"]).all()
    qz[1, 3] = 0x77777778
    qz[0, 0] = 0
    out, bad = orc.int4_prepare(d["qweight_kn"], qz, 64, 256)
    assert out is None and bad == 2


def test_int4_equals_mxfp4_on_shared_values(orc):
    """Codes whose c-8 is on the e2m1 grid and power-of-two fp16 scales give the
    same reference through the int4 path and the MXFP4 path."""
    g = np.random.default_rng(24)
    M, N, K = 3, 16, 256
    x8 = synth_fp8(g, M, K)
    xs = g.uniform(0.1, 1, M).astype(np.float32)
    vals = np.array([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6])
    v = vals[g.integers(0, len(vals), (N, K))]
    c = v + 8
    qw = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        qw |= (c[:, j::8].astype(np.uint32) << (4 * j))
    jexp = g.integers(-8, 4, (K // 128, N))
    scales = np.ldexp(1.0, jexp).astype(np.float16).view(np.uint16)
    ref_i4 = orc.int4_gemm(x8, xs, qw.view(np.int32), scales)
    e2m1_of = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7}
    code = np.vectorize(lambda t: e2m1_of[abs(t)] | (8 if t < 0 else 0))(v)
    wp = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    we = (127 + np.repeat(jexp.T, 4, axis=1)).astype(np.uint8)      # [N, K/32]
    ref_mx = orc.mxfp4_gemm(x8, xs, wp, we)
    assert np.array_equal(ref_i4, ref_mx)


def test_int4_gemm_matches_library_matmul(orc):
    d = synth.int4(seed=10, N=32, K=512)
    g = np.random.default_rng(25)
    x8 = synth_fp8(g, 4, 512)
    xs = g.uniform(0.1, 1, 4).astype(np.float32)
    qnk, _ = orc.int4_prepare(d["qweight_kn"], d["qzeros"], 32, 512)
    ref = orc.int4_gemm(x8, xs, qnk, d["scales"])
    u = qnk.view(np.uint32)
    codes = np.stack([(u >> (4 * j)) & 15 for j in range(8)], -1).reshape(32, 512).astype(np.int64)
    sc = d["scales"].view(np.float16).astype(np.float64)          # [K/128, N]
    wd = (codes - 8) * np.repeat(sc.T, 128, axis=1)
    lib = (torch.from_numpy(_dec_e4m3(x8)) @ torch.from_numpy(wd).T).numpy() * xs[:, None]
    assert np.allclose(ref, lib, rtol=1e-12, atol=1e-300)
