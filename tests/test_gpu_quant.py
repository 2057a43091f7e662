"""GPU parity: per-token fp8 activation quantization and NVFP4 -> MXFP4 requant.

Both are bit-exact contracts: every e4m3 code, fp32 token scale, e2m1 code and
e8m0 byte from the HIP kernels (called through the C ABI via the binding) must
equal the CPU oracle's.  Inputs are seeded synthetic data of the pages' shapes
(w4a8_gemm_amd.synth) plus hand-made edge cases.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import dev_bf16, dev_u8, host, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _act_case(bits, K=None, ldx=None, name=""):
    bits = np.ascontiguousarray(bits, np.uint16)
    M, L = bits.shape
    K = L if K is None else K
    say("act_quant", name, (M, K, L))
    xt = dev_bf16(bits)
    x8, s = w4.quant_act_fp8_per_token(xt[:, :K])
    r8, rs = oracle.quant_act_fp8(bits, K=K, ldx=L)
    g8, gs = host(x8), host(s)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), name
    bad = np.argwhere(g8 != r8)
    assert bad.size == 0, (name, bad[:5], g8[tuple(bad[0])], r8[tuple(bad[0])])


def test_act_quant_tiny():
    t = synth.tiny()
    _act_case(t["x"], name="tiny")


def test_act_quant_every_bf16_value():
    # a row whose amax is 448 has scale exactly 1, so every bf16 value in
    # [-448, 448] reaches the e4m3 rounding unchanged
    pos = np.arange(0, 0x43E1, dtype=np.uint16)            # +0 .. 448
    vals = np.concatenate([pos, pos | 0x8000])
    K = (vals.size + 7) // 8 * 8
    row = np.zeros(K, np.uint16)
    row[: vals.size] = vals
    # a second row: same values divided by 2^20 (scale 448 / 2^20, non-trivial y)
    f = torch.from_numpy(row.view(np.int16)).view(torch.bfloat16).float() / 2.0 ** 20
    row2 = _bf16_bits(f.numpy())
    _act_case(np.stack([row, row2]), name="all-bf16")


def test_act_quant_edge_rows():
    g = np.random.default_rng(7)
    K = 4096
    rows = [np.zeros(K, np.float32),                              # all zero: scale 1
            -np.zeros(K, np.float32),                             # negative zeros
            g.standard_normal(K).astype(np.float32) * 1e-38,      # subnormal bf16
            g.standard_normal(K).astype(np.float32) * 1e30,
            g.standard_normal(K).astype(np.float32) * 3e-5,
            np.where(g.random(K) < 0.99, 0.0, g.standard_normal(K)).astype(np.float32)]
    one = np.zeros(K, np.float32)
    one[123] = -7.0                                                # single nonzero
    rows.append(one)
    _act_case(np.stack([_bf16_bits(r) for r in rows]), name="edge-rows")


def test_act_quant_ragged_and_strided():
    x = synth.acts(37, 1104, seed=11, spread=100.0)
    _act_case(x, K=1001, name="ragged K=1001 ldx=1104")          # scalar path
    _act_case(x, K=1096, name="K=1096 ldx=1104")                 # vector path, strided rows
    _act_case(x[:1, :8], name="1x8")
    _act_case(x[:1, :1], name="1x1")


def test_act_quant_register_and_two_pass_boundaries():
    # rows held in registers take 1/2/4/8/16 uint4 per thread (K <= 32768);
    # K = 32776 falls back to the two-pass form
    for K in (8, 2048, 2056, 4104, 8200, 12288, 32768, 32776):
        _act_case(synth.acts(3, K, seed=(5, K), spread=50.0), name=f"K={K}")


def test_act_quant_decode_and_prefill_shapes():
    for M, K, seed in ((1, 5120, (1, 1)), (64, 5120, (1, 64)), (16, 17408, (2, 16))):
        _act_case(synth.acts(M, K, seed=seed, spread=10.0), name=f"M={M} K={K}")
    _act_case(synth.acts(4096, 5120, seed=3), name="prefill 4096x5120")


# ---------------------------------------------------------------------------
# requant
# ---------------------------------------------------------------------------

def _requant_case(d, mode, row_chunk=0, name="", stats=True):
    say("requant", name, mode, d["nv_packed"].shape, "row_chunk", row_chunk)
    mp, me, st = w4.requant_nvfp4_to_mxfp4(dev_u8(d["nv_packed"]), dev_u8(d["nv_scale"]),
                                           d["part_rows"], d["part_divisor"], mode=mode,
                                           row_chunk=row_chunk, stats=True)
    rp, re_, rst = oracle.requant_nvfp4_to_mxfp4(d["nv_packed"], d["nv_scale"], d["part_rows"],
                                                 d["part_divisor"], mode=mode)
    gp, ge = host(mp), host(me)
    bad = np.argwhere(ge != re_)
    assert bad.size == 0, (name, mode, "e8m0", bad[:5], ge[tuple(bad[0])], re_[tuple(bad[0])])
    bad = np.argwhere(gp != rp)
    assert bad.size == 0, (name, mode, "codes", bad[:5], gp[tuple(bad[0])], rp[tuple(bad[0])])
    if stats:
        np.testing.assert_allclose(host(st), rst, rtol=1e-6, atol=0)
    return gp, ge


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_requant_tiny(mode):
    _requant_case(synth.tiny(), mode, name="tiny")


def _random_nvfp4(rows, K, seed, divisors):
    g = np.random.default_rng(seed)
    packed = g.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scale = g.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    scale[(scale & 0x7F) == 0x7F] = 0x38        # no NaN scale bytes
    parts = np.full(len(divisors), rows // len(divisors), np.int64)
    parts[-1] += rows - parts.sum()
    return dict(nv_packed=packed, nv_scale=scale, part_rows=parts,
                part_divisor=np.asarray(divisors, np.float32))


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_requant_random_bytes_many_partitions(mode):
    # every code and scale byte, signed scales, subnormal scales, divisors from
    # 3e38 (subnormal weights, exponent clamp at -127) to 1e-30 (exponent ~100)
    d = _random_nvfp4(997, 96, 5, [2688.0, 1.0, 3e38, 1e-30, 0.37, 6.5e4, 1e-3])
    _requant_case(d, mode, name="random-bytes")
    _requant_case(d, mode, row_chunk=100, name="random-bytes chunked")


def test_requant_partition_edge_cases():
    d = _random_nvfp4(64, 32, 9, [5.0, 7.0, 11.0])
    d["part_rows"] = np.array([0, 64, 0], np.int64)                 # empty partitions
    _requant_case(d, "mse", name="empty partitions")
    z = dict(d)
    z["nv_packed"] = np.zeros_like(d["nv_packed"])                  # all-zero blocks: byte 127
    _, ge = _requant_case(z, "mse", name="zero blocks")
    assert (ge == 127).all()


def test_requant_gate_up_full_mse(gate_up_mx):
    g = synth.gate_up()
    gp, ge = _requant_case(g, "mse", row_chunk=4096, name="gate_up ROW_CHUNK=4096")
    assert np.array_equal(gp, gate_up_mx[0]) and np.array_equal(ge, gate_up_mx[1])


@pytest.mark.parametrize("mode", ["ocp", "noclip"])
def test_requant_gate_up_other_modes(mode):
    # the whole merged layer (both partitions, each with its divisor) in passes
    # of 4096 rows, as the full-layer requant config runs it
    _requant_case(synth.gate_up(), mode, row_chunk=4096, name="gate_up ROW_CHUNK=4096")


def test_requant_rejects_bad_arguments():
    d = synth.tiny()
    p, s = dev_u8(d["nv_packed"]), dev_u8(d["nv_scale"])
    with pytest.raises(ValueError):
        w4.requant_nvfp4_to_mxfp4(p, s, [128, 100], [1.0, 1.0])     # rows do not add up
    with pytest.raises(ValueError):
        w4.requant_nvfp4_to_mxfp4(p, s, [256], [0.0])               # divisor <= 0
    with pytest.raises(ValueError):
        w4.requant_nvfp4_to_mxfp4(p, s, [256], [float("inf")])
    with pytest.raises(ValueError):
        w4.requant_nvfp4_to_mxfp4(p[:, :8], s[:, :1], [256], [1.0])  # K = 16: K % 32 != 0


# ---------------------------------------------------------------------------
# bf16 / fp8 per-channel weights -> MXFP4 at load (the requant encoder)
# ---------------------------------------------------------------------------

def _load_case(kind, a, mode, name, scale=None):
    rows, K = a.shape
    say("load quant", kind, name, mode, (rows, K))
    if kind == "bf16":
        mp, me, st = w4.quant_bf16_to_mxfp4(dev_bf16(a), mode=mode, stats=True)
        rp, re_, rst = oracle.quant_bf16_to_mxfp4(a, mode)
    else:
        mp, me, st = w4.quant_fp8ch_to_mxfp4(dev_u8(a), torch.from_numpy(scale).cuda(), mode=mode, stats=True)
        rp, re_, rst = oracle.quant_fp8ch_to_mxfp4(a, scale, mode)
    gp, ge = host(mp), host(me)
    bad = np.argwhere(ge != re_)
    assert bad.size == 0, (kind, name, mode, "e8m0", bad[:5])
    bad = np.argwhere(gp != rp)
    assert bad.size == 0, (kind, name, mode, "codes", bad[:5])
    np.testing.assert_allclose(host(st), rst, rtol=1e-6, atol=0)


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_quant_bf16_random_bits(mode):
    # every finite bf16 pattern class: subnormals, zeros of both signs, the
    # largest finite values (exponent clamp at 127), ragged row counts
    g = np.random.default_rng(21)
    for rows, K in [(1, 32), (7, 96), (257, 320)]:
        a = g.integers(0, 1 << 16, (rows, K)).astype(np.uint16)
        a[(a & 0x7F80) == 0x7F80] &= 0xFF7F                       # no inf / NaN
        _load_case("bf16", a, mode, f"random {rows}x{K}")


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_quant_fp8ch_random_codes(mode):
    g = np.random.default_rng(22)
    for rows, K in [(1, 32), (9, 160), (300, 256)]:
        c = g.integers(0, 256, (rows, K)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x7E                              # no NaN codes
        s = np.exp2(g.uniform(-30, 20, rows)).astype(np.float32) * g.uniform(1, 2, rows).astype(np.float32)
        _load_case("fp8", c, mode, f"random {rows}x{K}", s)


def _decision_point_sweep():
    """fp8 per-channel rows built so that the encoder's fp32 -> e2m1 step sees
    every fp32 mantissa near each of its decision points.  Row r has scale
    s_r in [1, 2); block j (j = 0..4) holds e4m3 2^j at element 0, which fixes
    the ocp exponent at j - 2, and +-2^-i (i = k mod 5) at element k, so
    w = +-2^-i s_r exactly and the scaled magnitude is 4 s_r / 2^(i + j): s_r's
    mantissa lands on [4, 8), [2, 4), [1, 2), [0.5, 1) and [0.25, 0.5), where the
    nearest-even decisions sit at 5 (and the clip at 6), 2.5 and 3.5, 1.25 and
    1.75, 0.75, and 0.25.  The scales sweep 4096 fp32 steps on each side of
    mantissa 1, 1.25, 1.5, 1.75 and 2, plus random mantissas."""
    one = int(np.float32(1.0).view(np.uint32))
    centres = [one + (c << 21) for c in (0, 2, 4, 6, 8)]        # mantissas 1, 1.25, 1.5, 1.75, 2
    bits = np.concatenate([np.arange(c - 4096, c + 4097) for c in centres]
                          + [one + np.random.default_rng(31).integers(0, 1 << 23, 16384)])
    bits = bits[(bits >= one) & (bits < one + (1 << 23))]
    scale = bits.astype(np.uint32).view(np.float32)
    K = 160
    k = np.arange(K) % 32
    j = np.arange(K) // 32
    i = k % 5
    code = ((7 - i) << 3).astype(np.uint8)                     # e4m3 2^-i
    code[k % 2 == 1] |= 0x80                                  # every other element negative
    code[k == 0] = ((7 + j[k == 0]) << 3).astype(np.uint8)    # e4m3 2^j: the block's amax
    return np.tile(code, (scale.size, 1)), np.ascontiguousarray(scale)


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_quant_fp8ch_e2m1_decision_points(mode):
    codes, scale = _decision_point_sweep()
    _load_case("fp8", codes, mode, f"decision points {codes.shape}", scale)


def test_quant_bf16_gate_up_shape():
    a = synth.bf16_weight()
    _load_case("bf16", a, "mse", "gate_up-shaped")


def test_quant_fp8ch_gate_up_shape():
    d = synth.fp8ch_weight()
    _load_case("fp8", d["w8"], "mse", "gate_up-shaped", d["row_scale"])


def test_load_quant_rejects_bad_arguments():
    z = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        w4.quant_bf16_to_mxfp4(z)                                   # K % 32
    c = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        w4.quant_fp8ch_to_mxfp4(c, torch.ones(3, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        w4.quant_bf16_to_mxfp4(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"), mode="nearest")


# ---------------------------------------------------------------------------
# the same encoders writing the GEMM's fragment order directly: bit for bit the
# repack (w4a8_mxfp4_prepare) of the oracle's row-major codes and e8m0, padding
# rows and steps included
# ---------------------------------------------------------------------------

def _repacked(codes, e8m0):
    return w4.mxfp4_prepare(dev_u8(codes), dev_u8(e8m0))


def _same_prepared(got, want, name):
    gw, ww = host(got.w), host(want.w)
    bad = np.argwhere(gw != ww)
    assert bad.size == 0, (name, "codes", bad[:5])
    gs, ws = host(got.s), host(want.s)
    bad = np.argwhere(gs != ws)
    assert bad.size == 0, (name, "e8m0", bad[:5])
    assert (got.N, got.K) == (want.N, want.K)


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_requant_prepared_random_bytes(mode):
    # 157 rows (a partial last tile), K of 5 steps (three padding steps), three
    # partitions whose boundaries fall inside 16-row tiles, divisors from 1e-30
    # to 3e38
    d = _random_nvfp4(157, 640, 41, [2688.0, 3e38, 1e-30])
    say("requant prepared", mode, d["part_rows"])
    got = w4.requant_nvfp4_to_mxfp4_prepared(dev_u8(d["nv_packed"]), dev_u8(d["nv_scale"]), d["part_rows"],
                                             d["part_divisor"], mode=mode)
    rp, re_, _ = oracle.requant_nvfp4_to_mxfp4(d["nv_packed"], d["nv_scale"], d["part_rows"], d["part_divisor"],
                                               mode=mode)
    _same_prepared(got, _repacked(rp, re_), f"random {mode}")


def test_requant_prepared_gate_up(gate_up_mx):
    g = synth.gate_up()
    say("requant prepared", "gate_up", g["nv_packed"].shape)
    got = w4.requant_nvfp4_to_mxfp4_prepared(dev_u8(g["nv_packed"]), dev_u8(g["nv_scale"]), g["part_rows"],
                                             g["part_divisor"], mode="mse")
    _same_prepared(got, _repacked(gate_up_mx[0], gate_up_mx[1]), "gate_up")


@pytest.mark.parametrize("mode", ["ocp", "noclip", "mse"])
def test_load_quant_prepared_random(mode):
    g = np.random.default_rng(42)
    a = g.integers(0, 1 << 16, (257, 384)).astype(np.uint16)
    a[(a & 0x7F80) == 0x7F80] &= 0xFF7F                           # no inf / NaN
    say("bf16 prepared", mode, a.shape)
    rp, re_, _ = oracle.quant_bf16_to_mxfp4(a, mode)
    _same_prepared(w4.quant_bf16_to_mxfp4_prepared(dev_bf16(a), mode=mode), _repacked(rp, re_), f"bf16 {mode}")
    c = g.integers(0, 256, (300, 640)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E                                  # no NaN codes
    s = np.exp2(g.uniform(-30, 20, 300)).astype(np.float32)
    say("fp8ch prepared", mode, c.shape)
    rp, re_, _ = oracle.quant_fp8ch_to_mxfp4(c, s, mode)
    got = w4.quant_fp8ch_to_mxfp4_prepared(dev_u8(c), torch.from_numpy(s).cuda(), mode=mode)
    _same_prepared(got, _repacked(rp, re_), f"fp8ch {mode}")


def test_load_quant_prepared_rejects_bad_arguments():
    with pytest.raises(ValueError):
        w4.quant_bf16_to_mxfp4_prepared(torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda"))   # K % 128
    p = torch.zeros((32, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros((32, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        w4.requant_nvfp4_to_mxfp4_prepared(p, s, [2] * 16 + [0], [1.0] * 17)                    # 17 partitions
