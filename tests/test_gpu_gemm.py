"""GPU parity: MXFP4 and int4-g128 W4A8 GEMMs against the CPU oracle.

Tolerance contract: relative Frobenius error ||out - ref||_F / ||ref||_F <= 2e-3
against the oracle's fp64-accumulated dequantized product (bf16 output rounding
alone contributes ~1.66e-3).  The GEMM inputs (e4m3 activations and their
scales, MXFP4 weights) come from the generators and the oracle, never from the
HIP path.  Small shapes and every decode-sized call on the full-size layers
(M <= 64) are compared element by element over the whole output; the prefill
and long-M calls on sampled outputs the oracle computes one by one, with the
same per-element bound.  The split-K decode must be bitwise deterministic.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_f16, dev_f32, dev_i32, dev_u8, host_bf16_as_f64, rel_frobenius, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _acts(M, K, seed, spread=1.0):
    x8, s = oracle.quant_act_fp8(synth.acts(M, K, seed=seed, spread=spread))
    return x8, s


def _mx_full(name, x8, s, wp, we):
    M, N = x8.shape[0], wp.shape[0]
    say("mxfp4_gemm full", name, (M, N, x8.shape[1]))
    out = w4.mxfp4_gemm(dev_u8(x8), dev_f32(s), dev_u8(wp), dev_u8(we))
    got = host_bf16_as_f64(out)
    ref = oracle.mxfp4_gemm(x8, s, wp, we)
    assert_gemm_close(got, ref, name)
    return rel_frobenius(got, ref)


# full oracle outputs of the full-size layers, shared by the plain-layout and
# fragment-order tests of the same activations
_FULL_REF = {}


def _full_ref(key, x8, s, wp, we):
    if key not in _FULL_REF:
        _FULL_REF[key] = oracle.mxfp4_gemm(x8, s, wp, we)
    return _FULL_REF[key]


def _sample_idx(M, N, n_samples, seed):
    """Every row once, random (m, n) pairs, and the last row's last 64 columns."""
    g = np.random.default_rng(seed)
    mi = np.concatenate([np.arange(M), g.integers(0, M, n_samples), np.full(64, M - 1)])
    ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, n_samples), N - 1 - np.arange(64)])
    return mi, ni


def _mx_sampled(name, x8, s, wp, we, n_samples=4096, seed=0, ws=None, reps=2):
    M, N = x8.shape[0], wp.shape[0]
    say("mxfp4_gemm sampled", name, (M, N, x8.shape[1]))
    dx, ds, dw, de = dev_u8(x8), dev_f32(s), dev_u8(wp), dev_u8(we)
    outs = [host_bf16_as_f64(w4.mxfp4_gemm(dx, ds, dw, de, workspace=ws)) for _ in range(reps)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), (name, "not deterministic")
    mi, ni = _sample_idx(M, N, n_samples, seed)
    ref = oracle.mxfp4_gemm(x8, s, wp, we, mi=mi, ni=ni)
    assert_gemm_close(outs[0][mi, ni], ref, name)
    return outs[0]


def _mx_full_size(name, key, x8, s, wp, we, reps=2):
    """A full-size layer at decode M: every output against the oracle."""
    M, N = x8.shape[0], wp.shape[0]
    say("mxfp4_gemm full-size", name, (M, N, x8.shape[1]))
    dx, ds, dw, de = dev_u8(x8), dev_f32(s), dev_u8(wp), dev_u8(we)
    outs = [host_bf16_as_f64(w4.mxfp4_gemm(dx, ds, dw, de)) for _ in range(reps)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), (name, "not deterministic")
    assert_gemm_close(outs[0], _full_ref(key, x8, s, wp, we), name)
    return outs[0]


def test_mxfp4_tiny(gate_tiny):
    t = synth.tiny()
    x8, s = oracle.quant_act_fp8(t["x"])
    _mx_full("tiny", x8, s, *gate_tiny)


# decode band (M <= 64, split K) and prefill band (M > 64) on ragged shapes:
# N not a multiple of the tiles, K a multiple of 32 but not of 128, M = 1, 17, 65
RAGGED = [(1, 64, 128), (1, 300, 96), (4, 256, 512), (5, 100, 544), (16, 257, 1024),
          (17, 300, 224), (33, 129, 640), (64, 512, 2048), (64, 1000, 4096), (1, 6000, 2560),
          (65, 200, 384), (130, 260, 640), (256, 256, 256), (300, 77, 160)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_mxfp4_ragged_shapes(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K))
    x8, s = _acts(M, K, (M, K), spread=10.0)
    _mx_full(f"ragged {M}x{N}x{K}", x8, s, w["w_packed"], w["w_e8m0"])


def test_mxfp4_extreme_scales():
    # e8m0 bytes across the whole range used by real weights (incl. 2^-127)
    N, K = 96, 256
    w = synth.mxfp4_random(N, K, seed=3, e_lo=0, e_hi=140)
    x8, s = _acts(8, K, 5)
    _mx_full("extreme e8m0", x8, s, w["w_packed"], w["w_e8m0"])


@pytest.mark.parametrize("M", [1, 8, 16, 64])
def test_mxfp4_gate_up_decode(gate_up_mx, M):
    x8, s = _acts(M, synth.HIDDEN, (1, M), spread=10.0)
    _mx_full_size(f"gate_up M={M}", ("gate_up", M), x8, s, *gate_up_mx[:2])


@pytest.mark.parametrize("M", [1, 16, 64])
def test_mxfp4_down_proj_decode(M):
    d = synth.down_proj()
    x8, s = _acts(M, synth.INTERMEDIATE, (2, M))
    _mx_full_size(f"down_proj M={M}", ("down_proj", M), x8, s, d["w_packed"], d["w_e8m0"])


# the plain layout on wide layers at decode M: the spread tiles read [N, K/2]
# codes and [N, K/32] e8m0 in place (K steps a multiple of 8): the same
# products in the same order as on fragment-order weights, so bit-identical
# to the prepared entry point; every activation-tile count, a ragged N (a
# partial last tile, scalar stores), workgroups of 8 and 9 tiles
@pytest.mark.parametrize("M,N,K", [(1, 34816, 5120), (8, 25001, 1024), (17, 30000, 2048), (33, 24584, 1024),
                                   (64, 24576, 1024)])
def test_mxfp4_plain_layout_spread(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 13))
    x8, s = _acts(M, K, (M, K, 13), spread=10.0)
    say("plain-layout spread tiles", (M, N, K))
    dx, ds, dw, de = dev_u8(x8), dev_f32(s), dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"])
    got = host_bf16_as_f64(w4.mxfp4_gemm(dx, ds, dw, de))
    pw = w4.mxfp4_prepare(dw, de)
    assert np.array_equal(got, host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw)))
    mi, ni = _sample_idx(M, N, 8192, M + N)
    assert_gemm_close(got[mi, ni], oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni), (M, N, K))


# the plain layout above the decode band: each call repacks the weight into
# fragment order inside the workspace and runs the prepared tile kernel, so
# the value is the prepared entry point's, bit for bit; K % 128 != 0 keeps
# the row-major tile kernel (checked against the oracle).  A decode call on
# the same workspace afterwards still finds its split-K counters at zero.
@pytest.mark.parametrize("M,N,K", [(65, 5000, 1152), (300, 1000, 4096), (1024, 20000, 640), (200, 520, 1056)])
def test_mxfp4_plain_layout_prefill(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 14))
    x8, s = _acts(M, K, (M, K, 14), spread=10.0)
    say("plain-layout prefill", (M, N, K))
    dx, ds, dw, de = dev_u8(x8), dev_f32(s), dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"])
    ws = w4.Workspace(M, N, K, "mxfp4")
    got = host_bf16_as_f64(w4.mxfp4_gemm(dx, ds, dw, de, workspace=ws))
    if K % 128 == 0:
        pw = w4.mxfp4_prepare(dw, de)
        assert np.array_equal(got, host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw)))
    mi, ni = _sample_idx(M, N, 8192, M + N)
    assert_gemm_close(got[mi, ni], oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni), (M, N, K))
    # a split-K decode call on the same workspace
    xd, sd = _acts(16, K, (16, K, 14))
    a = host_bf16_as_f64(w4.mxfp4_gemm(dev_u8(xd), dev_f32(sd), dw, de, workspace=ws))
    b = host_bf16_as_f64(w4.mxfp4_gemm(dev_u8(xd), dev_f32(sd), dw, de))
    assert np.array_equal(a, b)


def test_mxfp4_prefill_full_size(gate_up_mx):
    x8, s = _acts(4096, synth.HIDDEN, 3)
    _mx_sampled("prefill 4096", x8, s, *gate_up_mx[:2], n_samples=16384, reps=1)


def test_mxfp4_split_k_deterministic_and_workspace_reuse():
    d = synth.down_proj()
    dw, de = dev_u8(d["w_packed"]), dev_u8(d["w_e8m0"])
    ws = w4.Workspace(64, d["N"], d["K"], "mxfp4")
    assert ws.nbytes > 0
    first = {}
    for rep in range(3):
        for M in (64, 1, 16, 3):
            x8, s = _acts(M, d["K"], (9, M))
            say("split-K repeat", rep, M)
            o = host_bf16_as_f64(w4.mxfp4_gemm(dev_u8(x8), dev_f32(s), dw, de, workspace=ws))
            if rep == 0:
                first[M] = o
            else:
                assert np.array_equal(o, first[M]), M


def test_split_k_in_place_counters_return_to_zero(down_proj_prepared):
    """Split-K reduced in place by the last split ("vllm-radiance (MXFP4)", The
    W4A8 fp8-WMMA kernel): calls with different split counts on one workspace
    (register tiles at M = 16 / 32, split-K decode at M = 3 / 8, the
    plain-layout decode kernel) each match the reference, repeat bit for bit,
    and leave every arrival counter at zero."""
    d, pw = down_proj_prepared
    ws = w4.Workspace(64, d["N"], d["K"], "prepared")
    ws_rm = w4.Workspace(64, d["N"], d["K"], "mxfp4")
    dw, de = dev_u8(d["w_packed"]), dev_u8(d["w_e8m0"])
    first = {}
    for rep in range(3):
        for M in (16, 3, 32, 8, 1):
            x8, s = _acts(M, d["K"], (11, M))
            say("split-K in place", rep, M)
            dx, ds = dev_u8(x8), dev_f32(s)
            o = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw, workspace=ws))
            o_rm = host_bf16_as_f64(w4.mxfp4_gemm(dx, ds, dw, de, workspace=ws_rm))
            if rep == 0:
                mi, ni = _sample_idx(M, d["N"], 4096, M)
                ref = oracle.mxfp4_gemm(x8, s, d["w_packed"], d["w_e8m0"], mi=mi, ni=ni)
                assert_gemm_close(o[mi, ni], ref, ("prepared", M))
                assert_gemm_close(o_rm[mi, ni], ref, ("row-major", M))
                first[M] = (o, o_rm)
            else:
                assert np.array_equal(o, first[M][0]), M
                assert np.array_equal(o_rm, first[M][1]), M
    torch.cuda.synchronize()
    for w in (ws, ws_rm):
        head = w.buf[:256].cpu().numpy()
        assert not head.any(), "arrival counters left nonzero"


def test_mxfp4_rejects_small_workspace():
    d = synth.down_proj()
    x8, s = _acts(16, d["K"], 1)
    need = w4.gemm_workspace_bytes(16, d["N"], d["K"])
    assert need > 0
    small = torch.zeros(need // 2 // 256 * 256, dtype=torch.uint8, device="cuda")
    lib = w4.lib()
    import ctypes
    dx, ds = dev_u8(x8), dev_f32(s)
    dw, de = dev_u8(d["w_packed"]), dev_u8(d["w_e8m0"])
    out = torch.empty((16, d["N"]), dtype=torch.bfloat16, device="cuda")
    st = lib.w4a8_mxfp4_gemm(ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(ds.data_ptr()),
                             ctypes.c_void_p(dw.data_ptr()), ctypes.c_void_p(de.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()), 16, d["N"], d["K"],
                             ctypes.c_void_p(small.data_ptr()), small.numel(), None)
    assert st == w4.binding.ERR_WORKSPACE


# ---------------------------------------------------------------------------
# int4 group-128 symmetric
# ---------------------------------------------------------------------------

def _int4_case(name, q, M, seed, full=False, n_samples=4096):
    N, K = q["N"], q["K"]
    say("int4 prepare", name, (N, K))
    nk = w4.int4g128_prepare(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]))
    ref_nk, bad = oracle.int4_prepare(q["qweight_kn"], q["qzeros"], N, K)
    assert bad == 0
    torch.cuda.synchronize()
    assert np.array_equal(nk.cpu().numpy(), ref_nk), name
    x8, s = _acts(M, K, seed)
    say("int4 gemm", name, (M, N, K))
    out = host_bf16_as_f64(w4.int4g128_gemm(dev_u8(x8), dev_f32(s), nk, dev_f16(q["scales"])))
    if M > 64:
        # above the decode band each call repacks into fragment order and runs
        # the prepared tile kernel: the prepared entry point's value, bit for bit
        pw = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))
        assert np.array_equal(out, host_bf16_as_f64(w4.int4g128_gemm_prepared(dev_u8(x8), dev_f32(s), pw))), name
    if full:
        ref = oracle.int4_gemm(x8, s, ref_nk, q["scales"])
        assert_gemm_close(out, ref, name)
    else:
        mi, ni = _sample_idx(M, N, n_samples, seed if isinstance(seed, int) else sum(seed))
        ref = oracle.int4_gemm(x8, s, ref_nk, q["scales"], mi=mi, ni=ni)
        assert_gemm_close(out[mi, ni], ref, name)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (4, 256, 512), (17, 136, 384), (64, 520, 1024),
                                   (65, 64, 256), (130, 200, 640)])
def test_int4_ragged(M, N, K):
    _int4_case(f"int4 {M}x{N}x{K}", synth.int4_random(N, K, seed=(N, K)), M, (M, K), full=True)


@pytest.mark.parametrize("M", [1, 64, 2048])
def test_int4_full_size(M):
    _int4_case(f"int4 I M={M}", synth.int4(), M, (4, M), full=M <= 64)


def test_int4_prepare_rejects_asymmetric_zeros():
    q = synth.int4_random(64, 256, seed=1)
    qz = q["qzeros"].copy()
    qz.view(np.uint32)[1, 3] = 0x77777778
    say("int4 prepare asymmetric")
    with pytest.raises(ValueError):
        w4.int4g128_prepare(dev_i32(q["qweight_kn"]), dev_i32(qz))


# ---------------------------------------------------------------------------
# MXFP4 weights in fragment order (prepared): split-K decode kernel for
# M <= 32, tiled kernel (64/128/256-row tiles) above
# ---------------------------------------------------------------------------

def _unprepare(wt, st, N, K):
    """Invert the documented fragment order on the host (layout check)."""
    tiles, steps = (N + 15) // 16, K // 128
    c_pad = (steps + 3) // 4
    w = wt.reshape(tiles, 4 * c_pad, 4, 16, 16)          # t, s, g, n, 16 bytes
    w = w.transpose(0, 3, 1, 2, 4).reshape(tiles * 16, 4 * c_pad * 64)[:N, : K // 2]
    sc = st.reshape(tiles, c_pad, 4, 16, 4)              # t, c, g, n, u
    sc = sc.transpose(0, 3, 1, 4, 2).reshape(tiles * 16, c_pad * 16)[:N, : K // 32]
    return w, sc


@pytest.mark.parametrize("N,K", [(64, 128), (100, 640), (5120, 17408), (34816, 5120)])
def test_prepare_layout_round_trip(N, K):
    w = synth.mxfp4_random(N, K, seed=(N, K))
    say("prepare", (N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    torch.cuda.synchronize()
    wt, st = pw.w.cpu().numpy(), pw.s.cpu().numpy()
    back_w, back_s = _unprepare(wt, st, N, K)
    assert np.array_equal(back_w, w["w_packed"]) and np.array_equal(back_s, w["w_e8m0"])
    # padding rows / steps: zero codes, e8m0 127
    tiles, c_pad = (N + 15) // 16, (K // 128 + 3) // 4
    full_w = wt.reshape(tiles, 4 * c_pad, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(tiles * 16, -1)
    assert (full_w[N:] == 0).all() and (full_w[:, K // 2:] == 0).all()
    full_s = st.reshape(tiles, c_pad, 4, 16, 4).transpose(0, 3, 1, 4, 2).reshape(tiles * 16, -1)
    assert (full_s[N:] == 127).all() and (full_s[:, K // 32:] == 127).all()


PREPARED = [(1, 64, 128), (1, 300, 640), (3, 100, 1152), (8, 257, 1024), (16, 1000, 4096),
            (17, 130, 512), (32, 512, 2048), (1, 6000, 2560)]


@pytest.mark.parametrize("M,N,K", PREPARED)
def test_mxfp4_prepared_ragged(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 1))
    x8, s = _acts(M, K, (M, K, 1), spread=10.0)
    say("prepared gemm", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"])
    assert_gemm_close(got, ref, (M, N, K))


@pytest.fixture(scope="module")
def gate_up_prepared(gate_up_mx):
    wp, we = gate_up_mx[:2]
    return w4.mxfp4_prepare(dev_u8(wp), dev_u8(we))


@pytest.fixture(scope="module")
def down_proj_prepared():
    d = synth.down_proj()
    return d, w4.mxfp4_prepare(dev_u8(d["w_packed"]), dev_u8(d["w_e8m0"]))


def _prepared_full_size(name, key, x8, s, pw, wp, we):
    say("prepared full-size", name, (x8.shape[0], pw.N, x8.shape[1]))
    dx, ds = dev_u8(x8), dev_f32(s)
    o1 = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    o2 = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    assert np.array_equal(o1, o2), (name, "not deterministic")
    assert_gemm_close(o1, _full_ref(key, x8, s, wp, we), name)


# every decode-band route on the gate_up layer: the split-K decode kernel (M up
# to 15, one launch; M = 16 with K split), the 64-row tiles above
@pytest.mark.parametrize("M", [1, 8, 12, 15, 16, 32, 64])
def test_mxfp4_prepared_gate_up(gate_up_mx, gate_up_prepared, M):
    x8, s = _acts(M, synth.HIDDEN, (1, M), spread=10.0)
    _prepared_full_size(f"gate_up M={M}", ("gate_up", M), x8, s, gate_up_prepared, *gate_up_mx[:2])


@pytest.mark.parametrize("M", [1, 16, 48, 64])
def test_mxfp4_prepared_down_proj(down_proj_prepared, M):
    d, pw = down_proj_prepared
    x8, s = _acts(M, synth.INTERMEDIATE, (2, M))
    _prepared_full_size(f"down_proj M={M}", ("down_proj", M), x8, s, pw, d["w_packed"], d["w_e8m0"])


# tiled band: every tile height, ragged M and N, K of one, two and three steps
# (the three-stage copy ring), an N that is not a multiple of 4 (scalar stores)
PREPARED_TILED = [(33, 64, 128), (64, 300, 256), (65, 257, 384), (100, 1000, 1152),
                  (128, 130, 4096), (129, 512, 640), (256, 1026, 2048), (300, 100, 1280),
                  (513, 600, 768)]


@pytest.mark.parametrize("M,N,K", PREPARED_TILED)
def test_mxfp4_prepared_tiled_ragged(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 2))
    x8, s = _acts(M, K, (M, K, 2), spread=10.0)
    say("prepared tiled gemm", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"])
    assert_gemm_close(got, ref, (M, N, K))


@pytest.mark.parametrize("M", [2048, 4096])
def test_mxfp4_prepared_tiled_gate_up(gate_up_mx, gate_up_prepared, M):
    x8, s = _acts(M, synth.HIDDEN, (3, M), spread=10.0)
    wp, we = gate_up_mx[:2]
    say("prepared tiled gate_up", M)
    dx, ds = dev_u8(x8), dev_f32(s)
    o1 = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, gate_up_prepared))
    o2 = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, gate_up_prepared))
    assert np.array_equal(o1, o2)
    mi, ni = _sample_idx(M, wp.shape[0], 16384, M + 11)
    assert_gemm_close(o1[mi, ni], oracle.mxfp4_gemm(x8, s, wp, we, mi=mi, ni=ni), M)


def test_mxfp4_prepared_tiled_down_proj(down_proj_prepared):
    d, pw = down_proj_prepared
    M = 4096
    x8, s = _acts(M, synth.INTERMEDIATE, (4, M))
    say("prepared tiled down_proj", M)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    mi, ni = _sample_idx(M, d["N"], 8192, 5)
    ref = oracle.mxfp4_gemm(x8, s, d["w_packed"], d["w_e8m0"], mi=mi, ni=ni)
    assert_gemm_close(got[mi, ni], ref, M)


# wide layers: the split-K decode kernel up to M = 16 while the activation
# slice of all of K fits LDS (four K parts when only two workgroups fit), the
# tiled kernel (256-wide tiles at every tile height) above: sampled outputs
# against the oracle
@pytest.mark.parametrize("M,N,K", [(13, 65600, 384), (16, 33000, 2560), (17, 33000, 384), (40, 65600, 256),
                                   (100, 65600, 384), (300, 33000, 384)])
def test_mxfp4_prepared_tiled_wide(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 3))
    x8, s = _acts(M, K, (M, K, 3), spread=10.0)
    say("prepared tiled wide", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    g = np.random.default_rng(M + N)
    mi = np.concatenate([np.arange(M), g.integers(0, M, 8192), np.full(64, M - 1)])
    ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, 8192), N - 1 - np.arange(64)])
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni)
    assert_gemm_close(got[mi, ni], ref, (M, N, K))


# narrow layers at 9 <= M <= 40: the register-streamed tiles (one to three
# 16-row activation tiles, eight waves per workgroup, K split across
# workgroups with fp32 partials and the reduction kernel): ragged N (a
# partial last tile, N not a multiple of 4), K of one step, K not a multiple
# of 512 (a padded last step), one split and several
DTILE = [(9, 64, 128), (16, 1000, 4096), (17, 130, 512), (24, 600, 1152), (32, 512, 2048),
         (33, 301, 3200), (40, 2000, 2048), (40, 1026, 640), (16, 5120, 17408)]


@pytest.mark.parametrize("M,N,K", DTILE)
def test_mxfp4_prepared_register_tiles(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 8))
    x8, s = _acts(M, K, (M, K, 8), spread=10.0)
    say("prepared register tiles", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    again = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, again)
    assert_gemm_close(got, oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"]), (M, N, K))


# spread tiles (wide MXFP4 layers, 2 <= M <= 64): every activation-tile
# count, ragged N (a partial last tile; N % 4 != 0 takes the scalar stores),
# padded K steps (K / 128 not a multiple of 4), workgroups of 8 and 9 tiles
# (1 and 2 per wave), through the default route and with each ring depth and
# e8m0 loading
SPREAD = [(2, 24576, 256), (9, 25001, 640), (16, 24600, 1152), (17, 30000, 512), (33, 24584, 384),
          (48, 26002, 256), (64, 24576, 512), (64, 34816, 5120)]


@pytest.mark.parametrize("M,N,K", SPREAD)
def test_mxfp4_prepared_spread(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 10))
    x8, s = _acts(M, K, (M, K, 10), spread=10.0)
    say("prepared spread tiles", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    s_pad = 4 * ((K // 128 + 3) // 4)
    # ring depth 4 and 8 with the e8m0 dwords per step, 4 with them per chunk (+100)
    for depth in (4, 8, 104):
        if depth in (8, 104) and s_pad % 8:
            with pytest.raises(ValueError):
                w4.decode_with_plan(dx, ds, pw.w, pw.s, -200, 0, depth, kind="prepared", N=N)
            continue
        forced = host_bf16_as_f64(w4.decode_with_plan(dx, ds, pw.w, pw.s, -200, 0, depth, kind="prepared", N=N))
        # the same products in the same order: bit-identical at either depth
        assert np.array_equal(forced, got), depth
    if M * N <= 64 * 26002:
        ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"])
        assert_gemm_close(got, ref, (M, N, K))
    else:
        mi, ni = _sample_idx(M, N, 8192, M + N)
        ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni)
        assert_gemm_close(got[mi, ni], ref, (M, N, K))


# layers wider than the spread tiles take (more than 2 x 8 tiles per
# workgroup) at 9 <= M <= 32 whose activation slice fits one workgroup's LDS:
# the split-K decode kernel with 16 tiles per workgroup (ragged N, a partial
# last group, K not a multiple of 512)
@pytest.mark.parametrize("M,N,K", [(9, 66000, 640), (24, 65600, 1152), (31, 70000, 4736), (32, 66008, 256)])
def test_mxfp4_prepared_wide_sixteen(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 9))
    x8, s = _acts(M, K, (M, K, 9), spread=10.0)
    say("prepared wide sixteen", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    mi, ni = _sample_idx(M, N, 8192, M + N)
    assert_gemm_close(got[mi, ni], oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni), (M, N, K))


# 256 x 256 tiles whose count leaves the last round part-empty: the leading
# columns on whole rounds, the tail columns on narrower tiles in a second
# launch (128 x 128 at M = 2048; 256 x 128 at M = 4096, here with ragged M and
# a ragged N that takes the scalar stores).  Every output is still one tile's
# full-K sum in step order: bit-identical to the single launch (the explicit
# tiled plan, which never splits the columns), and checked on a sample
# against the oracle.
@pytest.mark.parametrize("M,N,K", [(2048, 34816, 256), (4000, 34810, 384)])
def test_mxfp4_prepared_tail_columns(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 12))
    x8, s = _acts(M, K, (M, K, 12), spread=10.0)
    say("prepared tiled tail columns", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    whole = host_bf16_as_f64(w4.decode_with_plan(dx, ds, pw.w, pw.s, -100, 0, 1, kind="prepared", N=N))
    assert np.array_equal(got, whole)
    mi, ni = _sample_idx(M, N, 8192, M + N)
    # the tail columns in every sample
    mi = np.concatenate([mi, np.arange(M)[:: max(1, M // 512)]])
    ni = np.concatenate([ni, N - 1 - np.arange(len(mi) - len(ni)) % 2048])
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni)
    assert_gemm_close(got[mi, ni], ref, (M, N, K))


# narrow layers at 41 <= M <= 64: 64-row tiles 128 wide, K split across
# workgroups (fp32 partials + reduction) when long
@pytest.mark.parametrize("M,N,K", [(33, 16, 1152), (64, 200, 1024), (40, 2000, 2048), (48, 1000, 4096),
                                   (57, 301, 3200)])
def test_mxfp4_prepared_narrow_mid(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 4))
    x8, s = _acts(M, K, (M, K, 4), spread=10.0)
    say("prepared narrow mid", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    again = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, again)
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"])
    assert_gemm_close(got, ref, (M, N, K))


# K split across workgroups (few tiles on a long K): ragged N (scalar partial
# stores), and the full-size narrow layer at a few hundred rows
@pytest.mark.parametrize("M,N,K", [(100, 1002, 4096), (200, 520, 3072), (40, 20000, 4096)])
def test_mxfp4_prepared_tiled_split_ragged(M, N, K):
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 6))
    x8, s = _acts(M, K, (M, K, 6), spread=10.0)
    say("prepared tiled split", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    again = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, again)
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"])
    assert_gemm_close(got, ref, (M, N, K))


@pytest.mark.parametrize("M", [128, 512])
def test_mxfp4_prepared_tiled_split_down_proj(down_proj_prepared, M):
    d, pw = down_proj_prepared
    x8, s = _acts(M, synth.INTERMEDIATE, (7, M))
    say("prepared tiled split down_proj", M)
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    mi, ni = _sample_idx(M, d["N"], 4096, M + 13)
    ref = oracle.mxfp4_gemm(x8, s, d["w_packed"], d["w_e8m0"], mi=mi, ni=ni)
    assert_gemm_close(got[mi, ni], ref, M)


def test_mxfp4_prepared_tiled_tall():
    # 256-row tiles (one round of 137 of them beats two rounds of 128-row
    # tiles): ragged M, an N that is not a multiple of 4 (scalar stores),
    # sampled outputs including the last row and column
    M, N, K = 200, 34818, 384
    w = synth.mxfp4_random(N, K, seed=(M, N, K, 5))
    x8, s = _acts(M, K, (M, K, 5), spread=10.0)
    say("prepared tiled tall", (M, N, K))
    pw = w4.mxfp4_prepare(dev_u8(w["w_packed"]), dev_u8(w["w_e8m0"]))
    got = host_bf16_as_f64(w4.mxfp4_gemm_prepared(dev_u8(x8), dev_f32(s), pw))
    g = np.random.default_rng(9)
    mi = np.concatenate([np.arange(M), g.integers(0, M, 8192), np.full(64, M - 1)])
    ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, 8192), N - 1 - np.arange(64)])
    ref = oracle.mxfp4_gemm(x8, s, w["w_packed"], w["w_e8m0"], mi=mi, ni=ni)
    assert_gemm_close(got[mi, ni], ref, (M, N, K))


# ---------------------------------------------------------------------------
# int4 g128 weights in fragment order: the same four kernels as the prepared
# MXFP4 weights, the codes widened to e4m3 (c - 8) in registers
# ---------------------------------------------------------------------------

def _unprepare_int4(wt, st, N, K):
    """Invert the documented int4 fragment order on the host: -> qweight [N_pad,
    K_pad/8] words (transposed checkpoint layout) and fp16 scales [N_pad, K_pad/128]."""
    tiles, steps = (N + 15) // 16, K // 128
    s4 = 4 * ((steps + 3) // 4)
    w = wt.view(np.uint32).reshape(tiles, s4, 4, 16, 4)           # t, s, g, n, word
    w = w.transpose(0, 3, 1, 2, 4).reshape(tiles * 16, s4 * 16)     # word 16s + 4g + i
    sc = st.view(np.uint16).reshape(tiles, s4 // 4, 4, 4, 4)     # t, chunk, n / 4, step, n % 4
    sc = sc.transpose(0, 2, 4, 1, 3).reshape(tiles * 16, s4)
    return w, sc


@pytest.mark.parametrize("N,K", [(64, 128), (104, 640), (5120, 17408)])
def test_int4_prepare_fragments_layout(N, K):
    q = synth.int4_random(N, K, seed=(N, K, 7))
    say("int4 prepare fragments", (N, K))
    pw = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]),
                                       dev_f16(q["scales"]))
    torch.cuda.synchronize()
    w, sc = _unprepare_int4(pw.w.cpu().numpy(), pw.s.cpu().numpy(), N, K)
    assert np.array_equal(w[:N, :K // 8], q["qweight_kn"].view(np.uint32).T)
    assert np.array_equal(sc[:N, :K // 128], q["scales"].T)
    # padding: code 8 (value 0) and scale 0
    assert (w[N:] == 0x88888888).all() and (w[:, K // 8:] == 0x88888888).all()
    assert (sc[N:] == 0).all() and (sc[:, K // 128:] == 0).all()


def _int4_prepared_case(name, q, M, seed, full=False, n_samples=4096, spread=1.0):
    N, K = q["N"], q["K"]
    ref_nk, bad = oracle.int4_prepare(q["qweight_kn"], q["qzeros"], N, K)
    assert bad == 0
    say("int4 prepared", name, (M, N, K))
    pw = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]),
                                       dev_f16(q["scales"]))
    x8, s = _acts(M, K, seed, spread=spread)
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.int4g128_gemm_prepared(dx, ds, pw))
    again = host_bf16_as_f64(w4.int4g128_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, again), name
    if full:
        ref = oracle.int4_gemm(x8, s, ref_nk, q["scales"])
        sel = got
    else:
        mi, ni = _sample_idx(M, N, n_samples, seed if isinstance(seed, int) else sum(seed))
        ref = oracle.int4_gemm(x8, s, ref_nk, q["scales"], mi=mi, ni=ni)
        sel = got[mi, ni]
    assert_gemm_close(sel, ref, name)


# every route: split-K decode (M <= 32), tiled 64/128/256-row tiles with 128-
# and 256-wide columns
INT4_PREPARED = [(1, 64, 128), (3, 136, 1152), (17, 520, 1024), (32, 1000, 4096),
                 (33, 16, 1152), (48, 1000, 4096), (64, 200, 1024),
                 (65, 264, 384), (100, 1000, 1152), (129, 512, 640), (256, 1032, 2048),
                 (513, 600, 768), (48, 20000, 4096)]


@pytest.mark.parametrize("M,N,K", INT4_PREPARED)
def test_int4_prepared_ragged(M, N, K):
    _int4_prepared_case(f"{M}x{N}x{K}", synth.int4_random(N, K, seed=(M, N, K, 8)), M, (M, K, 8),
                        full=True, spread=10.0)


# wide layers: the spread tiles (9 <= M <= 64 where at most two 16-row tiles
# fall to a wave: N = 34816), else split-K decode (M <= 32; one and two 16-row
# activation tiles) and tiled (64/128/256-row tiles; N = 65600)
@pytest.mark.parametrize("M,N,K", [(5, 65600, 256), (13, 34816, 5120), (20, 65600, 384), (32, 34816, 5120),
                                   (33, 34816, 640), (40, 65600, 256),
                                   (300, 33000, 384), (600, 45064, 256)])
def test_int4_prepared_wide(M, N, K):
    _int4_prepared_case(f"wide {M}x{N}x{K}", synth.int4_random(N, K, seed=(M, N, K, 9)), M,
                        (M, K, 9), n_samples=8192)


# the spread tiles for symmetric int4 (above 8 rows): one to four 16-row activation tiles with
# ragged M, one or two weight tiles per wave, output rows stored by the
# products' lanes (N not a multiple of 16) or assembled, K ending inside a
# 4-step chunk, and an odd number of chunks, where the last trip of 8 steps
# runs past the padded steps with zero activation codes: after padding steps
# (K = 1152) and after a real step (K = 512, 1536)
INT4_SPREAD = [(9, 24576, 640), (17, 24600, 896), (33, 30000, 2048), (64, 65536, 512), (47, 40000, 5120),
               (40, 24576, 1152), (24, 24576, 1536), (12, 30000, 512), (64, 24600, 4608), (10, 24576, 128),
               (50, 24576, 256)]


@pytest.mark.parametrize("M,N,K", INT4_SPREAD)
def test_int4_prepared_spread(M, N, K):
    _int4_prepared_case(f"spread {M}x{N}x{K}", synth.int4_random(N, K, seed=(M, N, K, 12)), M,
                        (M, K, 12), full=M * N * K <= 2 ** 31, n_samples=8192, spread=10.0)


def test_int4_linear_spread():
    # the linear on bf16 rows through the spread tiles (quant kernel, then the
    # int4 spread tiles) against the quant and GEMM entry points called apart
    N, K, M = 34816, 1024, 24
    q = synth.int4_random(N, K, seed=(N, K, 14))
    pw = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))
    xb = torch.from_numpy(synth.acts(M, K, seed=(14, M)).view(np.int16)).view(torch.bfloat16).cuda()
    say("int4 linear spread", (M, N, K))
    x8, xs = w4.quant_act_fp8_per_token(xb)
    ref = host_bf16_as_f64(w4.int4g128_gemm_prepared(x8, xs, pw))
    got = host_bf16_as_f64(w4.int4g128_linear_prepared(xb, pw)[0])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M", [1, 16, 64, 128, 512, 2048])
def test_int4_prepared_full_size(M):
    _int4_prepared_case(f"I M={M}", synth.int4(), M, (10, M), full=M <= 64)


def test_int4_prepare_fragments_rejects_asymmetric_zeros():
    q = synth.int4_random(64, 256, seed=2)
    qz = q["qzeros"].copy()
    qz.view(np.uint32)[0, 5] = 0x77777770
    say("int4 prepare fragments asymmetric")
    with pytest.raises(ValueError):
        w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(qz), dev_f16(q["scales"]))
