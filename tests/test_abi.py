"""C ABI of libw4a8.so on the CPU (no GPU needed).

The library must load, export every function include/w4a8.h declares, and
reject bad arguments on the host before any device work: each call here fails
validation, so the (fake, aligned, never dereferenced) device pointers are
never touched.  Also pins the workspace-size function's contract.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

OK, INVALID, SHAPE, WORKSPACE, ASYM, HIP = range(6)
FAKE = 0x100000          # aligned stand-in for a device pointer (validation fails first)


@pytest.fixture(scope="module")
def L():
    from w4a8_gemm_amd import binding
    return binding.lib()


def _p(v=FAKE):
    return ctypes.c_void_p(v)


def test_exports_every_declared_function(L):
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(w4a8_[a-z0-9_]+)\s*\(", text)))
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    from w4a8_gemm_amd import binding
    assert binding.version().startswith("w4a8")
    for s in range(6):
        assert binding.status_string(s)


def _requant(L, packed=FAKE, scale=FAKE, rows=(64,), divs=(1.0,), n_parts=None, K=128, mode=2,
             row_chunk=0, out=FAKE, e8=FAKE, stats=None):
    pr = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    pd = (ctypes.c_float * max(len(divs), 1))(*divs)
    return L.w4a8_requant_nvfp4_to_mxfp4(_p(packed) if packed else None, _p(scale) if scale else None,
                                         pr, pd, len(rows) if n_parts is None else n_parts, K, mode,
                                         row_chunk, _p(out) if out else None, _p(e8) if e8 else None,
                                         _p(stats) if stats else None, None)


def test_requant_validation(L):
    assert _requant(L, packed=0) == INVALID
    assert _requant(L, out=0) == INVALID
    assert _requant(L, K=96 + 16) == SHAPE                       # K % 32
    assert _requant(L, mode=3) == INVALID
    assert _requant(L, n_parts=0) == INVALID
    assert _requant(L, row_chunk=-1) == INVALID
    assert _requant(L, divs=(0.0,)) == INVALID
    assert _requant(L, divs=(-1.0,)) == INVALID
    assert _requant(L, divs=(float("nan"),)) == INVALID
    assert _requant(L, divs=(float("inf"),)) == INVALID
    assert _requant(L, rows=(-5,)) == INVALID
    assert _requant(L, packed=FAKE + 8) == INVALID               # 16-byte alignment
    assert _requant(L, scale=FAKE + 1) == INVALID
    assert _requant(L, stats=FAKE + 4) == INVALID


def test_act_quant_validation(L):
    f = L.w4a8_quant_act_fp8_per_token
    assert f(None, 1, 8, 8, _p(), _p(), None) == INVALID
    assert f(_p(), 0, 8, 8, _p(), _p(), None) == INVALID
    assert f(_p(), 1, 0, 8, _p(), _p(), None) == INVALID
    assert f(_p(), 1, 8, 7, _p(), _p(), None) == SHAPE            # ldx < K
    assert f(_p(FAKE + 1), 1, 8, 8, _p(), _p(), None) == INVALID


def test_load_quant_validation(L):
    b = L.w4a8_quant_bf16_to_mxfp4
    f = L.w4a8_quant_fp8ch_to_mxfp4
    assert b(None, 4, 64, 2, _p(), _p(), None, None) == INVALID
    assert b(_p(), 4, 64, 3, _p(), _p(), None, None) == INVALID                 # bad mode
    assert b(_p(), -1, 64, 2, _p(), _p(), None, None) == INVALID
    assert b(_p(), 4, 48, 2, _p(), _p(), None, None) == SHAPE                   # K % 32
    assert b(_p(FAKE + 8), 4, 64, 2, _p(), _p(), None, None) == INVALID         # 16-byte aligned in
    assert b(_p(), 4, 64, 2, _p(FAKE + 8), _p(), None, None) == INVALID         # 16-byte aligned out
    assert b(_p(), 4, 64, 2, _p(), _p(), _p(FAKE + 4), None) == INVALID         # 8-byte aligned stats
    assert f(_p(), None, 4, 64, 2, _p(), _p(), None, None) == INVALID           # row scales required
    assert f(_p(), _p(FAKE + 2), 4, 64, 2, _p(), _p(), None, None) == INVALID
    assert f(_p(), _p(), 4, 96 + 16, 2, _p(), _p(), None, None) == SHAPE


def test_w4a4_validation(L):
    g = L.w4a8_w4a4_gemm_prepared
    assert g(None, _p(), _p(), _p(), _p(), 4, 64, 128, None, 0, None) == INVALID
    assert g(_p(), _p(FAKE + 2), _p(), _p(), _p(), 4, 64, 128, None, 0, None) == INVALID   # e8m0 4-byte aligned
    assert g(_p(), _p(), _p(), _p(FAKE + 2), _p(), 4, 64, 128, None, 0, None) == INVALID
    assert g(_p(), _p(), _p(), _p(), _p(), 4, 64, 96, None, 0, None) == SHAPE             # K % 128
    # a few tiles on a long K are split: the workspace is required and sized by kind 4
    need = L.w4a8_gemm_workspace_bytes(128, 5120, 17408, 4)
    assert need > 0
    assert g(_p(), _p(), _p(), _p(), _p(), 128, 5120, 17408, None, 0, None) == WORKSPACE
    assert L.w4a8_gemm_workspace_bytes(64, 5120, 17408, 4) <= need
    assert L.w4a8_gemm_workspace_bytes(4096, 34816, 5120, 4) == L.w4a8_gemm_workspace_bytes(128, 34816, 5120, 4)
    # decode-sized M on a narrow layer with a long K: the decode kernel splits
    # K in 4 (9 of the 34 four-step chunks per split), partials after the
    # 256-byte-rounded counter header of its 320 row tiles
    assert L.w4a8_gemm_workspace_bytes(32, 5120, 17408, 4) == 1280 + 4 * 32 * 5120 * 4
    assert g(_p(), _p(), _p(), _p(), _p(), 32, 5120, 17408, None, 0, None) == WORKSPACE
    assert L.w4a8_gemm_workspace_bytes(1, 34816, 5120, 4) == 0                  # one split, none needed


def test_gemm_validation(L):
    g = L.w4a8_mxfp4_gemm
    args = lambda **k: [_p(k.get("x", FAKE)) if k.get("x", FAKE) else None, _p(), _p(), _p(),
                        _p(k.get("out", FAKE)), k.get("M", 4), k.get("N", 64), k.get("K", 128),
                        None, 0, None]
    assert g(*args(x=0)) == INVALID
    assert g(*args(M=0)) == INVALID
    assert g(*args(K=100)) == SHAPE
    assert g(*args(out=FAKE + 2)) == INVALID
    # a decode shape that splits K needs a workspace
    need = L.w4a8_gemm_workspace_bytes(16, 5120, 17408, 0)
    assert need > 0
    a = args(M=16, N=5120, K=17408)
    assert g(*a) == WORKSPACE
    a[8], a[9] = _p(), need - 256
    assert g(*a) == WORKSPACE
    a[8], a[9] = _p(FAKE + 16), need
    assert g(*a) == WORKSPACE                                    # 256-byte alignment
    i = L.w4a8_int4g128_gemm
    assert i(_p(), _p(), _p(), _p(), _p(), 4, 60, 256, None, 0, None) == SHAPE   # N % 8
    assert i(_p(), _p(), _p(), _p(), _p(), 4, 64, 192, None, 0, None) == SHAPE   # K % 128
    p = L.w4a8_int4g128_prepare
    assert p(None, _p(), 64, 256, _p(), None) == INVALID
    assert p(_p(), _p(), 60, 256, _p(), None) == SHAPE
    assert p(_p(), _p(), 64, 200, _p(), None) == SHAPE
    pf = L.w4a8_int4g128_prepare_fragments
    assert pf(_p(), _p(), None, 64, 256, _p(), _p(), None) == INVALID
    assert pf(_p(), _p(), _p(), 60, 256, _p(), _p(), None) == SHAPE
    assert pf(_p(), _p(), _p(), 64, 200, _p(), _p(), None) == SHAPE
    assert pf(_p(), _p(), _p(), 64, 256, _p(FAKE + 8), _p(), None) == INVALID   # 16-byte aligned
    assert pf(_p(), _p(), _p(), 64, 256, _p(), _p(FAKE + 8), None) == INVALID   # 16-byte aligned
    ip = L.w4a8_int4g128_gemm_prepared
    assert ip(_p(), _p(), _p(), _p(), _p(), 4, 60, 256, None, 0, None) == SHAPE  # N % 8
    assert ip(_p(), _p(), _p(), _p(), _p(), 4, 64, 192, None, 0, None) == SHAPE  # K % 128
    assert ip(_p(), _p(), _p(), _p(FAKE + 4), _p(), 4, 64, 256, None, 0, None) == INVALID
    assert ip(_p(), _p(), _p(), None, _p(), 4, 64, 256, None, 0, None) == INVALID


def test_workspace_bytes_contract(L):
    wb = L.w4a8_gemm_workspace_bytes
    # prepared MXFP4 on a wide layer (the spread tiles): no workspace up to 16
    # rows; above, the linear's step-major copy of the codes, after the split-K
    # counters (one word per 16 rows, 256-byte rounded)
    up = lambda b: (b + 255) // 256 * 256
    Nw, Kw = 34816, 5120
    assert wb(1, Nw, Kw, 2) == 0 and wb(16, Nw, Kw, 2) == 0
    assert wb(17, Nw, Kw, 2) == up(((Nw + 15) // 16) * 4) + up(17 * Kw)
    assert wb(64, Nw, Kw, 2) == up(((Nw + 15) // 16) * 4) + up(64 * Kw)
    assert wb(0, 64, 128, 0) == 0
    assert wb(4, 64, 100, 0) == 0                                # K % 32
    assert wb(4, 60, 256, 1) == 0                                # int4 N % 8
    assert wb(4, 64, 128, 7) == 0                                # unknown kind
    # covers every smaller M
    prev = 0
    for m in (1, 2, 8, 16, 17, 32, 64, 65, 4096):
        cur = wb(m, 5120, 17408, 0)
        assert cur >= prev
        prev = cur
    # above 64 rows the plain-layout MXFP4 GEMM repacks its weight into the
    # workspace after the decode band's split-K counters (one per 16 rows,
    # 256-byte rounded): that and the two fragment-order buffers at least, and
    # exactly those plus the tile kernel's own split where none is needed
    N, K = 5120, 17408
    wbytes, sbytes = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.w4a8_mxfp4_prepared_bytes(N, K, ctypes.byref(wbytes), ctypes.byref(sbytes)) == 0
    up = lambda b: (b + 255) // 256 * 256
    repack = up(((N + 15) // 16) * 4) + up(wbytes.value) + up(sbytes.value)
    assert wb(4096, N, K, 0) >= repack and wb(4096, N, K, 0) > wb(64, N, K, 0)
    N2, K2 = 34816, 5120          # 256 x 256 tiles from 4096 rows on: no split at M_max; 128 rows: 136 tiles
    wb2, sb2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.w4a8_mxfp4_prepared_bytes(N2, K2, ctypes.byref(wb2), ctypes.byref(sb2)) == 0
    assert wb(128, N2, K2, 0) == up(((N2 + 15) // 16) * 4) + up(wb2.value) + up(sb2.value)
    # K % 128 != 0 keeps the row-major tile kernel: no repack
    assert wb(4096, 5120, 17440, 0) == wb(64, 5120, 17440, 0)


def test_prepared_tiled_split_workspace(L):
    """Few tiles on a long K: the tiled kernel splits K (fp32 partials), so a
    prepared GEMM above the decode band may need a workspace; sizing and the
    missing-workspace error are host-side."""
    N, K, M = 5120, 17408, 128
    # 128-row tiles, 128 wide (40 of them): at most one workgroup per CU ->
    # 6 splits of 24 steps; header of one counter per 16 rows, then [ks][M][N]
    header = (((N + 15) // 16) * 4 + 255) // 256 * 256
    want = header + 6 * M * N * 4
    for kind in (2, 3):
        assert L.w4a8_gemm_workspace_bytes(M, N, K, kind) == want
        assert L.w4a8_gemm_workspace_bytes(M + 64, N, K, kind) >= want
    # many tiles: no split, the decode band's need is all that remains (MXFP4);
    # int4 also splits K where fewer tiles than CUs leave some idle: 160
    # 256-row tiles at M = 2048 in three, 180 at M = 2304 in four (the largest
    # need up to M = 4096)
    assert L.w4a8_gemm_workspace_bytes(4096, N, K, 2) == L.w4a8_gemm_workspace_bytes(1024, N, K, 2)
    assert L.w4a8_gemm_workspace_bytes(2048, N, K, 3) == header + 3 * 2048 * N * 4
    assert L.w4a8_gemm_workspace_bytes(4096, N, K, 3) == header + 4 * 2304 * N * 4
    g = L.w4a8_mxfp4_gemm_prepared
    assert g(_p(), _p(), _p(), _p(), _p(), M, N, K, None, 0, None) == WORKSPACE
    assert g(_p(), _p(), _p(), _p(), _p(), M, N, K, _p(), want - 256, None) == WORKSPACE
    i = L.w4a8_int4g128_gemm_prepared
    assert i(_p(), _p(), _p(), _p(), _p(), M, N, K, None, 0, None) == WORKSPACE


def test_binding_rejects_mismatched_weight_sizes(L):
    """The ABI takes raw pointers, so the binding checks tensor sizes against
    N and K before a call (a flat prepared buffer must not be read as rows)."""
    from w4a8_gemm_amd import binding

    class Shape:
        def __init__(self, *shape):
            self.shape = shape

        def numel(self):
            n = 1
            for d in self.shape:
                n *= d
            return n

        def element_size(self):
            return 1

    N, K = 34816, 5120
    wb, sb = binding._size(), binding._size()
    assert binding.lib().w4a8_mxfp4_prepared_bytes(N, K, ctypes.byref(wb), ctypes.byref(sb)) == OK
    w, s = Shape(wb.value), Shape(sb.value)
    binding._check_weight_sizes("prepared", w, s, N, K)
    with pytest.raises(ValueError):
        binding._check_weight_sizes("prepared", w, s, wb.value, K)
    binding._check_weight_sizes("mxfp4", Shape(N, K // 2), Shape(N, K // 32), N, K)
    # int4 fragment order: 1 KiB per (16-row tile, 128-wide step), 128 B of fp16
    # scales per (tile, 4-step chunk); rows padded to 16, steps to 4
    N4, K4 = 5128, 17408 + 128
    assert binding.lib().w4a8_int4g128_prepared_bytes(N4, K4, ctypes.byref(wb), ctypes.byref(sb)) == OK
    tiles, chunks = (N4 + 15) // 16, (K4 // 128 + 3) // 4
    assert (wb.value, sb.value) == (tiles * chunks * 4096, tiles * chunks * 128)
    binding._check_weight_sizes("int4_prepared", Shape(wb.value), Shape(sb.value), N4, K4)
    with pytest.raises(ValueError):
        binding._check_weight_sizes("int4_prepared", Shape(wb.value), Shape(2 * sb.value), N4, K4)
    assert binding.lib().w4a8_int4g128_prepared_bytes(60, 256, ctypes.byref(wb), ctypes.byref(sb)) == SHAPE
    with pytest.raises(ValueError):
        binding._check_weight_sizes("mxfp4", Shape(N, K // 2), Shape(N, K // 16), N, K)
    with pytest.raises(ValueError):
        binding._check_weight_sizes("int4", Shape(N, K // 8), Shape(N, K // 128), N, K)


def test_linear_validation(L):
    for f in (L.w4a8_mxfp4_linear_prepared, L.w4a8_int4g128_linear_prepared):
        ok = lambda **k: [k.get("x", _p()), k.get("ldx", 256), _p(), _p(), _p(), 4, 64, k.get("K", 256),
                          k.get("x8", _p()), k.get("xs", _p()), None, 0, None]
        assert f(*ok(x=None)) == INVALID
        assert f(*ok(x=_p(FAKE + 1))) == INVALID                  # bf16 2-byte aligned
        assert f(*ok(ldx=128)) == SHAPE                           # ldx < K
        assert f(*ok(K=200, ldx=200)) == SHAPE                    # K % 128
        assert f(*ok(x8=None)) == INVALID                         # codes are an output
        assert f(*ok(x8=_p(FAKE + 8))) == INVALID                 # 16-byte aligned codes
        assert f(*ok(xs=_p(FAKE + 2))) == INVALID
    # the int4 form keeps N % 8
    a = [_p(), 256, _p(), _p(), _p(), 4, 60, 256, _p(), _p(), None, 0, None]
    assert L.w4a8_int4g128_linear_prepared(*a) == SHAPE


def test_int4_zp_validation(L):
    b, pf, g = L.w4a8_int4g128_zp_prepared_bytes, L.w4a8_int4g128_zp_prepare_fragments, L.w4a8_int4g128_zp_gemm_prepared
    import ctypes
    wb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert b(60, 256, ctypes.byref(wb), ctypes.byref(sb)) == SHAPE
    assert b(64, 256, ctypes.byref(wb), ctypes.byref(sb)) == 0
    assert sb.value == 4 * 1 * 256 and wb.value == 4 * 1 * 4 * 1024     # 4 tiles, 1 chunk
    assert pf(None, _p(), _p(), 64, 256, _p(), _p(), None) == INVALID
    assert pf(_p(), _p(), _p(), 64, 200, _p(), _p(), None) == SHAPE
    assert pf(_p(), _p(), _p(), 64, 256, _p(), _p(FAKE + 8), None) == INVALID   # 16-byte aligned records
    assert g(_p(), _p(), _p(), _p(), _p(), 4, 60, 256, None, 0, None) == SHAPE
    assert g(_p(), _p(), _p(), _p(FAKE + 8), _p(), 4, 64, 256, None, 0, None) == INVALID
    # the same routes and splits as the symmetric int4 kernels
    for M in (1, 16, 33, 128):
        assert L.w4a8_gemm_workspace_bytes(M, 5120, 17408, 5) == L.w4a8_gemm_workspace_bytes(M, 5120, 17408, 3)


def test_int5_validation(L):
    import ctypes
    b, pf, g = L.w4a8_int5g128_prepared_bytes, L.w4a8_int5g128_prepare_fragments, L.w4a8_int5g128_gemm_prepared
    wb, w5b, sb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert b(64, 200, ctypes.byref(wb), ctypes.byref(w5b), ctypes.byref(sb)) == SHAPE
    assert b(20, 640, ctypes.byref(wb), ctypes.byref(w5b), ctypes.byref(sb)) == 0
    # 2 tiles x 2 chunks: 4 KiB of codes, 1 KiB of fifth bits and one record per tile and chunk
    assert (wb.value, w5b.value, sb.value) == (2 * 2 * 4096, 2 * 2 * 1024, 2 * 2 * 256)
    assert pf(None, _p(), _p(), _p(), 64, 256, _p(), _p(), _p(), None) == INVALID
    assert pf(_p(), _p(), _p(), _p(), 64, 200, _p(), _p(), _p(), None) == SHAPE
    assert pf(_p(), _p(), _p(), _p(), 64, 256, _p(), _p(FAKE + 4), _p(), None) == INVALID
    assert g(_p(), _p(), _p(), None, _p(), _p(), 4, 64, 256, None, 0, None) == INVALID
    assert g(_p(), _p(), _p(), _p(), _p(), _p(), 4, 64, 200, None, 0, None) == SHAPE
    # M past 32 runs the tile kernel: the activation sums [K/512 chunks][M][4]
    # fp32 plus 4 KiB, rounded to 256 bytes (no K split at 9 steps), the most
    # at M_max; with a K split the partials come on top
    assert L.w4a8_gemm_workspace_bytes(300, 520, 1152, 6) == (3 * 300 * 16 + 4096 + 255) // 256 * 256
    assert L.w4a8_gemm_workspace_bytes(32, 5120, 17408, 6) > 0
    assert L.w4a8_gemm_workspace_bytes(64, 5120, 17408, 6) >= 34 * 64 * 16 + 4096 + 2 * 64 * 5120 * 4


def test_workspace_bytes_cover_every_smaller_call(L):
    """The size for M_max covers every call of m <= M_max rows: the function is
    non-decreasing in M_max for every prepared kind, also where the tile
    kernels split K beyond 32768 rows (int4 and int4 with zero points at 128-255
    tiles on a 256-wide layer, int5 at any M on a narrow one)."""
    wb = L.w4a8_gemm_workspace_bytes
    for kind in (2, 3, 4, 5, 6):
        for N, K in ((256, 8192), (5120, 17408), (34816, 5120)):
            prev = 0
            for m in sorted(set(range(1, 200)) | set(range(200, 70000, 977)) | {65536, 131072, 300000}):
                cur = wb(m, N, K, kind)
                assert cur >= prev, (kind, N, K, m, cur, prev)
                prev = cur
    # the cases a 32768-row cap missed: the need at M = 49138 (int4, N = 256)
    # and M = 40903 (int5) is inside the size for 65536 rows
    assert wb(65536, 256, 8192, 3) >= wb(49138, 256, 8192, 3) > 0
    assert wb(65536, 256, 8192, 6) >= wb(40903, 256, 8192, 6) > 0
