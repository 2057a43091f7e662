"""Pins for the oracle's MXFP4 block encoder and mse rule (CPU only).

Page: "radiance_nvfp4.py" -- _encode_blocks, quant_mxfp4 (mse trial of the
no-clip exponent and one binade finer, sign rule for negative zero, packing
with the low nibble first, e8m0 = e + 127).

Independent checks: blocks already on the grid (zero error, same exponent under
every rule), the all-zero block, brute-force exponent search with the squared
error recomputed in fp64 by a separate vectorised route, packing of distinct
codes at even and odd positions, and per-block range invariants.
"""
import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_idx(a):
    """argmin |a - GRID| with even-index ties, vectorised, fp64."""
    a = np.minimum(np.abs(a), 6.0)
    d = np.abs(a[..., None] - GRID)
    best = d.min(-1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even index
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1))
    return pick


def _err64(w, e):
    """Squared error of encoding block(s) w at exponent e, in fp64."""
    w = np.asarray(w, np.float64)
    s = np.ldexp(1.0, e)
    idx = _nearest_idx(w / s)
    q = GRID[idx] * np.sign(w) * s
    return ((q - w) ** 2).sum(-1), idx


def test_grid_aligned_block_is_lossless(orc):
    g = np.random.default_rng(1)
    for e in [-20, -7, 0, 3, 50]:
        for _ in range(20):
            idx = g.integers(0, 8, 32)
            idx[g.integers(0, 32)] = 7           # block max is exactly 6 * 2^e
            sgn = np.where(g.random(32) < 0.5, -1.0, 1.0)
            w = (GRID[idx] * sgn * 2.0 ** e).astype(np.float32)
            for mode in ("ocp", "noclip", "mse"):
                ee, code, err = orc.quant_block(w, mode)
                assert ee == e and err == 0.0, (mode, e)
                expect = idx | np.where((sgn < 0) & (idx > 0), 8, 0)
                assert np.array_equal(code, expect)


def test_all_zero_and_negative_zero(orc):
    z = np.zeros(32, np.float32)
    for mode in ("ocp", "noclip", "mse"):
        e, code, err = orc.quant_block(z, mode)
        assert e == 0 and err == 0 and not code.any()
    w = np.zeros(32, np.float32)
    w[0] = -0.0
    w[1] = 6.0
    w[2] = -1e-3         # rounds to index 0 at e = 0: must stay code 0, not 8
    w[3] = -6.0
    e, code, err = orc.quant_block(w, "noclip")
    assert e == 0
    assert code[0] == 0 and code[2] == 0 and code[1] == 7 and code[3] == 15
    assert 8 not in code


def test_mse_choice_brute_force(orc):
    g = np.random.default_rng(2)
    n_checked = n_diff_global = 0
    blocks = []
    for _ in range(3000):
        kind = g.integers(0, 4)
        if kind == 0:
            w = g.standard_normal(32)
        elif kind == 1:
            w = g.laplace(size=32)
        elif kind == 2:
            w = g.uniform(-1, 1, 32)
        else:                                    # one outlier over a small bulk
            w = g.standard_normal(32) * 0.05
            w[g.integers(0, 32)] = g.uniform(2, 6) * (1 if g.random() < 0.5 else -1)
        w = (w * 2.0 ** g.integers(-30, 30)).astype(np.float32)
        blocks.append(w)
    for w in blocks:
        e, code, err = orc.quant_block(w, "mse")
        e0 = orc.block_exponent(float(np.abs(w).max()), "noclip")
        assert e in (e0, e0 - 1)
        r0, _ = _err64(w, e0)
        r1, _ = _err64(w, e0 - 1)
        chosen = r1 if e == e0 - 1 else r0
        assert abs(float(err) - chosen) <= 1e-5 * chosen + 1e-45
        if abs(r0 - r1) > 1e-5 * max(r0, r1):
            n_checked += 1
            assert (e == e0 - 1) == (r1 < r0)
        errs = {k: _err64(w, k)[0] for k in range(e0 - 3, e0 + 3)}
        if min(errs, key=errs.get) not in (e0, e0 - 1):
            n_diff_global += 1
        # the chosen codes reproduce the chosen exponent's nearest indices
        _, idx = _err64(w, e)
        assert np.array_equal(code & 7, idx)
    assert n_checked > 2900
    print(f"mse: global argmin over e0-3..e0+2 outside the two candidates in "
          f"{n_diff_global}/{len(blocks)} blocks")


def test_mse_near_tie_keeps_noclip(orc):
    # A block whose two candidate errors are exactly equal: values midway in a
    # way that mirrors between e0 and e0-1 is hard to build in general; the
    # page's strict comparison is checked on blocks with zero error for both.
    w = np.zeros(32, np.float32)
    w[0] = 3.0            # e0 (noclip) = -1: 3 / 2^-1 = 6 exact; e0-1: 12 -> clips
    e, code, err = orc.quant_block(w, "mse")
    assert e == -1 and err == 0.0
    w[0] = 2.0            # noclip e0 = -1 (2 <= 3), finer e = -2 gives 8 -> clips to 6: worse
    e, _, _ = orc.quant_block(w, "mse")
    assert e == -1


def test_packing_low_nibble_even(orc):
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 6.0         # code 7 at k = 0
    w[0, 1] = -1.0        # code 10 at k = 1
    w[0, 30] = 0.5        # code 1 at k = 30
    w[0, 31] = -6.0       # code 15 at k = 31
    packed, e8m0, _, _ = orc.quant_mxfp4(w, "noclip")
    assert e8m0[0, 0] == 127
    assert packed[0, 0] == (7 | (10 << 4))
    assert packed[0, 15] == (1 | (15 << 4))
    assert not packed[0, 1:15].any()


def test_block_range_invariants(orc):
    g = np.random.default_rng(3)
    w = (g.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    w[g.random(w.shape) < 0.002] *= 20
    for mode in ("ocp", "noclip", "mse"):
        packed, e8m0, es, ss = orc.quant_mxfp4(w, mode)
        e = e8m0.astype(np.int64) - 127
        amax = np.abs(w.reshape(64, 32, 32)).max(-1).astype(np.float64)
        r = amax / np.ldexp(1.0, e)
        if mode == "ocp":
            assert ((r >= 4) & (r < 8)).all()
        elif mode == "noclip":
            assert ((r > 3) & (r <= 6)).all()
        else:
            assert (((r > 3) & (r <= 6)) | ((r > 6) & (r <= 12))).all()
        lo = packed & 15
        hi = packed >> 4
        assert not (lo == 8).any() and not (hi == 8).any()
        assert (e8m0 != 255).all()
        # decoded error equals the encoder's own error sum
        d = orc.dequant_mxfp4(packed, e8m0).astype(np.float64)
        direct = ((d - w.astype(np.float64)) ** 2).sum()
        assert abs(direct - es) <= 1e-5 * direct
        assert abs(ss - (w.astype(np.float64) ** 2).sum()) <= 1e-9 * ss


def test_vectorised_independent_encoder_agrees(orc):
    """A separate vectorised fp64 encoder (exponent from frexp, nearest grid
    index, fp64 errors) agrees with the oracle on every block whose two mse
    candidate errors are not within 1e-5 of each other."""
    g = np.random.default_rng(4)
    w = (g.standard_normal((256, 2048)) * 0.02).astype(np.float32)
    w[g.random(w.shape) < 0.001] *= 20
    wb = w.reshape(-1, 32).astype(np.float64)
    amax = np.abs(wb).max(-1)
    m, x = np.frexp(amax)                    # amax = m 2^x, m in [0.5, 1)
    p = x - 1
    e_ocp = p - 2
    e_nc = np.where(2 * m <= 1.5, p - 2, p - 1)
    for mode, e_ref in (("ocp", e_ocp), ("noclip", e_nc), ("mse", None)):
        packed, e8m0, _, _ = orc.quant_mxfp4(w, mode)
        e = e8m0.reshape(-1).astype(np.int64) - 127
        if e_ref is not None:
            assert np.array_equal(e, e_ref)
        else:
            r0 = _err64(wb, e_nc[:, None])[0]
            r1 = _err64(wb, e_nc[:, None] - 1)[0]
            clear = np.abs(r0 - r1) > 1e-5 * np.maximum(r0, r1)
            want = np.where(r1 < r0, e_nc - 1, e_nc)
            assert np.array_equal(e[clear], want[clear])
            assert clear.mean() > 0.99
            e_ref = e
        _, idx = _err64(wb, e_ref[:, None])
        code = idx | np.where((wb < 0) & (idx > 0), 8, 0)
        pk = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8).reshape(packed.shape)
        assert np.array_equal(pk, packed), mode
