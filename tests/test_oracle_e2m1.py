"""Pins for the oracle's e2m1 index and block exponent (CPU only).

* e2m1_index: the page's worked tie cases (golden), and the page's own
  three-branch round-half-even form (torch.round on 2a, a, a/2) compared with
  the oracle's argmin definition over every fp32 in [2^-5, 8) plus samples
  outside ("radiance_nvfp4.py", e2m1_index).
* _block_exponent: positive normal fp32 amax in every binade (a mantissa
  lattice plus every value near a decision point) is checked against the
  ranges the page states for the two rules, [4, 8) for ocp and (3, 6] for
  noclip, which fix e uniquely; plus the clamp and zero cases
  ("radiance_nvfp4.py", _block_exponent).
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


def test_e2m1_ties_golden(orc):
    for a, idx in _rows("e2m1_ties.txt"):
        assert orc.e2m1_index(float(np.float32(a))) == int(idx), a


def _three_branch(a: np.ndarray) -> np.ndarray:
    """The page's docstring form: clamp to 6; rne(2a) below 2, rne(a)+2 below 4,
    rne(a/2)+4 otherwise (np.rint rounds half to even)."""
    a = np.minimum(a.astype(np.float64), 6.0)
    lo = np.rint(a * 2.0)
    mid = np.rint(a) + 2.0
    hi = np.rint(a * 0.5) + 4.0
    return np.where(a < 2.0, lo, np.where(a < 4.0, mid, hi)).astype(np.uint8)


def test_e2m1_index_exhaustive_central_range(orc):
    # every fp32 from 2^-5 up to (not including) 8: all seven decision points
    lo = np.float32(2.0 ** -5).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    step = 1 << 24
    for start in range(int(lo), int(hi), step):
        u = np.arange(start, min(start + step, int(hi)), dtype=np.uint32)
        a = u.view(np.float32)
        got = orc.e2m1_index_array(a)
        ref = _three_branch(a)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, [(float(a[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def test_e2m1_index_outside_central_range(orc):
    g = np.random.default_rng(7)
    small = np.concatenate([np.ldexp(g.uniform(0, 1, 100000), -g.integers(5, 150, 100000)),
                            [0.0, 2.0 ** -149, 2.0 ** -126]]).astype(np.float32)
    assert (orc.e2m1_index_array(small) == 0).all()
    big = np.concatenate([g.uniform(8, 1e6, 100000), [8.0, 3.0e38, np.inf]]).astype(np.float32)
    assert (orc.e2m1_index_array(big) == 7).all()


def test_e2m1_index_brute_force_eighths(orc):
    grid = np.array([float(v) for _, v in _rows("e2m1_grid.txt")])
    for k in range(0, 65):
        a = k / 8.0
        ac = min(a, 6.0)
        d = np.abs(ac - grid)
        cand = np.nonzero(d == d.min())[0]
        expect = [c for c in cand if c % 2 == 0][0] if len(cand) > 1 else cand[0]
        assert orc.e2m1_index(a) == expect, (a, expect)


def _ranges():
    r = {}
    for name, lo, hi, lc, hc in _rows("exponent_rules.txt"):
        r[name] = (float(lo), float(hi), lc == "1", hc == "1")
    return r


def _normal_fp32_sweep():
    """Every positive normal fp32 exponent, with mantissas on a 2^-15 lattice and
    every value within 256 ulps of each point where either rule can change
    (mantissa 1.0, 1.5 and just below 2.0)."""
    m = np.concatenate([np.arange(0, 1 << 23, 1 << 8),
                        np.arange(0, 256), np.arange((1 << 23) - 256, 1 << 23),
                        np.arange((1 << 22) - 256, (1 << 22) + 256)]).astype(np.uint32)
    m = np.unique(m)
    E = np.arange(1, 255, dtype=np.uint32)
    u = (E[:, None] << np.uint32(23)) | m[None, :]
    return u.ravel().view(np.float32)


def test_block_exponent_all_binades(orc):
    rng = _ranges()
    lo4, hi8, lc_o, hc_o = rng["ocp"]
    lo3, hi6, lc_n, hc_n = rng["noclip"]
    assert (lc_o, hc_o, lc_n, hc_n) == (True, False, False, True)
    emin = int(rng["clamp"][0])
    A = _normal_fp32_sweep()
    At = torch.from_numpy(A.astype(np.float64))
    for mode, (lo, hi) in (("ocp", (lo4, hi8)), ("noclip", (lo3, hi6))):
        e = torch.from_numpy(orc.block_exponent_array(A, mode)).to(torch.float64)
        low = torch.ldexp(torch.full_like(At, lo), e)
        high = torch.ldexp(torch.full_like(At, hi), e)
        if mode == "ocp":
            ok = (low <= At) & (At < high)
        else:
            ok = (low < At) & (At <= high)
        # where the unclamped exponent would fall below -127 the clamp applies
        clamped = e == emin
        ok = ok | (clamped & (At < high))
        bad = torch.nonzero(~ok).ravel()
        assert bad.numel() == 0, (mode, [float(A[i]) for i in bad[:5]])
        assert bool((e >= emin).all()) and bool((e <= 127).all())


def test_block_exponent_special_values(orc):
    for mode in ("ocp", "noclip"):
        assert orc.block_exponent(0.0, mode) == 0
        assert orc.block_exponent(2.0 ** -149, mode) == -127   # subnormal: page clamps to tiny
        assert orc.block_exponent(2.0 ** -127, mode) == -127
    assert orc.block_exponent(np.finfo(np.float32).max, "ocp") == 125
    assert orc.block_exponent(np.finfo(np.float32).max, "noclip") == 126
    assert orc.block_exponent(6.0, "noclip") == 0
    assert orc.block_exponent(float(np.nextafter(np.float32(6.0), np.float32(7.0))), "noclip") == 1
    assert orc.block_exponent(3.0000002, "noclip") == 0
    assert orc.block_exponent(3.0, "noclip") == -1
    assert orc.block_exponent(4.0, "ocp") == 0
    assert orc.block_exponent(float(np.nextafter(np.float32(4.0), np.float32(0.0))), "ocp") == -1
