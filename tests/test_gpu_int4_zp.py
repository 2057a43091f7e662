"""GPU parity: int4 g128 with zero points (asymmetric), fragment order, against
the oracle; and, with every zero point 8, bit-identical to the symmetric
kernels (the zero term is then exactly zero)."""
import numpy as np
import pytest
import torch

import oracle
import w4a8_gemm_amd as w4
from gpu_util import assert_gemm_close, dev_f16, dev_f32, dev_i32, dev_u8, host_bf16_as_f64, say
from w4a8_gemm_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    w4.lib()


def _acts(M, K, seed, spread=1.0):
    bits = synth.acts(M, K, seed=seed, spread=spread)
    return oracle.quant_act_fp8(bits)


def _case(name, q, M, seed, sample=None, spread=10.0):
    N, K = q["N"], q["K"]
    say("int4 zp", name, (M, N, K))
    pw = w4.int4g128_zp_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))
    x8, s = _acts(M, K, seed, spread)
    dx, ds = dev_u8(x8), dev_f32(s)
    got = host_bf16_as_f64(w4.int4g128_zp_gemm_prepared(dx, ds, pw))
    again = host_bf16_as_f64(w4.int4g128_zp_gemm_prepared(dx, ds, pw))
    assert np.array_equal(got, again), name
    if sample is None:
        ref = oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"])
        assert_gemm_close(got, ref, name)
    else:
        g = np.random.default_rng(M + N)
        mi = np.concatenate([np.arange(M), g.integers(0, M, sample), np.full(64, M - 1)])
        ni = np.concatenate([g.integers(0, N, M), g.integers(0, N, sample), N - 1 - np.arange(64)])
        ref = oracle.int4_zp_gemm(x8, s, q["qweight_kn"], q["qzeros"], q["scales"], mi=mi, ni=ni)
        assert_gemm_close(got[mi, ni], ref, name)
    return pw, dx, ds, got


# decode kernel (one and two activation tiles, K split), tiled 64/128/256-row
# tiles with 128- and 256-wide columns, K split when tiles are few; ragged N
ZP = [(1, 64, 128), (3, 136, 1152), (17, 520, 1024), (32, 1000, 4096), (33, 16, 1152), (48, 1000, 4096),
      (65, 264, 384), (100, 1000, 1152), (129, 512, 640), (256, 1032, 2048), (513, 600, 768),
      (5, 20000, 512), (20, 20000, 384), (40, 20000, 256)]


@pytest.mark.parametrize("M,N,K", ZP)
def test_int4_zp_ragged(M, N, K):
    _case(f"{M}x{N}x{K}", synth.int4_zp(N, K, seed=(M, N, K, 41)), M, (M, K, 41))


# the spread tiles (wide layers, 9 <= M <= 64): one to four activation tiles,
# one or two weight tiles per wave, odd chunk counts (the last trip past the
# padded steps: after padding steps, K = 1152, and after a real step, K = 1536)
ZP_SPREAD = [(9, 24576, 640, None), (33, 30000, 2048, None), (64, 65536, 512, None), (40, 24576, 1152, None),
             (24, 24576, 1536, None), (64, 24600, 4608, 4096), (16, 24576, 128, None)]


@pytest.mark.parametrize("M,N,K,sample", ZP_SPREAD)
def test_int4_zp_spread(M, N, K, sample):
    _case(f"spread {M}x{N}x{K}", synth.int4_zp(N, K, seed=(M, N, K, 45)), M, (M, K, 45), sample=sample)


@pytest.mark.parametrize("M", [1, 16, 64, 2048])
def test_int4_zp_full_size(M):
    _case(f"zp M={M}", synth.int4_zp(), M, (42, M), sample=4096 if M > 64 else None)


@pytest.mark.parametrize("M,N,K", [(1, 136, 1152), (16, 1000, 4096), (64, 5120, 2048), (300, 600, 768),
                                   (24, 34816, 1024)])
def test_int4_zp_symmetric_zeros_equal_symmetric_kernels(M, N, K):
    # every zero point 8: the zero term adds exactly zero, so the outputs are
    # those of the symmetric kernels, bit for bit
    q = synth.int4_random(N, K, seed=(M, N, K, 43))
    pw, dx, ds, got = _case(f"sym {M}x{N}x{K}", q, M, (M, K, 43))
    ps = w4.int4g128_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))
    sym = host_bf16_as_f64(w4.int4g128_gemm_prepared(dx, ds, ps))
    assert np.array_equal(got, sym)


def test_int4_zp_prepared_records():
    # the records: scales of steps 0..3 x rows 0..15, then the bytes 16 - z,
    # both in lane-group order, then zero padding; rows past N: scale 0, z = 8
    N, K = 24, 640
    q = synth.int4_zp(N, K, seed=44)
    pw = w4.int4g128_zp_prepare_fragments(dev_i32(q["qweight_kn"]), dev_i32(q["qzeros"]), dev_f16(q["scales"]))
    st = pw.s.cpu().numpy()
    c_pad = (K // 128 + 3) // 4
    assert st.size == 2 * c_pad * 256
    z = np.stack([(q["qzeros"].view(np.uint32) >> (4 * j)) & 15 for j in range(8)], axis=2)
    z = z.reshape(K // 128, N).astype(np.int64) + 1
    for t in range(2):
        for c in range(c_pad):
            rec = st[(t * c_pad + c) * 256:(t * c_pad + c + 1) * 256]
            # lane-group order [row / 4][step][row % 4] -> [step][row]
            sc = rec[:128].view(np.uint16).reshape(4, 4, 4).transpose(1, 0, 2).reshape(4, 16)
            zb = rec[128:192].reshape(4, 4, 4).transpose(1, 0, 2).reshape(4, 16)
            assert (rec[192:] == 0).all()
            for u in range(4):
                s_ = 4 * c + u
                for r in range(16):
                    n = 16 * t + r
                    if n < N and s_ < K // 128:
                        assert sc[u, r] == q["scales"][s_, n] and zb[u, r] == 16 - z[s_, n]
                    else:
                        assert sc[u, r] == 0 and zb[u, r] == 8
