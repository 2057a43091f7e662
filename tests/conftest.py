import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def gate_tiny(orc):
    """Oracle MXFP4 (mse) of the tiny NVFP4 weight: (packed, e8m0)."""
    from w4a8_gemm_amd import synth
    t = synth.tiny()
    mp, me, _ = orc.requant_nvfp4_to_mxfp4(t["nv_packed"], t["nv_scale"], t["part_rows"],
                                          t["part_divisor"], mode="mse")
    return mp, me


@pytest.fixture(scope="session")
def gate_up_mx(orc):
    """Oracle MXFP4 (mse) of the merged gate_up NVFP4 weight: (packed, e8m0, stats)."""
    from w4a8_gemm_amd import synth
    g = synth.gate_up()
    return orc.requant_nvfp4_to_mxfp4(g["nv_packed"], g["nv_scale"], g["part_rows"],
                                      g["part_divisor"], mode="mse")
