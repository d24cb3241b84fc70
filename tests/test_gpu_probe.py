"""GPU check of the measurement support entry point sp24_probe_sclk: one record per wave, and values
inside what the hardware allows (an smfmac of 16x16x64 takes at least 16 cycles of issue; the shader
clock of an MI355X is at most 2.4 GHz)."""
import pytest
import torch

import structured_sparse_gemm_sp24_amd as sp
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def test_probe_sclk_plausible():
    require_gpu()
    say("sp24_probe_sclk")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    r = sp.sp24_probe_sclk(iters=200)
    assert r["waves"] == 4 * cus
    assert 300.0 < r["sclk_mhz"] < 2500.0, r
    assert 15.5 < r["cycles_per_smfmac"] < 200.0, r
    small = sp.sp24_probe_sclk(blocks=3, iters=10)
    assert small["waves"] == 12
