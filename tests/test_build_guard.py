"""The build's register-spill guard reads the compiler's resource remarks."""
from fp8_scaled_gemm_amd import build

SAMPLE = """./gemm_kernels.hpp:394:1: remark: Function Name: _ZN5fp8sg15k_gemm_pingpongE [-Rpass-analysis=kernel-resource-usage]
./gemm_kernels.hpp:394:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
./gemm_kernels.hpp:394:1: remark:     VGPRs Spill: 1228 [-Rpass-analysis=kernel-resource-usage]
./amax.hip:10:1: remark: Function Name: _ZN5fp8sg6k_amaxE [-Rpass-analysis=kernel-resource-usage]
./amax.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spill_report_is_parsed():
    s = build.spills(SAMPLE)
    assert s == {"_ZN5fp8sg15k_gemm_pingpongE": 1228, "_ZN5fp8sg6k_amaxE": 0}
    assert s["_ZN5fp8sg15k_gemm_pingpongE"] > build.MAX_SPILL_VGPRS
