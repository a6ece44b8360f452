"""Host-side checks of the build script's register-spill report."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(os.path.dirname(HERE), "autoround_signsgd_rounding_amd", "build.py")


def _build_module():
    spec = importlib.util.spec_from_file_location("ar_build_script", BUILD)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_spill_report_names_hot_kernels_only():
    b = _build_module()
    remarks = [
        "ar_gemm.hip:336:1: remark: Function Name: _ZN12_GLOBAL__N_112k_fwd_streamENS_13FwdStreamArgsE",
        "ar_gemm.hip:336:1: remark:     VGPRs Spill: 12",
        "ar_quant.hip:10:1: remark: Function Name: _ZN12_GLOBAL__N_18k_pack_wILi4ELb1EEEvPKhPjll",
        "ar_quant.hip:10:1: remark:     VGPRs Spill: 4",
        "ar_gemm.hip:76:1: remark: Function Name: _ZN12_GLOBAL__N_16k_gemmINS_8EpiWgradEEEvNS_8GemmArgsET_",
        "ar_gemm.hip:76:1: remark:     VGPRs Spill: 0",
    ]
    assert b._spills(remarks) == [("_ZN12_GLOBAL__N_112k_fwd_streamENS_13FwdStreamArgsE", 12)]
    assert b._spills([]) == []
