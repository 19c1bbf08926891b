"""Compile-time resources of every kernel in the library, from the compiler's
resource-usage remarks that the build records (gemv_gate_up_amd/build.py,
RESOURCE_FILE): no kernel may use scratch memory (private per-lane memory,
which register spills would go to) or a dynamic stack, and every kernel
family of the hot path must be there.  The record must come from the
current sources."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_swiglu_build_for_tests", os.path.join(ROOT, "gemv_gate_up_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


B = _build_module()

FAMILIES = ["pack_kernel", "pack_act_kernel", "fp8_scale_kernel", "pack_fp8_kernel",
            "mx_scale_kernel", "pack_mxfp4_kernel", "skinny_bf16_kernel", "skinny_f32_kernel",
            "skinny_f32m_kernel", "splitk_reduce_kernel", "wide_bf16_kernel", "rmsnorm_kernel",
            "mlp_fused_kernel"]


def _record():
    assert os.path.exists(B.RESOURCE_FILE), "build the library first (gemv_gate_up_amd/build.py)"
    with open(B.RESOURCE_FILE) as f:
        rec = json.load(f)
    assert rec["sources"] == B.source_fingerprint(), \
        "the resource record predates the current sources: rebuild the library"
    return rec


def test_remark_parser_reads_every_field():
    text = "\n".join([
        "a.hip:9:1: remark: Function Name: _ZN3swg1kEv [-Rpass-analysis=kernel-resource-usage]",
        "   9 | {",
        "a.hip:9:1: remark:     TotalSGPRs: 36 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs: 30 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     AGPRs: 4 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     Dynamic Stack: True [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     SGPRs Spill: 1 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     LDS Size [bytes/block]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: remark: Function Name: _ZN3swg1mEv [-Rpass-analysis=kernel-resource-usage]",
    ])
    ks = B.parse_resource_remarks(text)
    assert ks[0] == {"kernel": "_ZN3swg1kEv", "sgprs": 36, "vgprs": 30, "agprs": 4,
                     "scratch_bytes": 12, "dynamic_stack": True, "occupancy": 8,
                     "sgpr_spill": 1, "vgpr_spill": 2, "lds_bytes": 16}
    assert ks[1] == {"kernel": "_ZN3swg1mEv"}


def test_every_kernel_family_is_recorded():
    rec = _record()
    assert rec["arch"] == "gfx950"
    names = [k["kernel"] for k in rec["kernels"]]
    for fam in FAMILIES:
        assert any(fam in n for n in names), fam
    for k in rec["kernels"]:
        assert set(k) >= {"kernel", "source", "vgprs", "agprs", "scratch_bytes", "occupancy",
                          "vgpr_spill", "sgpr_spill", "dynamic_stack", "lds_bytes"}, k


def test_no_kernel_spills_or_uses_scratch():
    bad = [k for k in _record()["kernels"]
           if k["scratch_bytes"] or k["vgpr_spill"] or k["sgpr_spill"] or k["dynamic_stack"]]
    assert not bad, bad


def test_register_and_lds_budgets():
    for k in _record()["kernels"]:
        assert k["vgprs"] + k["agprs"] <= 512, k       # one wave's unified register file
        assert k["occupancy"] >= 1, k
        assert k["lds_bytes"] <= 160 * 1024, k         # static LDS; the wide kernel's is dynamic
