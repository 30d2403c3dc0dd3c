"""Register and memory budget of the persistent kernel (CPU only).

The compiler's resource report for every instantiation of the megakernel
(from the last build when the device sources are unchanged since, else from a
device-only compile of about half a minute) must keep the committed budget:
one 512-thread workgroup per compute unit needs two waves per SIMD, so at most
256 registers per lane; register spills may not grow past the counts the
kernel has now (each spilled register is a scratch round trip inside a
streaming loop); LDS stays within the 160 KiB of a CU.
"""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# instantiation (head dim, row tiles, FP8 feed-forward weights) -> most VGPR
# spills allowed; SGPR spills (to VGPR lanes, no memory traffic; the dense FFN
# claimer's own instance roughly doubles them) are bounded loosely
VGPR_SPILLS = {(64, 1, 0): 7, (64, 2, 0): 4, (128, 1, 0): 8, (128, 2, 0): 4,
               (64, 1, 1): 10, (64, 2, 1): 6, (128, 1, 1): 10, (128, 2, 1): 6}
# (the FP8 batch <= 16 instance holds the fused and the claiming MoE)
SGPR_SPILLS_MAX = {0: 350, 1: 400}


def _build_module():
    spec = importlib.util.spec_from_file_location("mk_build", os.path.join(ROOT, "moe_persistent_decode_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_megakernel_resource_budget():
    rep = _build_module().resource_report()["kernels"]
    seen = set()
    for sym, r in rep.items():
        if not sym.startswith("_Z9mk_interpILi"):
            continue
        # _Z9mk_interpILi<D>ELi<MT>ELb<FP8>EEv9mk_params
        d = int(sym.split("ILi")[1].split("ELi")[0])
        mt = int(sym.split("ELi")[1].split("ELb")[0])
        fp8 = int(sym.split("ELb")[1].split("EE")[0])
        key = (d, mt, fp8)
        seen.add(key)
        assert r["Occupancy [waves/SIMD]"] >= 2, (sym, r)
        assert r["VGPRs"] + r["AGPRs"] <= 256, (sym, r)
        assert r["VGPRs Spill"] <= VGPR_SPILLS[key], (sym, r)
        assert r["SGPRs Spill"] <= SGPR_SPILLS_MAX[fp8], (sym, r)
        assert r["ScratchSize [bytes/lane]"] <= 8 * VGPR_SPILLS[key] + 8, (sym, r)
        assert r["LDS Size [bytes/block]"] <= 160 * 1024, (sym, r)
        assert r["Dynamic Stack"] == "False", (sym, r)
    assert seen == set(VGPR_SPILLS), seen


def test_resource_remarks_parse():
    text = (
        "x.hip:1:1: remark: Function Name: _Z9mk_interpILi128ELi1EEv9mk_params [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 32 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    rep = _build_module().parse_resource_remarks(text)
    assert rep == {"_Z9mk_interpILi128ELi1EEv9mk_params": {"VGPRs": 256, "ScratchSize [bytes/lane]": 32,
                                                          "Dynamic Stack": "False"},
                   "k2": {"VGPRs Spill": 0}}
