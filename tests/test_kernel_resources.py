"""Every compiled gfx950 kernel fits its registers: no scratch memory.

Any kernel of the library can be reached (every tile variant can be named in
a config, and the fallbacks run on unusual strides), so a kernel that spills
its registers to scratch memory is a silent performance cliff. The build keeps
the device compiler's per-kernel resource report (``-Rpass-analysis=
kernel-resource-usage``); this CPU test reads it, rebuilding first when the
report is older than a source file.
"""
import os
import re

from fp8_w8a8_quantized_token_amd import build

FIELDS = {
    "ScratchSize [bytes/lane]": "scratch",
    "VGPRs Spill": "vgpr_spill",
    "SGPRs Spill": "sgpr_spill",
    "VGPRs": "vgprs",
    "AGPRs": "agprs",
}


def _report_is_fresh():
    if not os.path.exists(build.RESOURCE_REPORT) or not os.path.exists(build.LIB):
        return False
    t = os.path.getmtime(build.RESOURCE_REPORT)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs.append(os.path.join(build.INCLUDE, "fp8w8a8.h"))
    return all(os.path.getmtime(f) <= t for f in srcs)


def kernel_resources():
    if not _report_is_fresh():
        build.build()
    kernels = {}
    cur = None
    with open(build.RESOURCE_REPORT) as f:
        for line in f:
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = kernels.setdefault(m.group(1), {})
                continue
            for label, key in FIELDS.items():
                m = re.search(r"remark:\s+" + re.escape(label) + r": (\d+)", line)
                if m and cur is not None:
                    cur[key] = int(m.group(1))
                    break
    return kernels


def test_no_kernel_spills_or_uses_scratch():
    kernels = kernel_resources()
    assert len(kernels) > 50, "resource report missing kernels"
    # scalar registers spilled into vector-register lanes (no scratch) are
    # allowed; memory spills are not
    bad = {name: r for name, r in kernels.items()
           if r.get("scratch", -1) != 0 or r.get("vgpr_spill", -1) != 0}
    assert not bad, bad
    # the VGPR file of a lane holds 512 registers (architectural + accumulation)
    assert all(r["vgprs"] + r["agprs"] <= 512 for r in kernels.values())
