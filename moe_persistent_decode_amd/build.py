"""Build the HIP library libmk.so in-tree for gfx950 (hipcc, no GPU needed)."""
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed fp32 ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics on counters are issued by one lane; the optimizer's rewrite
    # (elect a lane, broadcast the result) waits for the result at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


# the compiler's per-kernel resource report (registers, spills, scratch, LDS,
# occupancy), kept beside the library
RESOURCES = os.path.join(HERE, "libmk.resources.json")
DEVICE_SOURCES = ("mk_device.hip", "mk_internal.h", "mk_launch.h")


def device_sources_sha16() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DEVICE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse_resource_remarks(text: str) -> dict:
    """{kernel symbol: {field: value}} from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1).strip()] = int(v) if v.isdigit() else v
    return out


def resource_report() -> dict:
    """The device code's resource report: from the last build when the device
    sources are unchanged since, else from a device-only compile."""
    sha = device_sources_sha16()
    try:
        with open(RESOURCES) as fh:
            rep = json.load(fh)
        if rep.get("device_sources_sha256_16") == sha:
            return rep
    except (OSError, ValueError):
        pass
    cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + [
        "--cuda-device-only", "-c", os.path.join(CSRC, "mk_device.hip"), "-o", os.devnull,
        "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError("hipcc failed compiling mk_device.hip")
    return {"device_sources_sha256_16": sha, "kernels": parse_resource_remarks(r.stderr)}


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, "mk_device.hip"), os.path.join(CSRC, "mk_host.cpp"), os.path.join(CSRC, "mk_service.cpp")]
    tmp = LIB + ".tmp"
    sha = device_sources_sha16()
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage"] + srcs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    kernels = parse_resource_remarks(r.stderr)
    if verbose:
        for k, v in kernels.items():
            sys.stderr.write(f"{k}: {v}\n")
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as fh:
        json.dump({"device_sources_sha256_16": sha, "kernels": kernels}, fh, indent=1)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
