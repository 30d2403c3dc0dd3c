"""Build the HIP library libmk.so in-tree for gfx950 (hipcc, no GPU needed)."""
import os
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


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, "mk_device.hip"), os.path.join(CSRC, "mk_host.cpp"), os.path.join(CSRC, "mk_service.cpp")]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
