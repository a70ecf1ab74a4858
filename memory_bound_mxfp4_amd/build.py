"""Build libmoe_mxfp4.so (hipcc, gfx950) in-tree, next to this file."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SO = os.path.join(PKG, "libmoe_mxfp4.so")
SOURCES = ["api.hip", "router.hip", "experts.hip", "dense.hip", "pack.hip", "layer.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for all device code.  The atomic
# optimizer is off: it rewrites a one-lane atomic into a wave-wide pattern
# whose result is broadcast straight away, which makes every work-queue pop
# wait for its round trip before the unit's own loads can issue.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(PKG, "csrc", s) for s in SOURCES]
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), *srcs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
