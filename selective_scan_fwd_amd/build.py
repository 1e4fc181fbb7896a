"""Build the HIP library libvmscan.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvmscan.so")
SOURCES = ["api.hip", "scan_kernel.hip", "scan_chunk.hip", "scan_bwd.hip", "layout_kernels.hip"]
# The VALU issue-rate probe behind the benchmark's ALU roofline: a library of
# its own, so that the scan library holds only the hot path.
PROBE_LIB = os.path.join(PKG, "libvmprobe.so")
PROBE_SOURCES = ["valu_probe.hip"]

# Packed fp32 VALU forms are turned off for all device code.
HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmds):
    """Runs the commands in parallel; raises with every failure's output."""
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
             for c in cmds]
    errors = []
    for c, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append("hipcc failed:\n" + " ".join(c) + "\n" + out + err)
    if errors:
        raise RuntimeError("\n".join(errors))


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc process per file, in parallel) and
    link libvmscan.so and the probe library libvmprobe.so (always recompiles)."""
    with tempfile.TemporaryDirectory(prefix="vmbuild") as tmpdir:
        objs = {}
        cmds = []
        for src in SOURCES + PROBE_SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            objs[src] = obj
            cmds.append([hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        _run(cmds)
        links = []
        for sources, lib in ((SOURCES, LIB), (PROBE_SOURCES, PROBE_LIB)):
            tmp = lib + ".tmp%d" % os.getpid()
            links.append(([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
                           *[objs[s] for s in sources], "-o", tmp], tmp, lib))
        _run([c for c, _, _ in links])
        for c, tmp, lib in links:
            if verbose:
                print(" ".join(c))
            os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
