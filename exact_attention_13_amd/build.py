"""Build step for libfa: compiles the HIP sources for gfx950 into libfa.so
(and the benchmark's MFMA-rate probe into libfa_probe.so).

Run ``python -m exact_attention_13_amd.build``.  The library is built
in-tree (``exact_attention_13_amd/libfa.so``) so that it travels with the
source tree.  The compiler's per-kernel resource report (VGPR/AGPR/SGPR
counts, scratch, LDS, occupancy) is kept in ``_build/kernel_resources.txt``.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libfa.so"
BUILD_DIR = PKG / "_build"
ARCH = "gfx950"

SOURCES = ["fa_api.hip", "fa_api_bwd.hip", "fa_fwd_h16.hip", "fa_fwd_f32.hip", "fa_combine.hip",
           "fa_bwd_h16.hip", "fa_bwd_f32.hip"]
# The benchmark's MFMA-rate probe: a library of its own, not part of libfa.
PROBE_LIB = PKG / "libfa_probe.so"
PROBE_SOURCES = ["mfma_probe.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # keep MFMA operands and accumulators in ordinary VGPRs (no AGPR copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: libfa needs the ROCm toolchain to build")


def _resource_report(stderr: str) -> str:
    keep = []
    for line in stderr.splitlines():
        m = re.search(r"remark:\s+(.*?)\s*\[-Rpass-analysis=kernel-resource-usage\]", line)
        if m:
            keep.append(m.group(1))
    return "\n".join(keep) + "\n"


def build(verbose: bool = False) -> Path:
    BUILD_DIR.mkdir(exist_ok=True)
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", str(ROOT / "include"), "-I", str(CSRC),
           "-Rpass-analysis=kernel-resource-usage",
           "-o", str(tmp), *[str(CSRC / s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building libfa")
    (BUILD_DIR / "kernel_resources.txt").write_text(_resource_report(r.stderr))
    if verbose:
        noise = ("kernel-resource-usage", "not a recognized feature")
        sys.stderr.write("\n".join(l for l in r.stderr.splitlines()
                                   if not any(n in l for n in noise)))
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> Path:
    """Compile libfa_probe.so (the measured MFMA-loop rate the benchmark
    reports beside the published peak)."""
    tmp = PROBE_LIB.with_name(PROBE_LIB.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", str(tmp), *[str(CSRC / s) for s in PROBE_SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building libfa_probe")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def resource_table() -> str:
    """The last build's per-kernel resource report as a markdown table:
    registers (VGPR, AGPR, SGPR), spills and scratch, LDS and occupancy."""
    text = (BUILD_DIR / "kernel_resources.txt").read_text()
    rows = []
    for block in text.split("Function Name: ")[1:]:
        name = block.split("\n", 1)[0].strip()
        f = dict(re.findall(r"^([A-Za-z][A-Za-z /]*(?:\[[^\]]*\])?):\s*(\S+)", block, re.M))
        demangled = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
        demangled = demangled.replace("fa_impl::(anonymous namespace)::", "").replace(
            "fa_impl::", "")
        demangled = re.sub(r"\(.*\)$", "", demangled)
        rows.append((demangled or name, f.get("VGPRs"), f.get("AGPRs"), f.get("TotalSGPRs"),
                     f.get("VGPRs Spill"), f.get("ScratchSize [bytes/lane]"),
                     f.get("LDS Size [bytes/block]"), f.get("Occupancy [waves/SIMD]")))
    out = ["| kernel | VGPR | AGPR | SGPR | VGPR spill | scratch B/lane | LDS B/block | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| `" + r[0] + "` | " + " | ".join(str(x) for x in r[1:]) + " |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    print(build(verbose="--quiet" not in sys.argv))
    if "--report" in sys.argv:
        dest = Path(sys.argv[sys.argv.index("--report") + 1])
        dest.write_text(resource_table())
        print(dest)
