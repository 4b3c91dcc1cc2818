"""Build libfa.so (the gfx950 HIP kernel and its C-ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa_api.hip")
LIB = os.path.join(PKG, "libfa.so")

# Packed fp32 VALU instructions are switched off for all device code (-packed-fp32-ops); the host
# pass does not know the feature and says so, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(extra_flags=(), out: str = LIB, src: str = SRC, mfma_vgpr_form: bool = True) -> str:
    """mfma_vgpr_form=False leaves the choice of MFMA accumulator registers to the compiler, which
    takes VGPRs in a kernel that uses no AGPRs and AGPRs in one that does."""
    tmp = out + ".tmp"
    flags = [f for f in HIPCC_FLAGS if mfma_vgpr_form or f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
    cmd = [hipcc(), *flags, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(ROOT, "tests", "fp8_mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "libfp8_mfma_probe.so")


ISSUE_SRC = os.path.join(ROOT, "tests", "issue_rate_probe.hip")
ISSUE_LIB = os.path.join(ROOT, "tests", "libissue_rate_probe.so")
BF16_PROBE_SRC = os.path.join(ROOT, "tests", "bf16_mfma_probe.hip")
BF16_PROBE_LIB = os.path.join(ROOT, "tests", "libbf16_mfma_probe.so")


def build_probe() -> str:
    """Test infrastructure: the probes the GPU tests run (the accuracy of the FP8 and of the bf16
    matrix instruction, and the issue rates of the forward's inner-loop instructions; one of its modes compares the matrix
    accumulators in AGPRs with the VGPRs that every other mode and the library use)."""
    build(out=ISSUE_LIB, src=ISSUE_SRC, mfma_vgpr_form=False)
    build(out=BF16_PROBE_LIB, src=BF16_PROBE_SRC)
    return build(out=PROBE_LIB, src=PROBE_SRC)


if __name__ == "__main__":
    print(build())
    print(build_probe())
