"""Build the HIP library libkvring.so in-tree for gfx950 with hipcc.

Every source is compiled with floating-point contraction off (the write, rotation and
quantisation arithmetic must round each operation on its own to match the CPU oracle bit
for bit; the attention kernel asks for fused multiply-adds explicitly where it wants them)
and with packed-FP32 instructions disabled."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvring.so")
SOURCES = ["kvring_abi.hip", "kv_ring_write.hip", "kv_ring_delta_rotate.hip", "ring_attention.hip",
           "kv_window.hip"]
ARCH = os.environ.get("KVRING_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results in ordinary VGPRs where they fit: the softmax reads every score
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-function",
        *[os.path.join(CSRC, s) for s in SOURCES], "-o", out, *(extra or []),
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libkvring.so (always recompiles).  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkvring.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
