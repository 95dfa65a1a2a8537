"""Build the HIP libraries in-tree with hipcc for gfx950.

    python attention_mla_causal_amd/build.py

Compiles the attention core's HIP sources under csrc/ into libmla_attn.so
next to this file, and the benchmark's measurement probes (csrc/mla_probe.hip,
outside the attention ABI) into libmla_probe.so. Always recompiles (it is the
"does it build" step); loading a library never builds it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmla_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["mla_attn_abi.hip", "mla_prefill.hip", "mla_decode.hip", "mla_latent.hip", "mla_rope.hip"]
PROBE_SOURCES = ["mla_probe.hip"]
PROBE_LIB_PATH = os.path.join(HERE, "libmla_probe.so")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs rather than AGPRs. The latent decode's
    # attention kernel rescales its 128 output accumulators every key tile;
    # kept in AGPRs, each rescale costs two register copies per value on top
    # of the multiply (batched latent decode 107 -> 97 us with this alone).
    # No other kernel here holds accumulators in AGPRs; their code is
    # unchanged by it.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Build libmla_attn.so and libmla_probe.so; returns the first's path."""
    _build_one(SOURCES, LIB_PATH, verbose, extra_flags)
    _build_one(PROBE_SOURCES, PROBE_LIB_PATH, verbose, extra_flags)
    return LIB_PATH


def _build_one(sources, lib_path, verbose, extra_flags) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
