"""Ahead-of-time build of the gfx950 HIP library ``libdrafter_attn.so`` (in-tree).

Usage: ``python -m speculative_decoding_drafter_amd.build`` or ``build_library()``.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "drafter_attn.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdrafter_attn.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Measurement builds, loaded only by bench.py: the same source with the static split
# plan alone (the reference `bench.py --mixed` measures the length-aware schedule
# against) and with phase timestamps (`bench.py --phases`); and the page-stream probe,
# the attention's context reads without the attention (`bench.py --ceiling`).
LIB_STATIC_PLAN = os.path.join(PKG, "libdrafter_attn_static_plan.so")
LIB_PHASES = os.path.join(PKG, "libdrafter_attn_phases.so")
LIB_PROBE = os.path.join(PKG, "libpage_stream_probe.so")
PROBE_SRC = os.path.join(PKG, "csrc", "page_stream_probe.hip")
VARIANTS = {None: (LIB, [], SRC), "static_plan": (LIB_STATIC_PLAN, ["-DDA_STATIC_PLAN_ONLY"], SRC),
            "phases": (LIB_PHASES, ["-DDA_PHASE_TRACE"], SRC), "probe": (LIB_PROBE, [], PROBE_SRC)}


def build_library(verbose: bool = False, variant: str = None) -> str:
    """Compile the library (or a measurement build) from source, always, and return
    the path of the .so."""
    lib, extra, src = VARIANTS[variant]
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-o", tmp, src]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msgs = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    for v in VARIANTS:
        print(build_library(verbose=True, variant=v))
