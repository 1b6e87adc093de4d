"""Build libpa.so (the HIP library behind include/pa.h) in-tree with hipcc for gfx950."""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed FP32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the prefill kernel rescales them in
    # place, which in AGPRs costs a copy out and back (the other kernels already
    # use the VGPR form)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # every atomic here is issued by one lane; the wave-level atomic rewrite
    # only adds instructions (and a wait for the returned value)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# The same library with the decode's PV product on the VALU in FP32 instead of
# MFMA (the build-time switch PA_DECODE_PV_VALU), for the measured comparison.
LIB_PV_VALU = os.path.join(PKG, "libpa_pv_valu.so")
SOURCES = ("pa_api.cpp", "pa_sched.cpp", "pa_kernels.hip", "pa_prefill.hip", "pa_rope.hip")


def _build_lib(out: str, defines=(), verbose: bool = False) -> None:
    srcs = [os.path.join(CSRC, f) for f in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *defines, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _build_lib(LIB, verbose=verbose)
    _build_lib(LIB_PV_VALU, ("-DPA_DECODE_PV_VALU=1",), verbose=verbose)
    # the streaming-read reference the benchmark times beside the kernels
    probe = os.path.join(PKG, "libpa_probe.so")
    cmd = [hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, "stream_probe.hip"), "-o", probe + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the streaming-read probe ({res.returncode}):\n{res.stderr}")
    os.replace(probe + ".tmp", probe)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
