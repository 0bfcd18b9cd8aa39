"""Build the gfx950 SDPA library (libsdpa_gfx950.so) in-tree with hipcc.

Every source is compiled as HIP for gfx950 only, with packed-fp32 VALU instructions
disabled on the device side (-packed-fp32-ops); the host pass prints a harmless warning
about that feature.  Each source is compiled to its own object (with its own extra flags)
and the objects are linked into one shared library.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsdpa_gfx950.so")
# source -> extra compiler flags.  The backward kernels run one wave per SIMD with more
# than 256 live registers; left to its heuristics the compiler gives their matrix
# products accumulator-register (AGPR) destinations and then copies every accumulator
# between the two register files on each loop iteration.  Forcing the VGPR form of the
# products keeps the accumulators in place.
SOURCES = {
    "sdpa_fwd_gfx950.hip": [],
    "sdpa_bwd_gfx950.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "sdpa_abi.cpp": [],
}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels never create a NaN from finite inputs; without NaN semantics the
    # row maxima lower to 3-input v_max3 instead of canonicalise + max pairs
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, extra_flags=()) -> str:
    objs = []
    with tempfile.TemporaryDirectory(prefix="sdpa_build_") as tmpdir:
        for src, flags in SOURCES.items():
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            _run([hipcc(), *HIPCC_FLAGS, *flags, *extra_flags, "-c", "-x", "hip",
                  os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
