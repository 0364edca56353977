"""Build libattn_prefill.so (HIP, gfx950 only) in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name) for name in ("attn_prefill.hip", "attn_fp8.hip", "attn_bwd.hip")]
SRC = SRCS[0]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_prefill.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax reads the scores straight from the
    # MFMA destination instead of copying them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # no NaN ever reaches fmax (masked scores are -inf, never NaN), so the
    # compiler may drop the quieting it adds around every max
    "-fno-honor-nans",
    "-Wall",
]


# the matrix-core rate probe the benchmark reports as context (a library of
# its own: nothing in the attention library uses it)
CEILING_SRC = os.path.join(PKG, "csrc", "mfma_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libmfma_ceiling.so")


def _compile(srcs, lib, verbose, extra=()):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra=()) -> str:
    """Compile the HIP sources into LIB and the rate probe into CEILING_LIB
    (always recompiles)."""
    _compile(SRCS, LIB, verbose, extra)
    _compile([CEILING_SRC], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
