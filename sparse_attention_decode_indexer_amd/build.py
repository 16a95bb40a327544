"""Builds the gfx950 HIP library ``libdsa.so`` in place (hipcc, no JIT cache), and the
benchmark's read-ceiling helper ``libdsa_read_ceiling.so`` (not part of the library)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["capi.hip", "index_topk.hip", "attention.hip", "layer.hip", "swa_out.hip", "layer_dsa.hip", "swa_chain.hip"]
LIB = os.path.join(HERE, "libdsa.so")
READ_CEILING_SOURCES = ["read_ceiling.hip"]
READ_CEILING_LIB = os.path.join(HERE, "libdsa_read_ceiling.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(" ".join(cmd))


def build(verbose: bool = False) -> str:
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(READ_CEILING_SOURCES, READ_CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
