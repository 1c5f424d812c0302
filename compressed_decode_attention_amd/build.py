"""Build libcda_hip.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m compressed_decode_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["compact.hip", "attn.hip", "chunk.hip", "abi.hip"]
OUT = os.path.join(HERE, "libcda_hip.so")
# the benchmark's measurement kernel (plain tile streaming), a library of its own
STREAM_SOURCES = ["stream.hip"]
STREAM_OUT = os.path.join(HERE, "libcda_stream.so")
ARCH = os.environ.get("CDA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    return "hipcc"


def command(out: str = OUT, sources=SOURCES) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed FP32 instructions stay off (see the build notes)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-o", out] + [os.path.join(CSRC, s) for s in sources]


def _build_one(out: str, sources, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """The attention library and the benchmark's measurement library."""
    _build_one(STREAM_OUT, STREAM_SOURCES, verbose)
    return _build_one(OUT, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
