"""Compile the sdit HIP library for gfx950, in-tree.

    python -m streaming_video_dit_amd.build

writes streaming_video_dit_amd/libsdit.so next to this file, and beside it
libsdit_single_stage.so: the same library with the attention kernel's
pipelined schedule replaced by a one-tile-at-a-time schedule
(SDIT_SINGLE_STAGE=1), which exists only so that tests can check that the
prefetching schedule gives bit-identical results. The two compile in
parallel.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsdit.so")
LIB_SINGLE_STAGE = os.path.join(HERE, "libsdit_single_stage.so")

SOURCES = ["sdit_api.cpp", "qknorm_rope3d.hip", "kv_quant_int8.hip", "attn_fwd.hip", "attn_merge.hip", "window_permute.hip",
           "norms.hip", "static_scratch.hip"]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # correctly rounded fp32 divide/sqrt (the int8 quantiser depends on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _command(out: str, extra_flags) -> list:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc()] + FLAGS + list(extra_flags or []) + ["-I", os.path.join(ROOT, "include"), "-o", out] + srcs


def _finish(proc, cmd, tmp, lib, verbose):
    out, err = proc.communicate()
    # the host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (out + err).splitlines() if noise not in l and l.strip()]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Build libsdit.so and libsdit_single_stage.so (in parallel); returns the
    path of libsdit.so."""
    jobs = []
    for lib, flags in ((LIB, list(extra_flags or [])),
                       (LIB_SINGLE_STAGE, list(extra_flags or []) + ["-DSDIT_SINGLE_STAGE=1"])):
        tmp = lib + ".tmp"
        cmd = _command(tmp, flags)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), cmd, tmp, lib))
    for proc, cmd, tmp, lib in jobs:
        _finish(proc, cmd, tmp, lib, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
