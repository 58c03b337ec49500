"""Builds libet.so (the HIP library behind include/et.h) for gfx950 in-tree.

Usage: python -m event_driven_moe_amd.build   (or build() from Python)
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libet.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["et_moe.hip", "et_block.hip", "et_api.hip", "et_splitk.hip", "et_mlp.hip", "et_decode.hip",
           "et_ceiling.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-munsafe-fp-atomics",
    # packed fp32 instructions stay off: scalar / float2 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no wave-aggregated atomics: every atomic here is issued by one lane (or
    # at per-item addresses), and the aggregated form reads its result back
    # at once, which would put the queue claim's round trip on the path the
    # claim-ahead takes it off
    "-Xarch_device", "-mllvm=-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]


def _compile(src, extra):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(extra_flags=(), verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra_flags)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
