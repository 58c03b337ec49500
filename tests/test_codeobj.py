"""The persistent kernels make no calls.

Every device function of the event runtime is inlined into the kernels (the
notify / wait / claim helpers are __forceinline__).  A version in which the
queue claim and the waits were out-of-line functions, called by one lane of
the workgroup, kept the launch context in per-lane scratch memory and
computed wrong down-projection rows in one tile variant under the dynamic
schedule; this test keeps calls out of the built code objects.  It
disassembles the library built in this tree (the gfx950 code objects inside
its offload bundles) with the ROCm LLVM tools; it is skipped when the
library or the tools are missing."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "event_driven_moe_amd", "libet.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(tmp):
    fat = os.path.join(tmp, "fatbin.bin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat, LIB],
                   check=True, capture_output=True)
    data = open(fat, "rb").read()
    starts = []
    i = data.find(MAGIC)
    while i >= 0:
        starts.append(i)
        i = data.find(MAGIC, i + 1)
    objs = []
    for n, s in enumerate(starts):
        end = starts[n + 1] if n + 1 < len(starts) else len(data)
        b = os.path.join(tmp, "bundle%d.bin" % n)
        with open(b, "wb") as fh:
            fh.write(data[s:end])
        o = os.path.join(tmp, "co%d.o" % n)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--input=" + b, "--output=" + o],
                       check=True, capture_output=True)
        objs.append(o)
    return objs


def test_persistent_kernels_make_no_calls():
    if not os.path.exists(LIB):
        pytest.skip("libet.so not built")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    tmp = tempfile.mkdtemp()
    try:
        objs = _code_objects(tmp)
        assert len(objs) >= 7          # one per HIP source of the library
        kernels = 0
        for o in objs:
            asm = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", o], check=True,
                                 capture_output=True, text=True).stdout
            # a call is s_swappc_b64 (s_setpc_b64 also ends the long branches
            # of these large kernels, so it proves nothing by itself)
            assert "s_swappc_b64" not in asm, "call in %s" % o
            # and no device function was emitted out of line: every function
            # symbol is a kernel, i.e. has a kernel descriptor NAME.kd
            syms = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-s", "-W", o], check=True,
                                  capture_output=True, text=True).stdout.split("\n")
            funcs = {l.split()[-1] for l in syms if " FUNC " in l}
            kds = {l.split()[-1][:-3] for l in syms if l.split() and l.split()[-1].endswith(".kd")}
            assert funcs and funcs <= kds, "non-kernel functions in %s: %s" % (o, sorted(funcs - kds))
            kernels += len(funcs)
        assert kernels > 0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
