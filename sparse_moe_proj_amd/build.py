"""Build liblmoe.so (gfx950) in-tree with hipcc: one object per .hip source under csrc/, compiled in
parallel, then linked into sparse_moe_proj_amd/liblmoe.so.  Also builds libpeaks.so from peaks/
(measurement kernels the benchmark reports against; not part of the block).

    python sparse_moe_proj_amd/build.py [--verbose]

Run it as a script (not `-m sparse_moe_proj_amd.build`): importing the package loads the library.

Packed fp32 arithmetic stays off in all device code: `-Xclang -target-feature -Xclang
-packed-fp32-ops` is passed to hipcc, which hands -Xclang options to both of its compile passes
(the driver does not forward -Xclang options to the device pass alone).  The host (x86) pass
therefore prints that it does not know the feature and ignores it; that message is left as the
compiler prints it (shown with --verbose).  Whether the device pass applied it is checked on the
result instead: every object's device code is unbundled and disassembled, and the build fails if
it holds any packed fp32 instruction.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PEAKS = os.path.join(PKG, "peaks")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "liblmoe.so")
PEAKS_LIB = os.path.join(PKG, "libpeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/lib/llvm/bin")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic stays off: plain fp32 VALU only (checked on the device code below)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# gfx950 packed fp32 VALU instructions (must not appear in the device code)
PACKED_FP32 = re.compile(r"\bv_pk_(?:add|mul|fma|mov)_f32\b")


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return r.stdout


def device_code_check(obj: str) -> int:
    """Unbundles the gfx950 code object embedded in `obj` and counts packed fp32 instructions in
    its disassembly (0 expected).  Objects without device code count 0."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        r = subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj,
                            os.path.join(tmp, "rest.o")], capture_output=True, text=True)
        if r.returncode != 0 or not os.path.exists(fat):
            return 0
        co = os.path.join(tmp, "dev.co")
        _run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
              f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"], False)
        dis = _run([os.path.join(LLVM, "llvm-objdump"), "-d", f"--mcpu={ARCH}", co], False)
        return len(PACKED_FP32.findall(dis))


def _compile_link(srcs, lib, objdir, verbose):
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *CFLAGS, "-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
    with ThreadPoolExecutor(min(8, len(objs))) as ex:
        counts = list(ex.map(device_code_check, objs))
    bad = {os.path.basename(o): c for o, c in zip(objs, counts) if c}
    if bad:
        raise RuntimeError(f"packed fp32 instructions in the device code: {bad}")
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _compile_link(sources(PEAKS), PEAKS_LIB, os.path.join(OBJ, "peaks"), verbose)
    return _compile_link(sources(CSRC), LIB, OBJ, verbose)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
