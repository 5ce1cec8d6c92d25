"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

api.hip is rebuilt with the sanitizers on its host pass only (-Xarch_host before each
-fsanitize; the device code is unchanged and never runs here), linked with the package's kernel
objects and the fuzz driver tests/sanitize/abi_fuzz.c, and run: 200,000 seeded size queries over
valid, inconsistent and extreme configurations, and every entry point with arguments that the
host validation must reject (NULL, misaligned, out of range, short workspace).  Any heap
overflow, use after free, leak from the library, signed overflow or other undefined behaviour in
that host code fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "_build", "obj")
OUT = os.path.join(ROOT, "_build", "asan")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not installed")
    if not all(os.path.exists(os.path.join(OBJ, f)) for f in ("kernels.o", "pack.o")):
        _run(["python3", os.path.join(ROOT, "sparse_moe_proj_amd", "build.py")])
    os.makedirs(OUT, exist_ok=True)
    host_san = [a for s in SAN for a in ("-Xarch_host", s)]
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'sparse_moe_proj_amd', 'csrc')}"]
    api_o = os.path.join(OUT, "api.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", *host_san, "-Xarch_host", "-fno-omit-frame-pointer", *inc, "-c",
          os.path.join(ROOT, "sparse_moe_proj_amd", "csrc", "api.hip"), "-o", api_o])
    fuzz_o = os.path.join(OUT, "abi_fuzz.o")
    _run([CLANG, "-O1", "-g", "-std=c11", *SAN, "-fno-omit-frame-pointer", *inc, "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.c"), "-o", fuzz_o])
    exe = os.path.join(OUT, "abi_fuzz")
    _run([CLANGXX, *SAN, fuzz_o, api_o, os.path.join(OBJ, "kernels.o"), os.path.join(OBJ, "pack.o"),
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    supp = os.path.join(OUT, "lsan.supp")
    with open(supp, "w") as f:  # allocations the ROCm runtime itself keeps until exit
        f.write("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libamd_comgr\nleak:librocprof\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               LSAN_OPTIONS=f"suppressions={supp}:print_suppressions=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout
    print(r.stdout)
