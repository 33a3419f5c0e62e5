"""The host-side argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no kernel runs).

moe_abi.hip -- every entry point's checks, workspace arithmetic and launch
sequencing -- is rebuilt with both sanitizers on its host code only
(`-Xarch_host`; device code cannot be instrumented) and linked with the other
objects of the in-tree build into a scratch copy of the library.  The CPU ABI
tests (tests/test_abi_cpu.py) then run against that copy in a child Python
with the clang sanitizer runtime preloaded: any out-of-bounds access, use
after free, signed overflow or invalid load in the validation paths aborts
the child.  A planted heap overflow in a throwaway C file shows that the
runtime and options used here do report errors.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "token_routed_expert_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def _env(rt):
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, LD_BIND_NOW="1", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = _runtime()
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    others = [o for o in objs if os.path.basename(o) != "moe_abi.o"]
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and rt and len(others) == len(objs) - 1):
        pytest.skip("needs hipcc, clang's sanitizer runtime and the in-tree build objects")
    sys.path.insert(0, ROOT)
    from token_routed_expert_amd import build
    d = tmp_path_factory.mktemp("san")
    obj = str(d / "moe_abi_san.o")
    flags = [f for f in build.CXXFLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    subprocess.run([HIPCC, *flags, "-c", os.path.join(PKG, "csrc", "moe_abi.hip"), "-o", obj],
                   check=True, capture_output=True, text=True)
    lib = str(d / "libtre_moe.so")
    subprocess.run([CLANG + "++", "-shared", "-fPIC", obj, *others, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", lib], check=True, capture_output=True, text=True)
    return lib, rt, d


def test_sanitizer_runtime_reports_errors(sanitized_lib):
    _, rt, d = sanitized_lib
    src = d / "overflow.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile char* p = malloc(8); p[8] = 1; "
                   "free((void*)p); return 0; }\n")
    exe = str(d / "overflow")
    subprocess.run([CLANG, "-g", "-fsanitize=address", "-shared-libsan", str(src), "-o", exe],
                   check=True, capture_output=True, text=True)
    env = _env(rt)
    env["LD_LIBRARY_PATH"] = os.path.dirname(rt)
    r = subprocess.run([exe], env=env, capture_output=True, text=True)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_abi_validation_under_sanitizers(sanitized_lib):
    lib, rt, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", lib], check=True, capture_output=True, text=True).stdout
    assert " U __asan_" in syms and " U __ubsan_" in syms, "moe_abi.hip was not instrumented"
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "from token_routed_expert_amd import _native\n"
        f"_native.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}, "
        "'-m', 'not gpu']))\n")
    r = subprocess.run([sys.executable, "-c", code], env=_env(rt), capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
