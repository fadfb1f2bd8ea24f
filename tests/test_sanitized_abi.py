"""The C-ABI validation layer under the address and undefined-behaviour sanitizers (CPU only).

The library's host-side entry points (rd_api.hip, rd_debug.hip) are
compiled again with -fsanitize=address,undefined on their host code only
(device code is compiled as usual; nothing here launches a kernel) and
linked with the ordinary kernel objects into a separate library.  A C driver
(tests/abi_validation.c), itself sanitized, calls every entry point with the
arguments that host validation must reject or short-circuit, and must
finish without a sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

from tree_attention_verification_rd_amd import build as rdbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
VALIDATION_SOURCES = ("rd_api.hip", "rd_debug.hip")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    return res


def build_sanitized() -> str:
    os.makedirs(SAN, exist_ok=True)
    objs = []
    for src in rdbuild.sources():
        name = os.path.basename(src)
        if name in VALIDATION_SOURCES:
            obj = os.path.join(SAN, name + ".o")
            run([rdbuild.HIPCC, *rdbuild.FLAGS, *HOST_SAN, "-c", src, "-o", obj])
        else:
            obj = os.path.join(rdbuild.BUILD, name + ".o")
            if not os.path.exists(obj):
                rdbuild.build()
        objs.append(obj)
    lib = os.path.join(SAN, "librd_san.so")
    run([rdbuild.HIPCC, f"--offload-arch={rdbuild.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan",
         *objs, "-o", lib])
    clang = shutil.which("clang", path="/opt/rocm/llvm/bin") or "clang"
    # the shared sanitizer runtimes (the one libclang_rt.asan-x86_64.so the driver loads)
    rtdir = os.path.dirname(run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip())
    if not os.path.exists(os.path.join(rtdir, "libclang_rt.asan-x86_64.so")):
        import glob
        rtdir = os.path.dirname(sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(clang)), "lib", "clang",
                                                              "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))[-1])
    exe = os.path.join(SAN, "abi_validation")
    run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_validation.c"),
         "-L", SAN, "-lrd_san", f"-Wl,-rpath,{SAN}", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rtdir}", "-o", exe])
    return exe


def test_validation_layer_is_clean_under_sanitizers():
    exe = build_sanitized()
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, f"{res.stdout}\n{res.stderr}"
    assert "ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
