"""The library's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libseer is compiled as the product build compiles it, except
that the host half is instrumented (``-Xarch_host -fsanitize=...``: the gfx950
device code is left alone). The objects are linked with the C harness in
``tests/sanitize/host_checks.c``, which calls every entry point of
``include/seer.h`` only on paths that must return before anything reaches the
GPU: argument, size, capacity and workspace checks, the size functions at
extreme sizes, and the status helpers. A sanitizer report or a wrong status
fails the test. No GPU is needed.
"""

import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

from block_sparse_attention_prefill_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "sanitize", "host_checks.c")
OUT = os.path.join(ROOT, "_build", "asan")
LLVM = "/opt/rocm/llvm/bin"
ROCM_LIB = "/opt/rocm/lib"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def _host_only(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def _toolchain():
    clang = os.path.join(LLVM, "clang")
    clangxx = os.path.join(LLVM, "clang++")
    rt = glob.glob(os.path.join(LLVM, "..", "lib", "clang", "*", "lib", "*",
                                "libclang_rt.asan*x86_64*"))
    rt += glob.glob(os.path.join(LLVM, "..", "lib", "clang", "*", "lib", "*", "*",
                                 "libclang_rt.asan*"))
    if not (os.path.exists(clang) and os.path.exists(clangxx) and rt):
        pytest.skip("ROCm clang with the ASan runtime is not installed")
    try:
        hipcc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    return hipcc, clang, clangxx


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"


def _compile(hipcc, src):
    # The product flags with -O3 lowered so the reports keep their frames.
    flags = [f for f in libbuild.flags_for(src) if f != "-O3"] + ["-O1", "-g"]
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    _run([hipcc, *flags, *_host_only(SAN), "-x", "hip", "-c",
          os.path.join(libbuild.CSRC, src), "-o", obj])
    return obj


def test_harness_calls_every_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(libbuild.INCLUDE, "seer.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(seer_[a-z_]+)\s*\(", text)))
    harness = open(HARNESS).read()
    missing = [n for n in names if not re.search(r"\b" + n + r"\(", harness)]
    assert not missing, missing


@pytest.mark.timeout(900)
def test_host_layer_under_asan_and_ubsan():
    hipcc, clang, clangxx = _toolchain()
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), libbuild.SOURCES))
    main_obj = os.path.join(OUT, "host_checks.o")
    _run([clang, "-std=c11", "-O1", "-g", *SAN, "-I", libbuild.INCLUDE, "-c", HARNESS,
          "-o", main_obj])
    exe = os.path.join(OUT, "host_checks")
    _run([clangxx, *SAN, "-o", exe, main_obj, *objs, "-L", ROCM_LIB, "-lamdhip64",
          f"-Wl,-rpath,{ROCM_LIB}"])
    env = dict(os.environ)
    # The HIP runtime keeps its device tables until exit; leaks are not checked.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    log = res.stdout + res.stderr
    assert res.returncode == 0, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
    assert re.search(r"host checks: \d+ passed", res.stdout), log
