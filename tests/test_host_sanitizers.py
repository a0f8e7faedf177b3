"""The host code of the C-ABI library under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every source is compiled with the sanitizers on its host side only (the device code is compiled as
usual and never runs: no device is visible), linked into a separate library, and then
  * the C consumer (tests/c/abi_consumer.c), built with the same sanitizers, calls it with leak
    checking on;
  * the argument-validation tests of tests/test_abi.py run in a Python process that preloads the
    sanitizer runtime and loads that library instead of the regular one.
Any report ends the process with an error (no recovery), so a clean exit means a clean run."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
HIPCC = "/opt/rocm/bin/hipcc"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LINK = ["-fsanitize=address,undefined", "-shared-libsan"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(os.path.join(LLVM, "clang++"))),
                                reason="needs the ROCm compilers")


def _build_module():
    spec = importlib.util.spec_from_file_location("_nvfp4_build", os.path.join(ROOT, "nvfp4_block_scaled_03_amd",
                                                                               "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _runtime_dir():
    out = subprocess.run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if os.path.exists(out):
        return os.path.dirname(out)
    base = subprocess.run([os.path.join(LLVM, "clang"), "-print-resource-dir"], capture_output=True, text=True,
                          check=True).stdout.strip()
    d = os.path.join(base, "lib", "linux")
    assert os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")), "no shared ASan runtime"
    return d


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    """(library path, runtime dir): the library's sources with the host side instrumented."""
    b = _build_module()
    d = tmp_path_factory.mktemp("san")
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_HOST
    procs = []
    for src in b.SOURCES:
        obj = str(d / (os.path.splitext(src)[0] + ".o"))
        procs.append((obj, subprocess.Popen([HIPCC, *flags, "-c", os.path.join(b.SRC, src), "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for obj, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    rt = _runtime_dir()
    lib = str(d / "libnvfp4_san.so")
    subprocess.run([os.path.join(LLVM, "clang++"), "-shared", "-fPIC", *SAN_LINK, "-o", lib, *[o for o, _ in procs],
                    "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rt}"],
                   check=True, capture_output=True, text=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the library is not instrumented"
    return lib, rt


def _env(rt, **kw):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(kw)
    return env


def test_sanitizers_catch_a_planted_overflow(tmp_path):
    """The toolchain's sanitizers are live: a one-past-the-end read is reported and ends the program."""
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { int* p = malloc(4 * sizeof(int));"
                   " (void)v; int r = p[3 + c]; free(p); return r & 1; }\n")
    exe = str(tmp_path / "oob")
    subprocess.run([os.path.join(LLVM, "clang"), "-g", *SAN_LINK, str(src), "-o", exe,
                    f"-Wl,-rpath,{_runtime_dir()}"], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


@pytest.mark.skipif(shutil.which("nm") is None, reason="needs nm")
def test_c_consumer_clean(sanitized, tmp_path):
    lib, rt = sanitized
    exe = str(tmp_path / "abi_consumer")
    os.symlink(lib, str(tmp_path / "libnvfp4.so"))
    subprocess.run([os.path.join(LLVM, "clang"), "-std=c99", "-g", *SAN_LINK, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", exe, "-L", str(tmp_path), "-lnvfp4",
                    f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{rt}"], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=_env(rt, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi consumer ok" in r.stdout and "Sanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("nm") is None, reason="needs nm")
def test_validation_tests_clean(sanitized):
    """tests/test_abi.py in a process with the ASan runtime preloaded and the instrumented library loaded
    (the interpreter's own allocations are not leak-checked: detect_leaks=0)."""
    lib, rt = sanitized
    probe = ("import nvfp4_block_scaled_03_amd as nv, sys; "
             "maps = open('/proc/self/maps').read(); "
             "sys.exit(0 if nv.LIB_PATH == sys.argv[1] and sys.argv[1] in maps else 3)")
    env = _env(rt, LD_PRELOAD=os.path.join(rt, "libclang_rt.asan-x86_64.so"), NVFP4_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", probe, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, "the instrumented library was not the one loaded\n" + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "Sanitizer" not in r.stdout + r.stderr
