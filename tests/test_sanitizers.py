"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds made here, in a temporary folder, then the CPU tests that drive them run in a
child process with the sanitizer runtime preloaded (the Python interpreter itself is not
instrumented, so the runtime has to come first):

* the oracle (csa2_oracle.c) built by gcc with -fsanitize=address,undefined, under every
  oracle pin (tests/test_oracle_*.py);
* libcsa2.so with its host code (the C ABI's argument checks, workspace arithmetic and
  launch set-up) built by hipcc with the sanitizers applied to the host pass only
  (``-Xarch_host`` before each flag; device code is never instrumented), under
  tests/test_abi_host.py, which calls every entry point with good and bad arguments.

Undefined behaviour aborts (-fno-sanitize-recover) and so does the first ASan report, so
any finding fails the child run.  A last test plants an overflow and a signed overflow in
a scrap C program, built and run the same way, to show the runtimes do report.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from compressed_sparse_attention_fp4_amd import build_lib  # noqa: E402

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _gcc_runtime():
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    libs = [subprocess.run(["gcc", "-print-file-name=%s" % n], capture_output=True, text=True).stdout.strip()
            for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc sanitizer runtimes not found")
    return ":".join(libs)


def _clang_runtime():
    try:
        hipcc = build_lib.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm")
    found = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        pytest.skip("clang ASan runtime not found")
    return os.path.realpath(found[-1])


def _run_pytest(files, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + files
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    return out


def _loaded_in_child(env_extra, preload, code):
    """/proc/self/maps of a child that loads the library under the same preload."""
    env = dict(os.environ, **SAN_ENV, **env_extra, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, "-c", code + "\nprint(open('/proc/self/maps').read())"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("san"))


def test_oracle_pins_under_asan_ubsan(san_dir):
    preload = _gcc_runtime()
    lib = os.path.join(san_dir, "liboracle_asan.so")
    cmd = ["gcc", "-O1", "-g"] + GCC_SAN + ["-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                                            "-std=c11", "-D_GNU_SOURCE", "-Wall", "-o", lib,
                                            os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(CSA2_ORACLE_LIBRARY=lib)
    maps = _loaded_in_child(env, preload, "import oracle.oracle as o; o._load()")
    assert lib in maps and "libasan" in maps
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert len(pins) >= 5
    _run_pytest(pins, env, preload)


def test_abi_host_under_asan_ubsan(san_dir):
    preload = _clang_runtime()

    def compile_one(src):
        obj = os.path.join(san_dir, os.path.splitext(src)[0] + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        common = [f for f in build_lib.COMMON if f != "-O3"] + ["-O1", "-g"]
        cmd = ([build_lib.hipcc()] + common + build_lib.EXTRA.get(src, []) + SAN_HOST + lang
               + ["-c", os.path.join(build_lib.CSRC, src), "-o", obj])
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(min(len(build_lib.SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, build_lib.SOURCES))
    lib = os.path.join(san_dir, "libcsa2_asan.so")
    cmd = [build_lib.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(CSA2_LIBRARY=lib)
    maps = _loaded_in_child(env, preload, "from compressed_sparse_attention_fp4_amd import binding as B; B.lib()")
    assert lib in maps and "libclang_rt.asan" in maps
    _run_pytest([os.path.join(ROOT, "tests", "test_abi_host.py")], env, preload)


def test_sanitizers_report(san_dir):
    """A heap overflow and a signed overflow in a scrap program are reported and abort."""
    _gcc_runtime()
    src = os.path.join(san_dir, "planted.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\n#include <limits.h>\n"
                "int main(int argc, char** argv) {\n"
                "  if (argc > 1) { int* a = malloc(4 * sizeof(int)); volatile int i = 4; a[i] = 1; free(a); }\n"
                "  else { volatile int x = INT_MAX; x = x + argc; return x == 0; }\n"
                "  return 0;\n}\n")
    exe = os.path.join(san_dir, "planted")
    subprocess.run(["gcc", "-O0", "-g"] + GCC_SAN + ["-o", exe, src], check=True, capture_output=True)
    env = dict(os.environ, **SAN_ENV)
    env.pop("LD_PRELOAD", None)
    heap = subprocess.run([exe, "heap"], env=env, capture_output=True, text=True, timeout=60)
    assert heap.returncode != 0 and "heap-buffer-overflow" in heap.stderr
    ub = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=60)
    assert ub.returncode != 0 and "runtime error" in ub.stderr
