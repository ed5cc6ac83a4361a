"""The host side of the C ABI (argument validation, workspace planning, the
layer tables) under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled again with the sanitizers on its
host code only (device code as usual), linked into a library of its own, and
the ABI tests of test_abi_cpu.py run against it in a child process with the
ASan runtime preloaded (ARK_LIBRARY selects the build).  No GPU is needed:
those tests stop at validation or at the first HIP call.  A report from
either sanitizer fails the test."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speech_decoder_int8_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and _asan_runtime()):
        pytest.skip("hipcc, clang++ or the ASan runtime is missing")
    out = tmp_path_factory.mktemp("ark_san")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", *HOST_SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-2000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(out, "libark_san.so")
    r = subprocess.run([CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libsan", "-o", lib,
                        *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    yield lib
    shutil.rmtree(out, ignore_errors=True)


def test_library_is_instrumented(sanitized_lib):
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is missing")
    r = subprocess.run([nm, "-D", "--undefined-only", sanitized_lib], capture_output=True, text=True)
    assert r.returncode == 0
    assert "__asan_report_load" in r.stdout and "__ubsan_handle" in r.stdout


def test_abi_validation_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env.update(ARK_LIBRARY=sanitized_lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    script = ("import sys, pytest\n"
              "from speech_decoder_int8_amd import ark\n"
              f"assert ark.LIB_PATH == {sanitized_lib!r}, ark.LIB_PATH\n"
              "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
              f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    r = subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert r.returncode == 0 and " passed" in report, report[-4000:]
