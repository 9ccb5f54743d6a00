"""CPU: the oracle and the library's host-side argument validation under
AddressSanitizer and UndefinedBehaviorSanitizer.

- tests/c/oracle_sanitize.c drives every oracle entry point on small inputs and
  edge cases, built with oracle/oasis_oracle.c by gcc with both sanitizers
  (leak detection on);
- tests/c/abi_validate.c calls every entry point of include/oasis.h with
  invalid and extreme arguments, linked against a build of the library whose
  host code of every unit carries both sanitizers (device code as usual; no
  GPU is touched: every call is refused before anything is enqueued).

A control first shows that each toolchain's sanitizers report a planted heap
overflow and a planted signed overflow, so a silent run means a clean one."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lookahead_sparse_kv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")

PLANTED = r"""
#include <stdio.h>
#include <stdlib.h>
int main(int argc, char **argv) {
    (void)argv;
    if (argc > 1) { int x = 2147483600 + argc * 100; printf("%d\n", x); return 0; }
    int *p = (int *)malloc(4 * sizeof(int));
    p[argc + 3] = 1;                       /* one past the end */
    printf("%d\n", p[0]);
    free(p);
    return 0;
}
"""


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


@pytest.mark.slow
@pytest.mark.parametrize("cc", ["gcc", CLANG])
def test_the_sanitizers_report_planted_mistakes(tmp_path, cc):
    if shutil.which(cc) is None and not os.path.exists(cc):
        pytest.skip(f"{cc} not found")
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    exe = tmp_path / "planted"
    b = _run([cc, "-g", "-O0", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              str(src), "-o", str(exe)])
    assert b.returncode == 0, b.stderr
    heap = _run([str(exe)], env=SAN_ENV)
    assert heap.returncode != 0 and "AddressSanitizer" in heap.stderr
    over = _run([str(exe), "x"], env=SAN_ENV)
    assert over.returncode != 0 and "runtime error" in over.stderr


@pytest.mark.slow
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    b = _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
              "-ffp-contract=off", "-Wall", "-Wextra", "-Werror", "-o", str(exe),
              os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
              os.path.join(ROOT, "oracle", "oasis_oracle.c"), "-lm"])
    assert b.returncode == 0, b.stderr
    r = _run([str(exe)], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1:exitcode=23"), timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitize ok" in r.stdout


@pytest.mark.slow
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("no ROCm toolchain")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    # host code of every unit with both sanitizers; the device code is built
    # as usual (packed fp32 off) but never runs here
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = [(s, subprocess.Popen([HIPCC, *flags, "-c", s, "-o",
                                   str(tmp_path / (os.path.basename(s) + ".o"))],
                                  stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
             for s in srcs]
    for s, p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}:\n{err}"
    drv = tmp_path / "drv.o"
    b = _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
              "-I", os.path.join(ROOT, "include"), "-c",
              os.path.join(ROOT, "tests", "c", "abi_validate.c"), "-o", str(drv)])
    assert b.returncode == 0, b.stderr
    exe = tmp_path / "abi_validate"
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    b = _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", str(drv), *objs, "-o", str(exe)])
    assert b.returncode == 0, b.stderr
    # the HIP runtime keeps allocations until exit: leak reports would be its own
    r = _run([str(exe)], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:exitcode=23"), timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi validation ok" in r.stdout
