"""Sanitizer builds, on the CPU.

- The oracle (plain C) under AddressSanitizer + UndefinedBehaviorSanitizer and
  under ThreadSanitizer, driven by tests/oracle_stress.c over random verify,
  diagnostics, decode and cascade shapes (k2 below, equal to and above k1),
  NaN/+inf rows, invalid temperatures and draft tokens, layout errors and
  every planted-mistake branch; the first report ends the run.
- A negative control: the same build with an inner-draft buffer of the cascade
  sized for k1 instead of k2 must be reported.
- The host code of libspecverify under ASan + UBSan (its device code built
  at -O0 only to link, never run), driven by tests/abi_stress.c through the argument
  checks of the C ABI: extreme shape fields, workspace queries of every entry
  point, null/misaligned/fake pointers, short workspaces and the no-allocation
  entry point's scratch limit, all refused before anything is enqueued.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
ORACLE_C = ROOT / "oracle" / "specv_oracle.c"
STRESS_C = ROOT / "tests" / "oracle_stress.c"
ABI_C = ROOT / "tests" / "abi_stress.c"
HIP_SOURCE = ROOT / "speculative_sampling_verify_amd" / "csrc" / "specverify.hip"
ROCM = Path(os.environ.get("ROCM_PATH", "/opt/rocm"))
CLANG = ROCM / "llvm" / "bin" / "clang"

SAN_ENV = {
    "ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1",
}
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
           "ERROR: LeakSanitizer")


def need(tool):
    path = shutil.which(tool) if "/" not in str(tool) else (str(tool) if Path(tool).exists() else None)
    if not path:
        pytest.skip("%s not available" % tool)
    return path


def compile_or_skip(cmd, what):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        err = res.stderr
        if "cannot find -l" in err and any(r in err for r in ("asan", "tsan", "ubsan")):
            pytest.skip("%s: sanitizer runtime missing" % what)
        raise AssertionError("%s failed:\n%s\n%s" % (what, " ".join(map(str, cmd)), err[-4000:]))


def run_clean(cmd, timeout=300):
    env = dict(os.environ, **SAN_ENV)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True, env=env,
                         timeout=timeout)
    reports = [r for r in REPORTS if r in res.stderr]
    assert res.returncode == 0 and not reports, (
        "%s: exit %d, reports %s\n%s" % (cmd, res.returncode, reports, res.stderr[-6000:]))
    return res.stdout


def oracle_build(out, sanitize, source=ORACLE_C):
    gcc = need("gcc")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=" + sanitize,
           "-fno-sanitize-recover=all", "-pthread", "-I", str(ROOT / "oracle"), str(STRESS_C),
           str(source), "-o", str(out), "-lm"]
    compile_or_skip(cmd, "oracle build (%s)" % sanitize)
    return out


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitizers")


def test_oracle_address_undefined(workdir):
    exe = oracle_build(workdir / "oracle_asan", "address,undefined")
    for seed in (1, 2, 3, 4):
        out = run_clean([exe, 40, seed])
        assert "40 cases ok" in out


def test_oracle_thread(workdir):
    exe = oracle_build(workdir / "oracle_tsan", "thread")
    for seed in (5, 6):
        out = run_clean([exe, 20, seed])
        assert "20 cases ok" in out


def test_planted_cascade_overflow_is_reported(workdir):
    # the inner draft tokens of a cascade packed into a buffer sized for k1:
    # with k2 > k1 the inner review writes past it
    text = ORACLE_C.read_text()
    right = "int32_t* ipack = (int32_t*)malloc((size_t)(B * k2 + 1) * 4);"
    assert right in text
    src = workdir / "specv_oracle_planted.c"
    src.write_text(text.replace(right, right.replace("k2", "k1")))
    exe = oracle_build(workdir / "oracle_planted", "address,undefined", source=src)
    env = dict(os.environ, **SAN_ENV)
    caught = False
    for seed in (1, 2, 3, 4):
        res = subprocess.run([str(exe), "40", str(seed)], capture_output=True, text=True, env=env,
                             timeout=300)
        if res.returncode != 0 and "heap-buffer-overflow" in res.stderr:
            assert "oracle_cascade_bigram" in res.stderr
            caught = True
            break
    assert caught, "the planted overflow went unreported"


def test_host_library_address_undefined(workdir):
    hipcc = need(str(ROCM / "bin" / "hipcc"))
    clang = need(str(CLANG))
    lib = workdir / "libspecverify_san.so"
    # device code at -O0 (it only has to link; nothing is launched), host code
    # instrumented: each sanitizer flag applies to the host pass alone
    compile_or_skip([hipcc, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-g0",
                     "-std=c++17", "-fPIC", "-shared", "-Xarch_host", "-g",
                     "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-fno-sanitize-recover=all",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-I", str(ROOT / "include"), "-I", str(HIP_SOURCE.parent), str(HIP_SOURCE),
                     "-o", str(lib)], "host library build")
    exe = workdir / "abi_stress"
    compile_or_skip([clang, "-O1", "-g", "-fsanitize=address,undefined",
                     "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
                     "-I", str(ROOT / "include"), "-I", str(ROCM / "include"), str(ABI_C),
                     "-o", str(exe), str(lib), "-L", str(ROCM / "lib"), "-lamdhip64",
                     "-Wl,-rpath," + str(workdir), "-Wl,-rpath," + str(ROCM / "lib")],
                    "ABI driver build")
    for seed in (1, 2, 3):
        out = run_clean([exe, 30000, seed])
        assert "30000 cases ok" in out
