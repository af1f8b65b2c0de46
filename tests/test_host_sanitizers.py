"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is built host-only (no device code, no HIP runtime) with both sanitizers
and linked into `host_sanitize/abi_driver.c`, which defines every HIP function the
library imports as a counting test double (failing, then succeeding).  The driver
runs the documented argument errors of every entry point, valid calls of each, a
profiling window, and a seeded fuzz of descriptors and parameters; it checks the
statuses, that no argument error makes a HIP call, that a failing HIP call always
surfaces as MR_ERR_DEVICE, and that every launch fits gfx950's launch limits.  Any
sanitizer report aborts it.  A deliberate over-read (a graph call that declares more
edges than its host list holds) shows that the instrumentation is live.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "dense_grounded_image_amd", "csrc", "mr.hip")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                                reason="needs ROCm's hipcc and clang++ (host compilation only)")

ENV_KEYS = ("ASAN_OPTIONS", "UBSAN_OPTIONS", "LSAN_OPTIONS")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("host_sanitize")
    fatbin = d / "empty.fatbin"   # no device code: an empty offload bundle is embedded
    fatbin.write_bytes(b"")
    lib = d / "libmr_san.so"
    lib_cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-no-hip-rt", "-O1", "-g", "-std=c++17",
               "-fPIC", "-shared",
               "-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(fatbin),
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), SRC, "-o", str(lib)]
    r = subprocess.run(lib_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = d / "abi_driver"
    exe_cmd = [CLANGXX, "-x", "c", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
               "-I", os.path.join(ROOT, "include"), DRIVER, "-L", str(d), "-lmr_san",
               "-Wl,-rpath," + str(d), "-o", str(exe)]
    r = subprocess.run(exe_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    yield str(exe)
    shutil.rmtree(d, ignore_errors=True)


def _run(exe, *args):
    env = {k: v for k, v in os.environ.items() if k not in ENV_KEYS}
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)


def test_validation_and_launch_setup_are_sanitizer_clean(driver):
    r = _run(driver, "20000")
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "LeakSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-4000:])
    fields = r.stdout.split()
    stats = dict(zip(fields[0::2], fields[1::2]))
    assert stats["failures"] == "0" and stats["bad_launches"] == "0"
    # the fuzz reached the launch code, not only the validation
    assert int(stats["launches"]) > 10000 and int(stats["hip_calls_failing"]) > 100


def test_sanitizer_sees_an_over_read(driver):
    r = _run(driver, "overflow")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
    assert "mr_fast_reciprocal_graph" in r.stderr


def test_launch_log(driver):
    """MR_LOG=1 prints each call with its maps, each launch, and each returned status;
    without it the library prints nothing."""
    r = _run(driver, "log")
    assert r.returncode == 0, r.stderr[-3000:]
    assert "[mr]" not in r.stderr
    env_run = subprocess.run([driver, "log"], capture_output=True, text=True, timeout=120,
                             env={**{k: v for k, v in os.environ.items() if k not in ENV_KEYS}, "MR_LOG": "1"})
    assert env_run.returncode == 0, env_run.stderr[-3000:]
    stats = dict(zip(env_run.stdout.split()[0::2], env_run.stdout.split()[1::2]))
    lines = env_run.stderr.splitlines()
    launches = [l for l in lines if l.startswith("[mr]   launch ")]
    entries = [l for l in lines if l.startswith("[mr] mr_") and " -> " not in l]
    statuses = [l for l in lines if l.startswith("[mr] mr_") and " -> " in l]
    assert len(launches) == int(stats["launches"]) > 0
    assert len(entries) == len(statuses) == int(stats["calls"])
    # every valid call returns ok, the argument error its status; launches carry shapes
    assert sum(l.endswith("-> 0 (ok)") for l in statuses) == len(statuses) - 1
    assert statuses[-1].startswith("[mr] mr_nn_argmax -> 4 ")
    assert all(" grid (" in l and " block (" in l for l in launches)
    assert any("rowcol_argmax_kernel" in l for l in launches)
    assert entries[0].startswith("[mr] mr_nn_argmax a 1x40x30x24 f32")
