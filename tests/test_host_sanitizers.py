"""Host code under the compilers' sanitizers (CPU only; no GPU code is built
with a sanitizer).

* The planner's worker pool, stress-tested in a small C++ program, plain and
  under ThreadSanitizer: thousands of batches of random sizes, each item
  counted, with a second thread calling the same pool.
* The library's host code (the C ABI and the planner) built with the host
  compiler under AddressSanitizer and UndefinedBehaviorSanitizer, the kernel
  launchers replaced by stubs, and loaded by the Python face (SKV_LIBRARY)
  while the ABI tests and a share of the planner parity tests run.
"""
import os
import shutil
import subprocess
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
CSRC = os.path.join(ROOT, "split_kv_partial_amd", "csrc")
GXX = shutil.which("g++")

pytestmark = pytest.mark.skipif(GXX is None, reason="needs the host C++ compiler")


def _build(out, sources, flags):
    cmd = [GXX, "-std=c++17", "-g", "-pthread", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *flags, *sources, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


@pytest.mark.parametrize("mode", ["plain", "tsan"])
def test_sim_pool_stress(tmp_path, mode):
    exe = str(tmp_path / f"pool_{mode}")
    flags = ["-O2"] if mode == "plain" else ["-O1", "-fsanitize=thread"]
    _build(exe, [os.path.join(TESTS, "csrc", "sim_pool_stress.cpp")], flags)
    batches = "20000" if mode == "plain" else "3000"
    r = subprocess.run([exe, batches, "8"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert " bad 0 " in r.stdout


# the planner parity tests run against the sanitized build: the closed-form
# Figure 8 checks, the small benchmark workloads, thread and size stress, and
# a spread of the random batches (every tenth seed); the large workloads'
# parity runs against the regular build only (its time is the pure-Python
# reference's, which the sanitizers do not touch)
PARITY = ["test_fig8_through_the_abi", "test_benchmark_workloads_bit_exact[1]",
          "test_benchmark_workloads_bit_exact[2]", "test_concurrent_planners_agree",
          "test_large_skewed_batches", "test_default_cap_benchmark_workload_2_bit_exact"]


def test_host_library_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libsplitkv_host_asan.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _build(lib, [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "planner.cpp"),
                 os.path.join(TESTS, "csrc", "launch_stubs.cpp")],
           ["-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fPIC", "-shared",
            "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
            "-L", os.path.join(rocm, "lib"), f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-lamdhip64"])
    asan_rt = subprocess.run([GXX, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.isabs(asan_rt) and os.path.exists(asan_rt), asan_rt
    env = dict(os.environ, SKV_LIBRARY=lib, LD_PRELOAD=asan_rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    sel = [os.path.join(TESTS, "test_abi.py")]
    sel += [f"{os.path.join(TESTS, 'test_planner_parity.py')}::{t}" for t in PARITY]
    sel += [f"{os.path.join(TESTS, 'test_planner_parity.py')}::test_random_batches_bit_exact[{s}]"
            for s in range(0, 160, 10)]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *sel],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=1200)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    # the sanitized build is the one that was loaded
    probe = subprocess.run([sys.executable, "-c", "import split_kv_partial_amd as s; print(s.LIB_PATH)"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr[-2000:]
