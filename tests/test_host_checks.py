"""Host-side checks that need no GPU.

* Every gfx950 kernel of the library compiles with no scratch (private
  segment) memory and no register spills, so the hot loops keep all their
  state in registers; the grouped GEMMs also keep two waves per SIMD.
* The C ABI layer built with AddressSanitizer and UndefinedBehaviorSanitizer
  on its host code passes the ABI tests (every argument check and error
  path) with the sanitizer runtime preloaded.
"""
import os
import subprocess
import sys

import pytest

from routed_expert_prefill_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("src", B.HIP_SOURCES)
def test_kernels_use_no_scratch_and_do_not_spill(src):
    rep = B.kernel_resource_report(src)
    assert rep, f"no kernels reported for {src}"
    for kern, r in rep.items():
        assert r["ScratchSize"] == 0, (kern, r)
        assert r["SGPRs Spill"] == 0, (kern, r)
        assert r["VGPRs Spill"] == 0, (kern, r)
        if "grouped_gemm" in kern:
            assert r["Occupancy"] >= 2, (kern, r)  # two waves per SIMD cover each other


def test_abi_under_host_sanitizers():
    rt = B.sanitizer_runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = B.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host code is instrumented
    env = dict(os.environ, MOE_PREFILL_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    which = subprocess.run([sys.executable, "-c", "from routed_expert_prefill_amd import _lib; "
                            "print(_lib.load()._name)"], cwd=ROOT, env=env, text=True,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=120)
    assert which.stdout.strip().endswith(lib), which.stdout  # the tests load that build
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "passed" in p.stdout and "AddressSanitizer" not in p.stdout and \
        "runtime error" not in p.stdout, p.stdout[-4000:]
