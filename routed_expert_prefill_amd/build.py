"""Build the gfx950 shared library ``libmoe_prefill.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only.  Packed-fp32 instructions are
disabled at the target-feature level; no fast-math flag is used, so fp32
division and square root stay correctly rounded (the fp8 quantiser relies on
IEEE division).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_prefill.so")

HIP_SOURCES = ["route_topk.hip", "route_build.hip", "combine.hip", "quant.hip", "ffn_grouped.hip",
               "ffn_fp8.hip"]
HOST_SOURCES = ["api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile all sources and link the shared library; returns its path.

    defines: extra -D flags (tuning knobs; the defaults are the shipped values).
    """
    os.makedirs(build_dir, exist_ok=True)
    extra = ["-D" + d for d in defines]
    cc = hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([cc, *COMMON, *extra, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        jobs.append([cc, *COMMON, *extra, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        for log in ex.map(_run, jobs):
            if verbose and log.strip():
                print(log)
    objs = [j[-1] for j in jobs]
    tmp = out + ".tmp"
    _run([cc, "-shared", "--offload-arch=gfx950", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


# Host-side sanitizers for the C ABI layer only: AddressSanitizer and
# UndefinedBehaviorSanitizer apply to the host pass of api.cpp (each flag
# behind -Xarch_host, so no GPU code is instrumented); the kernels are the
# normal gfx950 objects.  The result is loaded with the clang ASan runtime
# preloaded (sanitizer_runtime()) by the CPU tests of the ABI.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer"]


def sanitizer_runtime():
    """Path of the clang ASan runtime shared library of the ROCm toolchain, or None."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_sanitized(out_dir: str = os.path.join(BUILD, "host_sanitized")) -> str:
    """libmoe_prefill.so with the host code of api.cpp built under ASan and
    UBSan; returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        _run([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    api = os.path.join(out_dir, "api.cpp.o")
    _run([cc, *[f for f in COMMON if f != "-O3"], "-O1", "-g", *DEVICE, *HOST_SANITIZE, "-x", "hip",
          "-c", os.path.join(CSRC, "api.cpp"), "-o", api])
    lib = os.path.join(out_dir, "libmoe_prefill.so")
    _run([cc, "-shared", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, api, *objs])
    return lib


def kernel_resource_report(src: str) -> dict:
    """Per-kernel resource usage of one HIP source compiled for gfx950, from
    the compiler's kernel-resource-usage remarks: {kernel: {field: value}}."""
    import re

    cmd = [hipcc(), *COMMON, *DEVICE, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(CSRC, src), "-o", os.devnull]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + p.stdout)
    out, cur = {}, None
    for line in p.stdout.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
        if m and cur is not None:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
