"""Builds libmsa.so in-tree: the host validation unit with g++, the gfx950
kernels with hipcc, linked into one shared library next to this file; and
libmsa_probe.so, the benchmark's ceiling probes (streaming read, streaming
copy, MFMA loop)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libmsa.so")
# The benchmark's ceiling probes (measured HBM read and copy ceilings, MFMA
# loop), a separate object: nothing in libmsa uses it.
PROBE_LIBRARY = os.path.join(PKG, "libmsa_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# Kernel sources (each with its entry points), sharing msa_device.h.
KERNEL_SOURCES = ("msa_decode.hip", "msa_prefill.hip", "msa_backward.hip", "msa_project.hip",
                  "msa_noalloc.hip")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # hipcc forms packed fp32 instructions from plain float code on its own;
    # keep them off so every fp32 op is a scalar VALU op.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compiles every source and replaces libmsa.so atomically; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    run = (lambda cmd: subprocess.check_call(cmd)) if verbose else (
        lambda cmd: subprocess.run(cmd, check=True, stdout=subprocess.PIPE,
                                   stderr=subprocess.STDOUT))
    host_o = os.path.join(BUILD_DIR, "msa_host.o")
    try:
        run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
             "-c", os.path.join(CSRC, "msa_host.cpp"), "-o", host_o])
        kern_o = []
        for name in KERNEL_SOURCES:
            obj = os.path.join(BUILD_DIR, name.replace(".hip", ".o"))
            run([_hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
                 os.path.join(CSRC, name), "-o", obj])
            kern_o.append(obj)
        tmp = LIBRARY + ".tmp%d" % os.getpid()
        run([_hipcc(), "-shared", "-fPIC"] + kern_o + [host_o, "-o", tmp,
             "-Wl,-rpath,/opt/rocm/lib"])
        probe_tmp = PROBE_LIBRARY + ".tmp%d" % os.getpid()
        run([_hipcc()] + HIPCC_FLAGS + ["-shared", os.path.join(CSRC, "read_probe.hip"), "-o",
                                        probe_tmp, "-Wl,-rpath,/opt/rocm/lib"])
    except subprocess.CalledProcessError as exc:
        out = exc.stdout.decode(errors="replace") if exc.stdout else ""
        raise RuntimeError("libmsa build failed:\n" + out) from exc
    os.replace(tmp, LIBRARY)
    os.replace(probe_tmp, PROBE_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
