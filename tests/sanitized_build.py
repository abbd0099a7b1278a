"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds of the
library's host code (host.cpp and the host half of kernels.hip; the device
half is compiled without sanitizers and never launched) and of the oracle (oracle.c), for the CPU test
tier.  All three use clang's shared sanitizer runtime, which the test process
preloads.  CPU only: nothing here is built for or run on a GPU."""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "complexity_half_precision_amd", "csrc")
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def runtime() -> str:
    out = subprocess.run([f"{LLVM}/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(out):
        import glob
        hits = glob.glob(f"{LLVM}/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so")
        out = hits[0]
    return out


def build(out_dir: str) -> dict:
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in ("host.cpp", "kernels.hip"):
        obj = os.path.join(out_dir, src + ".o")
        if src == "kernels.hip":
            # its host half is launch glue only; the in-tree object, when it is
            # newer than the source, saves compiling the device code again
            built = os.path.join(ROOT, "complexity_half_precision_amd", "_build", "kernels.hip.o")
            if os.path.exists(built) and os.path.getmtime(built) >= os.path.getmtime(os.path.join(CSRC, src)):
                objs.append(built)
                continue
        # the sanitizer flags apply to the host compilation only (-Xarch_host);
        # the device code is compiled as usual and never run here
        cmd = [HIPCC, "-std=c++20", "-fPIC", "--offload-arch=gfx950", "-O1",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               *[f for flag in SAN for f in ("-Xarch_host", flag)],
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-command-line-argument",
               "-c", os.path.join(CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "liblcma_san.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address,undefined",
                    *objs, "-o", lib], check=True, capture_output=True, text=True)
    olib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run([f"{LLVM}/bin/clang", "-std=c11", "-fPIC", "-shared", "-shared-libsan", "-fopenmp",
                    "-ffp-contract=off", *SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o", olib, "-lm"],
                   check=True, capture_output=True, text=True)
    return {"lcma": lib, "oracle": olib, "runtime": runtime()}
