"""Build librht.so (and the benchmark's libstream_ceiling.so) in-tree: hipcc for gfx950,
no JIT, no torch extension."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librht.so")
# trivial streaming kernels the benchmark times as the achievable ceiling of
# the KV-block shapes (not part of librht or its ABI)
CEIL_SRC = os.path.join(HERE, "bench_kernels", "stream_ceiling.hip")
CEIL_LIB = os.path.join(HERE, "libstream_ceiling.so")
ARCH = os.environ.get("RHT_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions stay off: hipcc -O3 would otherwise form
# v_pk_add/mul/fma_f32 from scalar float code.
# MFMA accumulators are kept in ordinary VGPRs (the results feed VALU code
# directly instead of going through v_accvgpr_read).
DEVICE_FLAGS = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=" + ARCH,
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wall"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs, objs = [], []
    for src in sorted(os.listdir(CSRC)):
        stem, ext = os.path.splitext(src)
        if ext not in (".hip", ".cpp"):
            continue
        obj = os.path.join(BUILD, stem + ".o")
        flags = DEVICE_FLAGS if ext == ".hip" else HOST_FLAGS
        jobs.append(["hipcc"] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    ceil_tmp = CEIL_LIB + ".tmp%d" % os.getpid()
    jobs.append(["hipcc"] + DEVICE_FLAGS + ["-shared", CEIL_SRC, "-o", ceil_tmp])
    with concurrent.futures.ThreadPoolExecutor(min(len(jobs), 8)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    os.replace(ceil_tmp, CEIL_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
