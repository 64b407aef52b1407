"""Build libpa.so in-tree for gfx950 with hipcc (host checks with g++).

    python -m paged_kv_cache_size_amd.build

Always recompiles.  The shared library lands next to this file, where the
binding loads it from.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 instructions are kept out of the device code (the compiler would
# otherwise form v_pk_* f32 operations from plain float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA accumulators in ordinary VGPRs: the softmax rescale multiplies them in place
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libpa needs the ROCm toolchain to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")
    if verbose and res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
        lines = [x for x in res.stderr.splitlines() if "packed-fp32-ops" not in x]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        host_objs, dev_objs, steps = [], [], []
        for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp")):
            obj = os.path.join(tmp, src[:-4] + ".o")
            steps.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
                          os.path.join(CSRC, src), "-o", obj])
            host_objs.append(obj)
        for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
            obj = os.path.join(tmp, src[:-4] + ".o")
            steps.append([hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", *DEVICE_FLAGS,
                          "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
            dev_objs.append(obj)
        # the translation units compile independently: one process each, a few at a time
        workers = max(1, min(len(steps), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            for fut in [pool.submit(_run, cmd, verbose) for cmd in steps]:
                fut.result()
        out_tmp = LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *host_objs, *dev_objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
