"""Builds libmpgemm.so (the C-ABI library: planner + gfx950 HIP kernels) in-tree.

    python -m mixed_precision_gemm_amd.build [--verbose]
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmpgemm.so")
SOURCES = ["gemm_plan.cpp", "gemm_kernels.hip", "attention_kernels.hip"]
# gemm_kernels.hip is compiled in parts, in parallel: part 0 is the host code
# and the kernel table, parts 1-4 the GEMM kernels of one input type and
# epilogue flag each (see the top of that file).
KERNEL_PARTS = 5
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-fp32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src, obj, defines, extra_flags, verbose):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *defines, "-I", INCLUDE,
           "-I", CSRC, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l)   # host-pass notice
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defines)}:\n{errs}")
    return " ".join(cmd), errs


def build(verbose: bool = False, extra_flags=None) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        stem = os.path.splitext(src)[0]
        if src == "gemm_kernels.hip":
            for part in range(KERNEL_PARTS):
                jobs.append((src, os.path.join(bdir, f"{stem}_part{part}.o"),
                             [f"-DMPGEMM_PART={part}"]))
        else:
            jobs.append((src, os.path.join(bdir, stem + ".o"), []))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_compile, s, o, d, extra_flags, verbose) for s, o, d in jobs]
        for f in futs:
            cmd, errs = f.result()
            if verbose:
                print(cmd, flush=True)
                if errs.strip():
                    print(errs, file=sys.stderr)
    objs = [o for _, o, _ in jobs]
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
