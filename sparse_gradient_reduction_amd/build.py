"""Build libsparcml.so (HIP kernels + C ABI) and libsparcml_bench.so (the
measurement-only bandwidth reference) for gfx950, in-tree.

    python -m sparse_gradient_reduction_amd.build
"""
import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsparcml.so")
BENCH_LIB = os.path.join(PKG, "libsparcml_bench.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "topk_ef.hip", "topk_row.hip", "topk_bucketed.hip", "qsgd.hip", "sparse_reduce.hip"]
BENCH_SOURCES = ["reference_stream.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # bit-reproducible fp32: no contraction into FMA, no fast-math, denormals kept
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    subprocess.run([hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, out)


def build(jobs: int = 4) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(_compile, SOURCES + BENCH_SOURCES))
    except subprocess.CalledProcessError as e:
        raise RuntimeError(f"hipcc failed:\n{e.stdout.decode(errors='replace')}") from e
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
