"""Build libmq.so (HIP, gfx950) in-tree.

Every .hip / .cpp file under csrc/ is compiled with hipcc for gfx950 and the
objects are linked into quant_gemm_amd/libmq.so. The library is linked
against the HIP runtime that PyTorch ships (torch/lib/libamdhip64.so), with a
run path to it, so that a process that imports torch and loads libmq holds a
single HIP runtime: stream handles and device pointers from torch are then
valid in libmq.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmq.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Kernel code generation flags:
#  - packed fp32 instructions are disabled (the compiler would otherwise form
#    v_pk_* f32 ops from scalar code);
#  - f32 division and sqrt are correctly rounded and f32 denormals are kept,
#    so the activation quantizer is bit-exact against a host IEEE evaluation;
#  - no fast-math.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    "-Wall", "-Wno-unused-function",
]


def torch_lib_dir() -> str:
    """Directory of torch's bundled HIP runtime (found without importing torch)."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is not importable: cannot find its HIP runtime")
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {d}")
    return d


# Per-file code generation: the machine scheduler's max-ILP strategy for the
# Q4_K prefill GEMM unit. Measured on MI355X, same-box A/B at M=3314,
# N=18944, K=3584: 785 against 797 us (plain), and 1.4-1.6% for its
# decoded-scale and fused-FFN forms. Not for the Q6_K unit (its raw-block
# GEMM ran 5-6% slower, its planes GEMM 2% faster only at M=512), Q5_K
# (one more spilled register), the 32-token tiles (more VGPRs) or the
# decode kernels (mixed).
FILE_FLAGS = {
    "gemm_q4k.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def kernel_flags(src: str) -> list:
    """The hipcc flags a kernel source file is compiled with."""
    return [*HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *kernel_flags(src), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *kernel_flags(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tl = torch_lib_dir()
    tmp = LIB + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp, *objs, f"-L{tl}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{tl}", "-Wl,--no-undefined", "-Wl,-z,defs"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probes(verbose)
    return LIB


PROBES_SRC = os.path.join(HERE, "probes", "probes.hip")
PROBES_LIB = os.path.join(HERE, "libmq_probes.so")


def build_probes(verbose: bool = False) -> str:
    """libmq_probes.so: the ceiling probes bench.py --ceilings measures (a
    separate library; nothing of it is linked into libmq.so)."""
    tl = torch_lib_dir()
    tmp = PROBES_LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-shared", PROBES_SRC, "-o", tmp, f"-L{tl}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{tl}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBES_LIB)
    if verbose:
        print(f"built {PROBES_LIB}")
    return PROBES_LIB


def clean() -> None:
    shutil.rmtree(os.path.join(ROOT, "_build"), ignore_errors=True)
    for lib in (LIB, PROBES_LIB):
        if os.path.exists(lib):
            os.remove(lib)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
