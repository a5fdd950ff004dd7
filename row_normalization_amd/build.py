"""Build ``librmsnorm.so`` (gfx950 kernels + host C ABI) in-tree.

``python -m row_normalization_amd.build`` or ``build()``.  The host TUs
(validation, planning, entry points of the RMSNorm and LayerNorm ABIs) are
compiled by g++, the kernels by hipcc for gfx950 only; hipcc links them into
one shared library next to this file.  Independent steps run in parallel.
Packed fp32 vector instructions are disabled in device code.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librmsnorm.so")
EXAMPLE_DIR = os.path.join(ROOT, "tests", "native", "bin")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 (v_pk_*_f32) instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


HOST_SOURCES = ("rmsnorm_api.cpp", "layernorm_api.cpp", "elementwise_api.cpp")
KERNEL_SOURCES = ("rmsnorm_kernels.hip", "layernorm_kernels.hip", "elementwise_kernels.hip")


def build(verbose: bool = True) -> str:
    """Compile the library; returns its path.  Always recompiles."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    objects, compile_steps = [], []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        objects.append(obj)
        compile_steps.append(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                              f"-I{INCLUDE}", f"-I{os.path.join(ROCM, 'include')}", "-c", os.path.join(CSRC, src),
                              "-o", obj])
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objects.append(obj)
        compile_steps.append([hipcc, *HIP_FLAGS, f"-I{INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj])
    for cmd in compile_steps:
        if verbose:
            print("+", " ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=len(compile_steps)) as pool:
        for f in [pool.submit(_run, cmd) for cmd in compile_steps]:
            f.result()
    tmp = LIB + ".tmp"
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp]
    if verbose:
        print("+", " ".join(link), flush=True)
    _run(link)
    os.replace(tmp, LIB)
    # a plain C++ caller of the ABI, run by the GPU tests (tests/native/abi_example.cpp)
    os.makedirs(EXAMPLE_DIR, exist_ok=True)
    example = [
        "g++", "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
        f"-I{os.path.join(ROCM, 'include')}", os.path.join(ROOT, "tests", "native", "abi_example.cpp"),
        "-o", os.path.join(EXAMPLE_DIR, "abi_example"), f"-L{PKG}", "-lrmsnorm", f"-L{os.path.join(ROCM, 'lib')}",
        "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,$ORIGIN/../../../row_normalization_amd",
        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
    ]
    if verbose:
        print("+", " ".join(example), flush=True)
    _run(example)
    # the planner's exhaustive check; with --widths it lists the widths at
    # which the GPU tests run every row shape the planner can emit
    plan_check = ["g++", "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
                  f"-I{os.path.join(ROCM, 'include')}", f"-I{CSRC}",
                  os.path.join(ROOT, "tests", "native", "plan_check.cpp"), "-o", os.path.join(EXAMPLE_DIR, "plan_check")]
    if verbose:
        print("+", " ".join(plan_check), flush=True)
    _run(plan_check)
    # the streaming-ceiling probe bench.py reports beside the kernels
    # (tests/native/stream_ceiling.hip)
    probe = [hipcc, *HIP_FLAGS, os.path.join(ROOT, "tests", "native", "stream_ceiling.hip"),
             "-o", os.path.join(EXAMPLE_DIR, "stream_ceiling")]
    if verbose:
        print("+", " ".join(probe), flush=True)
    _run(probe)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
