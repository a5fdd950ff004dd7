"""Host logic on the CPU: an exhaustive native check of every launch plan
(tests/native/plan_check.cpp) and a brute-force check of the exact strided
overlap test (tests/native/overlap_check.cpp), both compiled here with g++
against csrc/host_plan.h."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_native(tmp_path, name):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{os.environ.get('ROCM_PATH', '/opt/rocm')}/include",
                    f"-I{ROOT}/row_normalization_amd/csrc", os.path.join(ROOT, "tests", "native", name + ".cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert " 0 bad" in r.stdout


def test_every_plan_is_valid(tmp_path):
    _run_native(tmp_path, "plan_check")


def test_strided_overlap_is_exact(tmp_path):
    _run_native(tmp_path, "overlap_check")
