"""The launch planner on the CPU: an exhaustive native check of every plan
(tests/native/plan_check.cpp, compiled here with g++ against csrc/host_plan.h)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_plan_is_valid(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{os.environ.get('ROCM_PATH', '/opt/rocm')}/include",
                    f"-I{ROOT}/row_normalization_amd/csrc", os.path.join(ROOT, "tests", "native", "plan_check.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert "0 bad" in r.stdout
