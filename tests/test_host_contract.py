"""Host side of every entry point under AddressSanitizer and UBSan (CPU).

tests/native/host_contract.cpp replaces the kernel launchers with stubs that
check what the host hands the kernels, and drives every entry point over a
grid of valid shapes, dtypes, strides, flags and aliasing cases; it is linked
with the library's own host translation units (csrc/*_api.cpp), all built
here with g++ and the sanitizers (no device code is involved)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "row_normalization_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_host_contract_under_sanitizers(tmp_path):
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    srcs = [os.path.join(CSRC, f) for f in ("rmsnorm_api.cpp", "layernorm_api.cpp", "elementwise_api.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "native", "host_contract.cpp"))
    exe = str(tmp_path / "host_contract")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
                    f"-I{rocm_inc}", f"-I{CSRC}", *srcs, "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 bad" in r.stdout, r.stdout
