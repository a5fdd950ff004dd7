"""The streaming-ceiling probe bench.py reports beside the kernels
(tests/native/stream_ceiling.hip) runs and prints one well-formed JSON line:
for each read/write mix (read only, one read per write, two reads per write,
two reads per write in place, three reads with three writes) a best hot and cold rate, the shape that gave it
and the rate of every shape timed."""
import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(__file__), "native", "bin", "stream_ceiling")


def test_probe_reports_every_mix():
    print("case: stream_ceiling probe", flush=True)
    assert os.path.exists(PROBE), "built by row_normalization_amd.build"
    r = subprocess.run([PROBE], capture_output=True, text=True, timeout=170)
    assert r.returncode == 0, r.stderr
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["bytes_per_operand"] == 256 << 20
    for mix in ("read", "read1_write1", "read2_write1", "read2_write1_in_place", "read3_write3"):
        m = res[mix]
        shapes = m["hot_gbps_by_shape"]
        assert m["best_hot_shape"] in shapes and m["hot_gbps"] == max(shapes.values())
        assert 1000 < m["cold_gbps"] < 10000 and 1000 < m["hot_gbps"] < 10000, m
