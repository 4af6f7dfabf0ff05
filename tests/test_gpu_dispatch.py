"""Host dispatch cost of the C ABI and graph replay, measured by the
qlin_dispatch_bench program built with the library (MI355X)."""
import json
import os
import subprocess

import pytest

import int8_gemm_linear_amd as q

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(q.LIB_PATH), "qlin_dispatch_bench")


@pytest.mark.parametrize("shape", [("1", "2048", "2048"), ("32", "2048", "6144")])
def test_dispatch_bench_runs_and_graph_amortizes(shape):
    print("[gpu-dispatch]", shape, flush=True)
    r = subprocess.run([EXE, *shape], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("select_us", "reject_us", "launch_us", "empty_launch_us", "graph_launch_us",
              "graph_gpu_us_per_call"):
        assert d[k] > 0, k
    # the library adds little over HIP's own launch, and the whole graph of
    # calls costs the host less than launching the calls one by one
    assert d["select_us"] < 5 and d["reject_us"] < 5
    assert d["graph_launch_us"] < d["launch_us"] * d["graph_calls"]
