"""Host-side logic of bench.py, on the CPU: the single-GPU contract, the byte
models the rooflines use, the counter-summary lookup and the oracle
baselines (on the tiny workloads)."""
import glob
import os
import subprocess
import sys

import pytest

import bench
from workload import get_config, get_fff_config, make_fff_workload, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       env=dict(os.environ, **env), capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_fff_byte_model():
    cfg = get_fff_config("fff_D6_P64_d2048")
    bm = bench.fff_byte_model(cfg)
    # per token: 64 trees x 7 visited nodes x (input + output row of 2048 bf16), x in bf16, y in fp32
    per_token = 64 * 7 * 2 * 2048 * 2 + 2048 * 2 + 2048 * 4
    assert bm["per_token"] == per_token
    assert bm["step"] == 4096 * per_token == 15082717184
    assert bm["dense_per_token"] == 64 * 127 * 2 * 2048 * 2 + 2048 * 6
    assert round(bm["dense_per_token"] / bm["per_token"], 2) == 18.09


def test_counter_summaries_parse():
    files = glob.glob(os.path.join(ROOT, "profiles", "*__hbm_counters.txt"))
    assert files
    for path in files:
        kernel, workload = os.path.basename(path).split("__")[:2]
        assert kernel in bench.KERNEL_SOURCES, path
        vals = dict(line.split("=", 1) for line in open(path).read().splitlines()
                    if "=" in line and not line.startswith("#"))
        for key in ("hbm_bytes_per_launch", "fetch_scale", "write_scale", "source_digest", "trace_average_ns"):
            assert key in vals, (path, key)
        assert float(vals["hbm_bytes_per_launch"]) > 0
        # the lookup returns the bytes exactly when the kernel's sources still match
        t = bench.profiled_traffic(kernel, workload)
        if vals["source_digest"].strip() == bench.source_digest(kernel):
            assert t == float(vals["hbm_bytes_per_launch"])
        else:
            assert t is None
    assert bench.profiled_traffic("expert_down", "no_such_workload") is None


def test_oracle_baselines_on_tiny_workloads():
    cfg = get_config("tiny_f32_L4")
    layer, tok = make_workload(cfg)
    cb = bench.cpu_baseline(cfg, layer, tok.x, 0.5)
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert "16 of 16 chunks" in cb["sample"]
    fc = get_fff_config("fff_tiny_f32")
    fl, fx = make_fff_workload(fc)
    fb = bench.fff_cpu_baseline(fc, fl, fx, 0.5)
    assert fb["value"] > 0 and "48 of 48 tokens" in fb["sample"]
