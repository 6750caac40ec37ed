"""MLA_PAGED_LOG: with it set, every kernel launch prints one line to stderr
naming the kernel, its grid and its shapes; without it, nothing.  Run in child
processes, since the setting is read once per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SCRIPT = r'''
import sys
sys.path.insert(0, %r)
sys.path.insert(0, %r)
import torch
import workloads as W
from gpu_util import run_decompress
torch.cuda.set_device(0)
# 65 rows: the few-rows kernel; 730 rows: the gather, then the product
run_decompress(W.decompress_case("log_few", seed=31, cache_lengths=[40, 30], cache_offsets=[0, 5], page_size=16,
                                 kv_lora_rank=512, rope_dim=64, N=256))
run_decompress(W.decompress_case("log_many", seed=32, cache_lengths=[300, 280, 150], cache_offsets=[0, 0, 0],
                                 page_size=16, kv_lora_rank=512, rope_dim=64, N=512))
torch.cuda.synchronize()
print("done", flush=True)
''' % (ROOT, HERE)


def _run(log):
    env = dict(os.environ)
    env.pop("MLA_PAGED_LOG", None)
    if log is not None:
        env["MLA_PAGED_LOG"] = log
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-3000:]
    return [l for l in r.stderr.splitlines() if l.startswith("mla_paged: ")]


def test_launch_log_names_each_kernel():
    lines = _run("1")
    assert any(l.startswith("mla_paged: decompress_small_bf16<gather> grid ") for l in lines), lines
    assert any(l.startswith("mla_paged: gather_rows_kernel grid ") for l in lines), lines
    assert any("gemm_bf16" in l and " M=" in l and " K=512" in l for l in lines), lines


def test_no_log_unless_asked():
    assert _run(None) == []
    assert _run("0") == []
