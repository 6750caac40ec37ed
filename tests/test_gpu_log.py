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


FP8_SCRIPT = r'''
import sys
sys.path.insert(0, %r)
sys.path.insert(0, %r)
import torch
import workloads as W
from gpu_util import run_decompress, run_decompress_fp8_cache
torch.cuda.set_device(0)
for form, dtype, run in (("quant", "bf16", run_decompress), ("cache", "e4m3", run_decompress_fp8_cache)):
    for n in (64, 65, 193):
        sys.stderr.write("mla_paged: case %%s %%d\n" %% (form, n))
        sys.stderr.flush()
        run(W.decompress_case("log_fp8", seed=33, cache_lengths=[n], cache_offsets=[0], page_size=16,
                              kv_lora_rank=512, rope_dim=64, N=256, dtype=dtype, fp8=True))
        torch.cuda.synchronize()
print("done", flush=True)
''' % (ROOT, HERE)


def test_fp8_calls_take_the_form_their_row_count_selects():
    """The fp8 calls by row count: at most 64 rows one launch (gather,
    quantisation or code copy, and product); 65 to 192 rows the gather pass, then
    the few-rows product; more, the gather pass, then the large product."""
    env = dict(os.environ, MLA_PAGED_LOG="1")
    r = subprocess.run([sys.executable, "-c", FP8_SCRIPT], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-3000:]
    kernels, case = {}, None
    for l in r.stderr.splitlines():
        if l.startswith("mla_paged: case "):
            case = tuple(l.split()[2:4])
            kernels[case] = []
        elif l.startswith("mla_paged: ") and case is not None:
            kernels[case].append(l.split()[1])
    assert kernels[("quant", "64")] == ["decompress_small_fp8_gq"], kernels
    assert kernels[("quant", "65")] == ["gather_quant_fp8_kernel", "decompress_small_fp8"], kernels
    assert kernels[("quant", "193")] == ["gather_quant_fp8_kernel", "gemm_fp8_ring"], kernels
    assert kernels[("cache", "64")] == ["decompress_small_fp8_gc"], kernels
    assert kernels[("cache", "65")] == ["gather_rows_kernel", "decompress_small_fp8"], kernels
    assert kernels[("cache", "193")] == ["gather_rows_kernel", "gemm_fp8_ring"], kernels
