"""The oracle's C code under host sanitizers: a copy of oracle/mla_oracle.c built
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only) runs
every oracle entry point on small cases in a child process.  An out-of-bounds
access, a use after free or an undefined operation (signed overflow, a bad
shift, a misaligned access) aborts the child, and the test shows its report."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

# Small cases of every oracle function, paged gathers with ragged requests and
# odd page sizes included (the same builders the pin tests use).
SCRIPT = r'''
import sys
sys.path.insert(0, %r)
import numpy as np
import oracle
import workloads as W

c = W.small_decompress(1, batch=3, max_len=70, page_size=7, N=96)
oracle.gather(c)
oracle.decompress_k(c)
oracle.decompress_k(W.small_decompress(2, batch=2, max_len=40, page_size=5, N=64, dtype="f32"))
f8 = W.small_decompress(3, batch=3, max_len=60, page_size=16, N=256, fp8=True)
oracle.decompress_k_fp8(f8)
e = W.small_decompress(4, batch=3, max_len=50, page_size=16, N=256, dtype="e4m3", fp8=True)
oracle.gather_scales(e)
oracle.decompress_k_fp8_cache(e)
oracle.decompress_kv_fp8_cache(e, W.with_second_projection(e, seed=104, N=128))
oracle.decompress_kv(c, W.with_second_projection(c, seed=101, N=64))
kv = W.small_kv_matmul(5, batch=3, max_len=30, hidden_dim=128, num_kv_heads=1, head_dim=128, page_size=8)
oracle.kv_matmul(kv)
oracle.kv_destinations(kv)
lw = W.latent_write_case("asan", seed=6, seq_lens=[3, 0, 5], start_lengths=[2, 7, 0], page_size=4, K=256, R=64)
oracle.latent_write(lw)
lw8 = W.latent_write_case("asan8", seed=7, seq_lens=[2, 4], start_lengths=[1, 3], page_size=4, K=256, R=64,
                          dtype="e4m3")
oracle.latent_write_fp8(lw8)
oracle.absorb_q(W.absorb_case("asan", seed=8, T=9, H=3, d_nope=32, d_rope=16, kv_latent_dim=64))
oracle.absorb_q_fp8(W.absorb_case("asan8", seed=9, T=5, H=2, d_nope=128, d_rope=64, kv_latent_dim=128, fp8=True))
x = (np.random.default_rng(10).standard_normal((7, 300)) * 3).astype(np.float32)
oracle.quantize_f32_rows(x)
oracle.quantize_e4m3_rows(W.to_bf16_bits(x), 256)
oracle.e4m3_decode(oracle.e4m3_encode(x.ravel()))
print("sanitized oracle run complete")
''' % ROOT


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("this gcc has no AddressSanitizer runtime")
    lib = tmp_path / "liboracle_sanitized.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(lib), SRC, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", MLA_ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and "sanitized oracle run complete" in r.stdout, r.stderr[-6000:]
