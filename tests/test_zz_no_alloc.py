"""GPU parity of mla_decompress_k_paged_fp8_noalloc (the fp8 call that keeps its
activation codes and scales in the library's fixed device array instead of a
caller workspace) against mla_decompress_k_paged_fp8 with a workspace: the
same kernels on the same inputs, so the gathered rows and k_buffer must be
identical bit for bit.  Two calls in a row, the first at the array's full size
(the 64K-row fp8 prefill batch), the second smaller, so the second runs over
what the first left in the array; the small call is also checked against the
oracle."""
import numpy as np
import pytest
import torch

import mla_paged_latent_page_amd as mp
import oracle
import workloads as W
from gpu_util import FP8_TOL, POISON_OUT, check_close, run_decompress, say, to_bits

pytestmark = pytest.mark.gpu


def _noalloc(case, extra_rows=3):
    dc, t = W.device_decompress(case)
    M, D, N = case.M, case.D_c, case.N
    lat = torch.empty((M + extra_rows, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M + extra_rows, N), dtype=torch.bfloat16, device="cuda")
    lat.view(torch.int16).fill_(POISON_OUT)
    out.view(torch.int16).fill_(POISON_OUT)
    say(f"[gpu] {case.name} noalloc: M={M} N={N} K={case.K}")
    mp.mla_decompress_k_paged_fp8_noalloc(t["buffer_row_offsets"], t["cache_offsets"], M, t["weight_q"],
                                          t["weight_scale"], mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths),
                                          case.layer_idx, lat, out)
    torch.cuda.synchronize()
    return lat, out


def _same_as_workspace_call(case):
    lat, out = _noalloc(case)
    ref = run_decompress(case, extra_rows=3)
    assert torch.equal(lat.view(torch.int16), ref["lat"].view(torch.int16)), "gathered rows differ"
    assert torch.equal(out.view(torch.int16), ref["out"].view(torch.int16)), "k_buffer differs"
    return out


def test_noalloc_matches_the_workspace_call_twice():
    big = W.c3_fp8()
    assert mp.mla_decompress_k_paged_fp8_workspace_size(big.M, big.K) == mp.MLA_FP8_NOALLOC_SCRATCH_BYTES
    _same_as_workspace_call(big)
    small = W.small_decompress(41, batch=5, max_len=300, page_size=16, N=512, fp8=True)
    out = _same_as_workspace_call(small)
    M = small.M
    lat, q, s, ref = oracle.decompress_k_fp8(small)
    check_close(out[:M].double().cpu().numpy(), ref, FP8_TOL, "noalloc k_buffer (small, second call)")
    assert np.all(to_bits(out)[M:] == POISON_OUT)


def test_noalloc_refuses_a_call_larger_than_its_array():
    case = W.small_decompress(42, batch=2, max_len=40, page_size=16, N=128, fp8=True)
    dc, t = W.device_decompress(case)
    rows = 65537
    lat = torch.empty((rows, case.D_c), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((rows, case.N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mp.MlaError, match="MLA_ERR_WORKSPACE"):
        mp.mla_decompress_k_paged_fp8_noalloc(t["buffer_row_offsets"], t["cache_offsets"], rows, t["weight_q"],
                                              t["weight_scale"],
                                              mp.PagedKVCache(dc.pool, dc.page_table, dc.cache_lengths),
                                              case.layer_idx, lat, out)
