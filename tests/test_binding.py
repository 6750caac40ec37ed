"""The Python binding refuses misuse with ValueError before it calls the
library: tensors on the host, outputs of the wrong dtype, buffers smaller (in
bytes) than what the call writes.  Runs without a GPU: every tensor here is a
host tensor, so a call whose arguments are otherwise right stops at the
residency check, and a call with a wrong dtype or size stops before it."""
import pytest
import torch

import mla_paged_latent_page_amd as mp


def cache(dtype=torch.bfloat16, pages=4, ps=16, D=576, num_kv=1, heads=1, batch=2, maxp=2, lengths=True,
          scales=False):
    pool = torch.zeros((pages, 2, num_kv, ps, heads, D // heads), dtype=dtype)
    pt = torch.zeros((batch, maxp), dtype=torch.int32)
    cl = torch.zeros(batch, dtype=torch.int32) if lengths else None
    sc = torch.zeros((pages, 2, num_kv, ps, -(-D // 128)), dtype=torch.float32) if scales else None
    return mp.PagedKVCache(pool, pt, cl, scales=sc)


M, N, K = 10, 256, 512
bro = torch.tensor([0, 4, 10], dtype=torch.int32)
co = torch.zeros(2, dtype=torch.int32)


def decompress(c=None, w=None, lat=None, out=None, dt=torch.bfloat16):
    c = c or cache(dt)
    w = torch.zeros((N, K), dtype=dt) if w is None else w
    lat = torch.zeros((M, 576), dtype=dt) if lat is None else lat
    out = torch.zeros((M, N), dtype=dt) if out is None else out
    mp.mla_decompress_k_paged(bro, co, M, w, c, 1, lat, out)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="current GPU"):
        decompress()
    with pytest.raises(ValueError, match="current GPU"):
        decompress(dt=torch.float32)


def test_output_dtype_must_match_the_cache():
    with pytest.raises(ValueError, match="k_buffer must be of dtype"):
        decompress(c=cache(torch.float32), w=torch.zeros((N, K)), lat=torch.zeros((M, 576)),
                   out=torch.zeros((M, N), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="k_buffer must be of dtype"):
        decompress(out=torch.zeros(M * N * 2, dtype=torch.uint8))      # enough bytes, wrong type
    with pytest.raises(ValueError, match="k_latent_buffer must be of dtype"):
        decompress(lat=torch.zeros((M, 576), dtype=torch.float16))
    with pytest.raises(ValueError, match="weight must be of dtype"):
        decompress(w=torch.zeros((N, K), dtype=torch.float32))


def test_buffers_are_measured_in_bytes():
    with pytest.raises(ValueError, match="k_buffer holds"):
        decompress(out=torch.zeros((M, N - 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="k_latent_buffer holds"):
        decompress(lat=torch.zeros((M - 1, 576), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="buffer_row_offsets must have"):
        mp.mla_decompress_k_paged(bro[:2], co, M, torch.zeros((N, K), dtype=torch.bfloat16), cache(), 1,
                                  torch.zeros((M, 576), dtype=torch.bfloat16),
                                  torch.zeros((M, N), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="32-bit integer"):
        mp.mla_decompress_k_paged(bro.float(), co, M, torch.zeros((N, K), dtype=torch.bfloat16), cache(), 1,
                                  torch.zeros((M, 576), dtype=torch.bfloat16),
                                  torch.zeros((M, N), dtype=torch.bfloat16))


def test_fp8_forms():
    c = cache()
    wq = torch.zeros((N, K), dtype=torch.uint8)
    ws = torch.ones((N // 128, K // 128))
    lat = torch.zeros((M, 576), dtype=torch.bfloat16)
    out = torch.zeros((M, N), dtype=torch.bfloat16)
    work = torch.zeros(M * K + 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="weight_e4m3 must be of dtype"):
        mp.mla_decompress_k_paged_fp8(bro, co, M, wq.float(), ws, c, 1, lat, out, work)
    with pytest.raises(ValueError, match="weight_scale holds"):
        mp.mla_decompress_k_paged_fp8(bro, co, M, wq, ws[:1, :1], c, 1, lat, out, work)
    with pytest.raises(ValueError, match="workspace is required"):
        mp.mla_decompress_k_paged_fp8(bro, co, M, wq, ws, c, 1, lat, out, None)
    with pytest.raises(ValueError, match="current GPU"):
        mp.mla_decompress_k_paged_fp8(bro, co, M, wq, ws, c, 1, lat, out, work)
    c8 = cache(torch.uint8, scales=True)
    lat8 = torch.zeros((M, 576), dtype=torch.uint8)
    lsc = torch.zeros((M, 5))
    with pytest.raises(ValueError, match="k_latent_scales holds"):
        mp.mla_decompress_k_paged_fp8_cache(bro, co, M, wq, ws, c8, 1, lat8, torch.zeros((M, 4)), out)
    with pytest.raises(ValueError, match="k_latent_buffer must be of dtype"):
        mp.mla_decompress_k_paged_fp8_cache(bro, co, M, wq, ws, c8, 1, lat, lsc, out)
    with pytest.raises(ValueError, match="current GPU"):
        mp.mla_decompress_k_paged_fp8_cache(bro, co, M, wq, ws, c8, 1, lat8, lsc, out)


def test_write_paths_and_absorption():
    ck = cache(num_kv=2, heads=2, D=256)
    T = 7
    iro = torch.tensor([0, 3, 7], dtype=torch.int32)
    with pytest.raises(ValueError, match="hidden_state must be of dtype"):
        mp.kv_matmul_paged(torch.zeros((T, 256)), iro, torch.zeros((256, 512), dtype=torch.bfloat16), ck, 1)
    with pytest.raises(ValueError, match="current GPU"):
        mp.kv_matmul_paged(torch.zeros((T, 256), dtype=torch.bfloat16), iro,
                           torch.zeros((256, 512), dtype=torch.bfloat16), ck, 1)
    cl = cache()
    x = torch.zeros((T, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kv_norm_gamma holds"):
        mp.mla_write_latent_paged(x, iro, torch.ones(100), 1e-6, torch.zeros((64, 64)), 512, cl, 1)
    with pytest.raises(ValueError, match="kv_norm_gamma must be of dtype"):
        mp.mla_write_latent_paged(x, iro, torch.ones(512, dtype=torch.float64), 1e-6, torch.zeros((64, 64)), 512, cl, 1)
    with pytest.raises(ValueError, match="current GPU"):
        mp.mla_write_latent_paged(x, iro, torch.ones(512), 1e-6, torch.zeros((64, 64)), 512, cl, 1)
    q = torch.zeros((4, 8, 192), dtype=torch.bfloat16)
    w = torch.zeros((8, 512, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q_latent must be of dtype"):
        mp.mla_absorb_q(q, w, torch.zeros((4, 8, 576)))
    with pytest.raises(ValueError, match="w_uk must be of dtype"):
        mp.mla_absorb_q(q, w.float(), torch.zeros((4, 8, 576), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="current GPU"):
        mp.mla_absorb_q(q, w, torch.zeros((4, 8, 576), dtype=torch.bfloat16))
