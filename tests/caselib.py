"""Test helpers: build cases from the hand-worked fixtures and small explicit inputs."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_worked():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def worked_decompress_case():
    ex = load_worked()["decompress"]
    ps, npg, nl, li, K, D = (ex[k] for k in ("page_size", "num_pages", "num_layers", "layer_idx", "K", "D_c"))
    pool = np.full((npg, nl, 1, ps, 1, D), W.POISON_F32_BITS, dtype=np.uint32)
    for key, row in ex["layer_rows"].items():
        pg, sl = (int(v) for v in key.split(":"))
        pool[pg, li, 0, sl, 0, :] = f32_bits(row)
    cache = W.PagedCache(pool, "f32", np.array(ex["page_table"], np.uint32),
                         np.array(ex["cache_lengths"], np.uint32), used_pages=3)
    case = W.DecompressCase("worked", cache, li, np.array(ex["buffer_row_offsets"], np.uint32),
                            np.array(ex["cache_offsets"], np.uint32), K, len(ex["weight"]),
                            f32_bits(ex["weight"]).copy(), "f32")
    return case, np.array(ex["k_latent"], np.float32), np.array(ex["k_buffer"], np.float64)


def worked_kv_case():
    ex = load_worked()["kv_matmul"]
    ps, npg, nl, li, H, D = (ex[k] for k in ("page_size", "num_pages", "num_layers", "layer_idx",
                                             "num_kv_heads", "head_dim"))
    pool = np.full((npg, nl, 2, ps, H, D), W.POISON_BF16, dtype=np.uint16)
    cache = W.PagedCache(pool, "bf16", np.array(ex["page_table"], np.uint32),
                         np.array(ex["cache_lengths"], np.uint32), used_pages=3)
    case = W.KvMatmulCase("worked_kv", cache, li, W.to_bf16_bits(np.array(ex["hidden"], np.float32)),
                          np.array(ex["input_row_offsets"], np.uint32),
                          W.to_bf16_bits(np.array(ex["weight"], np.float32)))
    return case, ex["written"]


def explicit_decompress_case(pool_bits, dtype, page_table, cache_lengths, cache_offsets, rows,
                             layer_idx, K, weight_bits, weight_dtype):
    """A case from explicit arrays (pool shaped [pages, layers, 1, ps, 1, D])."""
    cache = W.PagedCache(pool_bits, dtype, np.asarray(page_table, np.uint32),
                         np.asarray(cache_lengths, np.uint32), used_pages=pool_bits.shape[0])
    bro = np.zeros(len(rows) + 1, np.uint32)
    bro[1:] = np.cumsum(rows)
    N = weight_bits.shape[0] if weight_bits is not None else 0
    return W.DecompressCase("explicit", cache, layer_idx, bro, np.asarray(cache_offsets, np.uint32),
                            K, N, weight_bits, weight_dtype)


def decode_tag(bits):
    """(page, layer, kv, slot, col) of elements of a tagged f32 pool."""
    b = np.asarray(bits).view(np.uint32).astype(np.int64)
    return b >> 20, (b >> 19) & 1, (b >> 18) & 1, (b >> 10) & 0xFF, b & 0x3FF


def bf16_bits_to_f32(bits):
    """bf16 bits -> float32 through a torch cast (a library routine, independent of the oracle)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def e4m3_bits_to_f64(codes):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.double().numpy()


def elem_f64(bits, dtype):
    """Library decoding of raw element bits to float64 (torch casts / numpy views)."""
    if dtype == "f32":
        return np.asarray(bits).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "e4m3":
        return e4m3_bits_to_f64(bits)
    raise ValueError(dtype)
