"""CPU oracle for the paged MLA latent-K path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
binding) never does, and this package never imports the product: the two
share nothing but the seeded inputs from ``workloads``.

The arithmetic lives in ``mla_oracle.c`` (plain scalar C, binary64 sums in k
order); this module builds it with gcc and marshals numpy arrays.  Every
function cites the page passage it follows in the C source.

Parity pins (tests/test_oracle_*.py, all ``-m "not gpu"``):
  * codecs: all 65536 bf16 and all 256 e4m3fn codes against torch's casts,
    e4m3 rounding (ties, subnormals, saturation) against torch and closed forms;
  * gather: tagged pools whose elements name their own page/slot/column, the
    identity page table equal to a contiguous slice, page_size 1 equal to an
    index_select, precondition errors;
  * products: numpy float64 matmul, identity and selection weights, NaN rope
    columns ignored, lossless fp8 blocks equal to the plain product, the
    e4m3 relative error bound, all-zero blocks;
  * write path: selection weight puts hidden columns into the named slots,
    destinations are distinct and inside the pages the page table lists.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
# tests that plant mistakes in a copy of the oracle point this at the mutant
_OVERRIDE = os.environ.get("MLA_ORACLE_LIB_OVERRIDE")
_lock = threading.Lock()
_lib = None

F32, BF16, E4M3 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "e4m3": E4M3}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_int = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _OVERRIDE:
            lib = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        lib.or_bf16_decode.argtypes = [_p, _p, _i64]
        lib.or_e4m3_decode.argtypes = [_p, _p, _i64]
        lib.or_e4m3_encode.argtypes = [_p, _p, _i64]
        lib.or_gather.argtypes = [_p, _int, _i64, _i64, _i64, _u32, _u32, _u32, _p, _u32, _u32,
                                  _p, _p, _p, _i64, _u32, _i64, _p]
        lib.or_gather.restype = _int
        lib.or_matmul_nt.argtypes = [_p, _int, _i64, _p, _int, _i64, _i64, _i64, _p, _i64, _p]
        lib.or_quantize_e4m3_rows.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _p]
        lib.or_quantize_f32_rows.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        lib.or_fp8_matmul_nt.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _i64, _p]
        lib.or_matmul_nn.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p]
        lib.or_kv_destinations.argtypes = [_i64, _i64, _i64, _i64, _u32, _u32, _u32, _p, _u32,
                                           _u32, _p, _p, _u32, _p]
        lib.or_kv_destinations.restype = _int
        lib.or_latent_rows.argtypes = [_p, _i64, _i64, _i64, _p, ctypes.c_double, _p, _i64, _p, _p]
        lib.or_latent_rows.restype = _int
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


class OracleError(RuntimeError):
    pass


# ---------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().or_bf16_decode(_ptr(bits), _ptr(out), bits.size)
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().or_e4m3_decode(_ptr(codes), _ptr(out), codes.size)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().or_e4m3_encode(_ptr(x), _ptr(out), x.size)
    return out


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------
def gather(case, *, check_lengths: bool = True) -> np.ndarray:
    """k_latent_buffer [M, D_c] (raw bits, the pool's element type)."""
    c = case.cache
    sp, sl, skv, st = c.strides()
    M, D = case.M, case.D_c
    out = np.empty((M, D), dtype=c.pool.dtype)
    pt = np.ascontiguousarray(c.page_table, np.uint32)
    cl = np.ascontiguousarray(c.cache_lengths, np.uint32)
    bro = np.ascontiguousarray(case.buffer_row_offsets, np.uint32)
    co = np.ascontiguousarray(case.cache_offsets, np.uint32)
    rc = _load().or_gather(_ptr(c.pool), c.elem_bytes, sp, sl, st, c.num_pages, c.num_layers,
                           c.page_size, _ptr(pt), c.max_pages_per_seq, case.batch,
                           _ptr(cl) if check_lengths else None, _ptr(bro), _ptr(co), M,
                           case.layer_idx, D, _ptr(out) if out.size else None)
    if rc != 0:
        raise OracleError(f"gather precondition failed ({rc})")
    return out


def gather_scales(case, *, check_lengths: bool = True) -> np.ndarray:
    """The scales that go with the gathered rows of an e4m3 cache, float32
    [M, blocks per row]: the same copy as ``gather`` (same requests, positions,
    pages and slots) applied to the cache's scale pool, whose token rows hold one
    fp32 scale per ``scale_gran`` columns (page "generic_flare_mla_decompress_k_cache_ragged_paged",
    the collection's ``scale_dtype_`` and ``quantization_granularity_``)."""
    c = case.cache
    if c.scales is None:
        raise OracleError("the cache has no scales")
    sp, sl, skv, st = c.scale_strides()
    M, nb = case.M, c.scale_blocks
    out = np.empty((M, nb), dtype=np.float32)
    pt = np.ascontiguousarray(c.page_table, np.uint32)
    cl = np.ascontiguousarray(c.cache_lengths, np.uint32)
    bro = np.ascontiguousarray(case.buffer_row_offsets, np.uint32)
    co = np.ascontiguousarray(case.cache_offsets, np.uint32)
    sc = np.ascontiguousarray(c.scales)
    rc = _load().or_gather(_ptr(sc), 4, sp, sl, st, c.num_pages, c.num_layers,
                           c.page_size, _ptr(pt), c.max_pages_per_seq, case.batch,
                           _ptr(cl) if check_lengths else None, _ptr(bro), _ptr(co), M,
                           case.layer_idx, nb, _ptr(out) if out.size else None)
    if rc != 0:
        raise OracleError(f"scale gather precondition failed ({rc})")
    return out


# ---------------------------------------------------------------------------
# products
# ---------------------------------------------------------------------------
def _rows_arg(rows, M):
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    return rows


def matmul_nt(A_bits, a_dtype, W_bits, w_dtype, K, rows=None) -> np.ndarray:
    """out[j, n] = sum_{k<K} A[rows[j], k] * W[n, k] in binary64."""
    A_bits = np.ascontiguousarray(A_bits)
    W_bits = np.ascontiguousarray(W_bits)
    rows = _rows_arg(rows, A_bits.shape[0])
    N = W_bits.shape[0]
    out = np.empty((len(rows), N), np.float64)
    if len(rows) and N:
        _load().or_matmul_nt(_ptr(A_bits), _DT[a_dtype], A_bits.shape[1], _ptr(W_bits),
                             _DT[w_dtype], W_bits.shape[1], N, K, _ptr(rows), len(rows), _ptr(out))
    return out


def quantize_e4m3_rows(A_bf16_bits, K, k_gran=128):
    """(codes uint8 [M, K], scales float32 [M, ceil(K/k_gran)]) of the first K columns."""
    A = np.ascontiguousarray(A_bf16_bits, dtype=np.uint16)
    M = A.shape[0]
    nkb = -(-K // k_gran)
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, nkb), np.float32)
    if M:
        _load().or_quantize_e4m3_rows(_ptr(A), A.shape[1], M, K, k_gran, _ptr(q), _ptr(s))
    return q, s


def quantize_f32_rows(Y, gran=128):
    """(codes uint8 [T, D], scales float32 [T, ceil(D/gran)]) of binary32 rows
    (blocks of gran columns, the last one possibly shorter)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    T, D = Y.shape
    nb = -(-D // gran)
    q = np.empty((T, D), np.uint8)
    s = np.empty((T, nb), np.float32)
    if T:
        _load().or_quantize_f32_rows(_ptr(Y), T, D, gran, _ptr(q), _ptr(s))
    return q, s


def fp8_matmul_nt(q_a, s_a, q_w, s_w, n_gran=128, k_gran=128, rows=None) -> np.ndarray:
    q_a = np.ascontiguousarray(q_a, np.uint8)
    s_a = np.ascontiguousarray(s_a, np.float32)
    q_w = np.ascontiguousarray(q_w, np.uint8)
    s_w = np.ascontiguousarray(s_w, np.float32)
    M, K = q_a.shape
    N = q_w.shape[0]
    assert q_w.shape[1] == K and s_w.shape == (-(-N // n_gran), -(-K // k_gran))
    rows = _rows_arg(rows, M)
    out = np.empty((len(rows), N), np.float64)
    if len(rows) and N:
        _load().or_fp8_matmul_nt(_ptr(q_a), _ptr(s_a), _ptr(q_w), _ptr(s_w), N, K, n_gran, k_gran,
                                 _ptr(rows), len(rows), _ptr(out))
    return out


def matmul_nn(H_bits, W_bits, rows=None) -> np.ndarray:
    """out[j, n] = sum_k H[rows[j], k] * W[k, n] in binary64 (bf16 operands)."""
    H = np.ascontiguousarray(H_bits, np.uint16)
    W = np.ascontiguousarray(W_bits, np.uint16)
    rows = _rows_arg(rows, H.shape[0])
    K, N = W.shape
    assert H.shape[1] == K
    out = np.empty((len(rows), N), np.float64)
    if len(rows) and N:
        _load().or_matmul_nn(_ptr(H), K, _ptr(W), N, N, K, _ptr(rows), len(rows), _ptr(out))
    return out


# ---------------------------------------------------------------------------
# whole operations, composed from the steps above in the pages' order
# ---------------------------------------------------------------------------
def decompress_k(case, rows=None):
    """(k_latent bits [M, D_c], k_buffer rows as binary64 [len(rows), N]).

    Gather, then multiply the first K columns of each gathered row by W_k^T."""
    lat = gather(case)
    if case.weight_dtype == "e4m3":
        raise OracleError("use decompress_k_fp8 for an e4m3 weight")
    out = matmul_nt(lat, case.cache.dtype, case.weight, case.weight_dtype, case.K, rows)
    return lat, out


def decompress_k_fp8(case, rows=None):
    """(k_latent bits, activation codes, activation scales, k_buffer rows binary64)."""
    lat = gather(case)
    q, s = quantize_e4m3_rows(lat, case.K, case.k_gran)
    out = fp8_matmul_nt(q, s, case.weight_q, case.weight_scale, case.n_gran, case.k_gran, rows)
    return lat, q, s, out


def decompress_k_fp8_cache(case, rows=None):
    """(k_latent codes uint8 [M, D_c], their scales float32 [M, blocks per row],
    k_buffer rows binary64) for an e4m3 cache and an e4m3 W_k.

    The gathered codes and scales are bit copies of the cache's; the product is
    the block-scaled one of the fp8 form (page "mla_prefill_decode_graph_fp8",
    Parameters m/n/k_scale_granularity, Args w_k, w_k_scale) on the first K
    columns, with the cache's own per-128-column scales as the activation scales:
    no quantisation step, the cache is already quantised."""
    c = case.cache
    if c.dtype != "e4m3" or c.scale_gran != case.k_gran:
        raise OracleError("an e4m3 cache with one scale per k_gran columns is required")
    codes = gather(case)
    scales = gather_scales(case)
    kb = -(-case.K // case.k_gran)
    out = fp8_matmul_nt(codes[:, :case.K], scales[:, :kb], case.weight_q, case.weight_scale,
                        case.n_gran, case.k_gran, rows)
    return codes, scales, out


def decompress_kv_fp8_cache(case_k, case_v, rows=None):
    """(codes, scales, k_buffer rows, v_buffer rows): decompress_k_fp8_cache for
    W_k and for W_uv on the same gathered codes and scales (case_v is case_k
    with the weight replaced by W_uv).  Pinned by: K and V each equal the
    single-projection form on that projection's own weight, and a selection
    W_uv (code 1.0, unit scales) returns the named latent columns dequantised
    with their own block's scale, exactly."""
    assert case_v.cache is case_k.cache and case_v.K == case_k.K
    codes, scales, k = decompress_k_fp8_cache(case_k, rows)
    kb = -(-case_v.K // case_v.k_gran)
    v = fp8_matmul_nt(codes[:, :case_v.K], scales[:, :kb], case_v.weight_q, case_v.weight_scale,
                      case_v.n_gran, case_v.k_gran, rows)
    return codes, scales, k, v


def absorb_q(case):
    """(latent part binary64 [T, H, kv_latent_dim], rope part bits [T, H, d_rope]
    or None): query absorption (page "mla_prefill_decode_graph_fp8", Args q
    [tot_seq_len, num_heads, qk_nope_head_dim + qk_rope_head_dim] and w_uk
    [num_heads, kv_latent_dim, qk_nope_head_dim], which takes the non-rope part
    of each query head into the latent space):
        latent[t, h, c] = sum_{d < d_nope} q[t, h, d] * w_uk[h, c, d]
    one product per head, and the rope part q[t, h, d_nope:] carried over
    unchanged after it when case.copy_rope."""
    T, H, _ = case.q.shape
    DN, NL = case.d_nope, case.kv_latent_dim
    out = np.empty((T, H, NL), np.float64)
    for h in range(H):
        a = np.ascontiguousarray(case.q[:, h, :DN])
        out[:, h, :] = matmul_nt(a, "bf16", np.ascontiguousarray(case.w_uk[h]), "bf16", DN)
    rope = np.ascontiguousarray(case.q[:, :, DN:]) if case.copy_rope else None
    return out, rope


def absorb_q_fp8(case):
    """(latent part binary64 [T, H, kv_latent_dim], rope bits or None, query codes
    uint8 [T, H, d_nope], query scales float32 [T, H]): the fp8 form of query
    absorption (page "mla_prefill_decode_graph_fp8": w_uk in fp8_dtype with
    w_uk_scale, granularities m 1, n 128, k 128).  Each head's non-rope query
    part is quantised per 1 x 128 block like the decompress activations, then
    multiplied block by block with the e4m3 w_uk of that head and both scales."""
    T, H, _ = case.q.shape
    DN, NL = case.d_nope, case.kv_latent_dim
    out = np.empty((T, H, NL), np.float64)
    codes = np.empty((T, H, DN), np.uint8)
    scales = np.empty((T, H), np.float32)
    for h in range(H):
        qa, sa = quantize_e4m3_rows(np.ascontiguousarray(case.q[:, h, :DN]), DN, 128)
        codes[:, h], scales[:, h] = qa, sa[:, 0]
        out[:, h, :] = fp8_matmul_nt(qa, sa, np.ascontiguousarray(case.w_q[h]),
                                     np.ascontiguousarray(case.w_scale[h]), 128, 128)
    rope = np.ascontiguousarray(case.q[:, :, DN:]) if case.copy_rope else None
    return out, rope, codes, scales


def decompress_kv(case_k, case_v, rows=None):
    """(k_latent bits, k_buffer rows, v_buffer rows), binary64 products.

    The fused K and V form (page "mla_prefill_decode_graph_fp8", Args w_k and
    w_uv: w_uv projects the latent values to V): one gather, then the first K
    columns of each gathered row times W_k^T and times W_uv^T.  ``case_v`` is
    ``case_k`` with the weight replaced by W_uv (same cache, offsets and K)."""
    assert case_v.cache is case_k.cache and case_v.K == case_k.K
    lat = gather(case_k)
    if case_k.weight_dtype == "e4m3":
        q, s = quantize_e4m3_rows(lat, case_k.K, case_k.k_gran)
        k = fp8_matmul_nt(q, s, case_k.weight_q, case_k.weight_scale, case_k.n_gran, case_k.k_gran, rows)
        v = fp8_matmul_nt(q, s, case_v.weight_q, case_v.weight_scale, case_v.n_gran, case_v.k_gran, rows)
    else:
        k = matmul_nt(lat, case_k.cache.dtype, case_k.weight, case_k.weight_dtype, case_k.K, rows)
        v = matmul_nt(lat, case_v.cache.dtype, case_v.weight, case_v.weight_dtype, case_v.K, rows)
    return lat, k, v


def kv_destinations(case) -> np.ndarray:
    """int64 [T, 2]: element offsets into the pool of each token's K and V rows."""
    c = case.cache
    sp, sl, skv, st = c.strides()
    T = case.T
    dst = np.empty((T, 2), np.int64)
    pt = np.ascontiguousarray(c.page_table, np.uint32)
    cl = np.ascontiguousarray(c.cache_lengths, np.uint32)
    iro = np.ascontiguousarray(case.input_row_offsets, np.uint32)
    rc = _load().or_kv_destinations(sp, sl, skv, st, c.num_pages, c.num_layers, c.page_size,
                                    _ptr(pt), c.max_pages_per_seq, len(iro) - 1, _ptr(cl),
                                    _ptr(iro), case.layer_idx, _ptr(dst) if T else None)
    if rc != 0:
        raise OracleError(f"kv destination precondition failed ({rc})")
    return dst


def latent_write(case):
    """(row values binary64 [T, D_c], element offsets int64 [T] of each token's
    cache row): the latent write path (page "mla_prefill_decode_graph_fp8", Args
    kv_input_fn, kv_norm_gamma, epsilon, freqs_cis, input_row_offsets): the
    RMS-normalised latent part and the rotated rope part of each new token, and
    where its row goes (the token placement of the write path, kv half 0)."""
    T, D = case.x.shape
    K, R = case.K, D - case.K
    iro = np.asarray(case.input_row_offsets, np.int64)
    cl = np.asarray(case.cache.cache_lengths, np.int64)
    pos = np.empty(T, np.int64)
    for b in range(len(iro) - 1):
        pos[iro[b]:iro[b + 1]] = cl[b] + np.arange(iro[b + 1] - iro[b])
    x = np.ascontiguousarray(case.x, np.uint16)
    gamma = np.ascontiguousarray(case.gamma, np.float32)
    freqs = np.ascontiguousarray(case.freqs, np.float32)
    out = np.empty((T, D), np.float64)
    if T:
        rc = _load().or_latent_rows(_ptr(x), T, K, R, _ptr(gamma), float(case.eps), _ptr(freqs),
                                    freqs.shape[0], _ptr(pos), _ptr(out))
        if rc != 0:
            raise OracleError(f"latent write precondition failed ({rc})")
    return out, kv_destinations(case)[:, 0]


def latent_write_fp8(case):
    """(codes uint8 [T, D_c], scales float32 [T, nblk], row values binary64
    [T, D_c], element offsets int64 [T] of each token's cache row, float offsets
    int64 [T] of its scales) for an e4m3 cache: the latent write path's values
    (latent_write), rounded to binary32 (the precision the quantisation
    decisions are taken in) and quantised per scale block of the cache
    (quantize_f32_rows)."""
    c = case.cache
    if c.dtype != "e4m3" or c.scales is None:
        raise OracleError("an e4m3 cache with scales is required")
    ref, dst = latent_write(case)
    q, s = quantize_f32_rows(ref.astype(np.float32), c.scale_gran)
    sp, sl, skv, st = c.scale_strides()
    pos_page = dst // c.strides()[0]
    slot = (dst - pos_page * c.strides()[0] - case.layer_idx * c.strides()[1]) // c.strides()[3]
    sdst = pos_page * sp + case.layer_idx * sl + slot * st
    return q, s, ref, dst, sdst


def kv_matmul(case, rows=None):
    """(out rows binary64 [len(rows), N], destinations int64 [T, 2])."""
    out = matmul_nn(case.hidden, case.weight, rows)
    return out, kv_destinations(case)
