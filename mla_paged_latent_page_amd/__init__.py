"""Python binding of the gfx950 paged MLA latent-K library (``include/mla_paged.h``).

Argument marshalling only: every step of every operation runs in the HIP
kernels of ``_build/libmla_paged.so``.  Tensors are torch tensors on the
current HIP device; the current torch stream is passed as the HIP stream.
There is no fallback: if the library has not been built, every call raises.

Entry points (same names as the C ABI):
  mla_decompress_k_paged       gather latent rows from a paged cache, up-project them
  mla_decompress_k_paged_fp8   the fp8 block-scaled form (1x128 activation, 128x128 weight scales)
  mla_decompress_kv_paged(_fp8)  one gather, K and V up-projections
  mla_decompress_k_paged_fp8_cache  the fp8 form on an e4m3 cache with per-128-column scales
  mla_write_latent_paged       RMSNorm + rope rotation of new tokens' rows into the cache pages
  mla_absorb_q(_fp8)           per-head product of the non-rope query columns with w_uk (decode)
  kv_matmul_paged              project hidden states and write them into K/V cache pages
  mla_gather_latent_paged      the gather step alone
  mla_latent_matmul            the up-projection step alone (rows already gathered)
  mla_check_indices            debug validation of index arrays (synchronous)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmla_paged.so")

MLA_DTYPE_F32, MLA_DTYPE_BF16, MLA_DTYPE_F8E4M3FN = 0, 1, 2
STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL_POINTER", 2: "MLA_ERR_INVALID_SHAPE",
          3: "MLA_ERR_INVALID_DTYPE", 4: "MLA_ERR_MISALIGNED", 5: "MLA_ERR_OUT_OF_RANGE",
          6: "MLA_ERR_WORKSPACE", 7: "MLA_ERR_UNSUPPORTED_DEVICE", 8: "MLA_ERR_HIP"}
EXPORTS = ("mla_paged_cache_default_strides", "mla_decompress_k_paged", "mla_gather_latent_paged",
           "mla_latent_matmul", "mla_decompress_k_paged_fp8_workspace_size", "mla_decompress_k_paged_fp8",
           "kv_matmul_paged", "mla_check_indices", "mla_status_string", "mla_last_hip_error",
           "mla_abi_version", "mla_decompress_kv_paged", "mla_decompress_kv_paged_fp8",
           "mla_write_latent_paged", "mla_decompress_k_paged_fp8_cache", "mla_absorb_q", "mla_absorb_q_fp8",
           "mla_write_latent_paged_fp8", "mla_decompress_kv_paged_fp8_cache")


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class CacheDesc(ctypes.Structure):
    """Mirror of ``mla_paged_cache_t``."""
    _fields_ = [
        ("blocks", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("num_layers", ctypes.c_uint32), ("num_pages", ctypes.c_uint32),
        ("page_size", ctypes.c_uint32), ("num_kv", ctypes.c_uint32),
        ("num_heads", ctypes.c_uint32), ("head_dim", ctypes.c_uint32),
        ("stride_page", ctypes.c_int64), ("stride_layer", ctypes.c_int64),
        ("stride_kv", ctypes.c_int64), ("stride_token", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("batch_size", ctypes.c_uint32),
        ("max_pages_per_seq", ctypes.c_uint32), ("cache_lengths", ctypes.c_void_p),
    ]


class ScalesDesc(ctypes.Structure):
    """Mirror of ``mla_cache_scales_t``."""
    _fields_ = [
        ("scales", ctypes.c_void_p), ("granularity", ctypes.c_uint32),
        ("stride_page", ctypes.c_int64), ("stride_layer", ctypes.c_int64),
        ("stride_kv", ctypes.c_int64), ("stride_token", ctypes.c_int64),
    ]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"HIP library not built ({LIB_PATH}); run __graft_entry__.build() "
                                   "or python -m mla_paged_latent_page_amd.build")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
            L.mla_paged_cache_default_strides.argtypes = [ctypes.POINTER(CacheDesc)]
            L.mla_paged_cache_default_strides.restype = i32
            L.mla_decompress_k_paged.argtypes = [vp, vp, i32, vp, i32, i32, ctypes.POINTER(CacheDesc), u32,
                                                 vp, vp, vp]
            L.mla_decompress_k_paged.restype = i32
            L.mla_decompress_k_paged_fp8_workspace_size.argtypes = [i32, i32, i32]
            L.mla_decompress_k_paged_fp8_workspace_size.restype = sz
            L.mla_decompress_k_paged_fp8.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(CacheDesc), u32, vp, vp, vp, sz, vp]
            L.mla_decompress_k_paged_fp8.restype = i32
            L.mla_decompress_kv_paged.argtypes = [vp, vp, i32, vp, i32, vp, i32, i32, ctypes.POINTER(CacheDesc),
                                                  u32, vp, vp, vp, vp]
            L.mla_decompress_kv_paged.restype = i32
            L.mla_decompress_kv_paged_fp8.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                      ctypes.POINTER(CacheDesc), u32, vp, vp, vp, vp, sz, vp]
            L.mla_decompress_kv_paged_fp8.restype = i32
            L.mla_write_latent_paged.argtypes = [vp, vp, i32, vp, ctypes.c_float, vp, i32, i32,
                                                 ctypes.POINTER(CacheDesc), u32, vp]
            L.mla_write_latent_paged.restype = i32
            L.mla_write_latent_paged_fp8.argtypes = [vp, vp, i32, vp, ctypes.c_float, vp, i32, i32,
                                                     ctypes.POINTER(CacheDesc), ctypes.POINTER(ScalesDesc), u32, vp]
            L.mla_write_latent_paged_fp8.restype = i32
            L.mla_decompress_k_paged_fp8_cache.argtypes = [vp, vp, i32, vp, vp, i32, i32, ctypes.POINTER(CacheDesc),
                                                           ctypes.POINTER(ScalesDesc), u32, vp, vp, vp, vp]
            L.mla_decompress_k_paged_fp8_cache.restype = i32
            L.mla_decompress_kv_paged_fp8_cache.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32,
                                                            ctypes.POINTER(CacheDesc), ctypes.POINTER(ScalesDesc), u32,
                                                            vp, vp, vp, vp, vp]
            L.mla_decompress_kv_paged_fp8_cache.restype = i32
            L.mla_absorb_q.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, vp, vp]
            L.mla_absorb_q.restype = i32
            L.mla_absorb_q_fp8.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp]
            L.mla_absorb_q_fp8.restype = i32
            L.kv_matmul_paged.argtypes = [vp, vp, i32, i32, vp, ctypes.POINTER(CacheDesc), u32, vp]
            L.kv_matmul_paged.restype = i32
            L.mla_gather_latent_paged.argtypes = [vp, vp, i32, ctypes.POINTER(CacheDesc), u32, vp, vp]
            L.mla_gather_latent_paged.restype = i32
            L.mla_latent_matmul.argtypes = [vp, ctypes.c_int64, i32, vp, i32, i32, i32, vp, vp]
            L.mla_latent_matmul.restype = i32
            L.mla_check_indices.argtypes = [vp, vp, i32, ctypes.POINTER(CacheDesc),
                                            ctypes.POINTER(ctypes.c_int64), vp]
            L.mla_check_indices.restype = i32
            L.mla_status_string.argtypes = [i32]
            L.mla_status_string.restype = ctypes.c_char_p
            L.mla_last_hip_error.restype = i32
            L.mla_abi_version.restype = i32
            _lib = L
        return _lib


# ---------------------------------------------------------------------------
# cache descriptor from torch tensors
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PagedKVCache:
    """A paged pool as torch tensors.

    pool          [num_pages, num_layers, num_kv, page_size, num_heads, head_dim]
                  (float32, bfloat16, or uint8 / float8_e4m3fn codes; may be a strided
                  view with contiguous token rows)
    page_table    int32/uint32 [batch, max_pages_per_seq] page ids (raw 32-bit values)
    cache_lengths int32/uint32 [batch] or None
    scales        fp8 pools only: float32 [num_pages, num_layers, num_kv, page_size, nblk],
                  one scale per scale_granularity columns of a token row
    """
    pool: "object"
    page_table: "object"
    cache_lengths: Optional["object"] = None
    scales: Optional["object"] = None
    scale_granularity: int = 128

    def descriptor(self) -> CacheDesc:
        import torch
        p = self.pool
        if p.dim() != 6:
            raise ValueError("pool must be [pages, layers, kv, page_size, heads, head_dim]")
        if p.stride(5) != 1 or p.stride(4) != p.shape[5]:
            raise ValueError("token rows of the pool must be contiguous")
        dt = {torch.float32: MLA_DTYPE_F32, torch.bfloat16: MLA_DTYPE_BF16, torch.uint8: MLA_DTYPE_F8E4M3FN,
              torch.float8_e4m3fn: MLA_DTYPE_F8E4M3FN}.get(p.dtype, -1)
        d = CacheDesc()
        d.blocks = p.data_ptr()
        d.dtype = dt
        d.num_pages, d.num_layers, d.num_kv, d.page_size, d.num_heads, d.head_dim = p.shape
        d.stride_page, d.stride_layer, d.stride_kv, d.stride_token = p.stride(0), p.stride(1), p.stride(2), p.stride(3)
        pt = self.page_table
        if pt.dim() != 2 or not pt.is_contiguous() or pt.element_size() != 4:
            raise ValueError("page_table must be a contiguous 32-bit [batch, max_pages] tensor")
        d.page_table = pt.data_ptr()
        d.batch_size, d.max_pages_per_seq = pt.shape
        if self.cache_lengths is not None:
            cl = self.cache_lengths
            if not cl.is_contiguous() or cl.element_size() != 4 or cl.numel() != pt.shape[0]:
                raise ValueError("cache_lengths must be a contiguous 32-bit [batch] tensor")
            d.cache_lengths = cl.data_ptr()
        return d

    def scales_descriptor(self) -> ScalesDesc:
        import torch
        sc = self.scales
        if sc is None:
            raise ValueError("this cache has no scale pool")
        if sc.dim() != 5 or sc.dtype != torch.float32 or sc.stride(4) != 1:
            raise ValueError("scales must be float32 [pages, layers, kv, page_size, nblk] with contiguous rows")
        if tuple(sc.shape[:4]) != tuple(self.pool.shape[:4]):
            raise ValueError("scales must have the pool's pages, layers, kv halves and slots")
        d = ScalesDesc()
        d.scales = sc.data_ptr()
        d.granularity = int(self.scale_granularity)
        d.stride_page, d.stride_layer, d.stride_kv, d.stride_token = sc.stride(0), sc.stride(1), sc.stride(2), sc.stride(3)
        return d


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _u32(t, what):
    if t.element_size() != 4 or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous 32-bit tensor")
    return t.data_ptr()


def _check_outputs(M, desc, N, k_latent_buffer, k_buffer):
    D = desc.num_heads * desc.head_dim
    if k_latent_buffer.numel() < M * D or k_buffer.numel() < M * N:
        raise ValueError(f"outputs must hold at least [{M}, {D}] and [{M}, {N}] elements")
    if not (k_latent_buffer.is_contiguous() and k_buffer.is_contiguous()):
        raise ValueError("outputs must be contiguous")


def _check(status, what):
    if status != 0:
        if status == 8:
            raise MlaError(status, f"{what} (hipError {lib().mla_last_hip_error()})")
        raise MlaError(status, what)


# ---------------------------------------------------------------------------
# operations
# ---------------------------------------------------------------------------
def mla_decompress_k_paged(buffer_row_offsets, cache_offsets, buffer_length: int, weight,
                           cache: PagedKVCache, layer_idx: int, k_latent_buffer, k_buffer,
                           stream=None) -> None:
    """k_latent_buffer[r] = paged cache row; k_buffer = k_latent_buffer[:, :K] @ weight.T."""
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [N, K] tensor")
    N, K = weight.shape
    desc = cache.descriptor()
    _check_outputs(buffer_length, desc, N, k_latent_buffer, k_buffer)
    st = lib().mla_decompress_k_paged(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                      _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                      weight.data_ptr(), N, K, ctypes.byref(desc), int(layer_idx),
                                      k_latent_buffer.data_ptr(), k_buffer.data_ptr(), _stream(stream))
    _check(st, "mla_decompress_k_paged")


def mla_gather_latent_paged(buffer_row_offsets, cache_offsets, buffer_length: int, cache: PagedKVCache,
                            layer_idx: int, k_latent_buffer, stream=None) -> None:
    """k_latent_buffer[r] = paged cache row (the gather step alone)."""
    desc = cache.descriptor()
    D = desc.num_heads * desc.head_dim
    if k_latent_buffer.numel() < buffer_length * D or not k_latent_buffer.is_contiguous():
        raise ValueError(f"k_latent_buffer must be contiguous and hold at least [{buffer_length}, {D}]")
    st = lib().mla_gather_latent_paged(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                       _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                       ctypes.byref(desc), int(layer_idx), k_latent_buffer.data_ptr(),
                                       _stream(stream))
    _check(st, "mla_gather_latent_paged")


def mla_latent_matmul(k_latent_buffer, buffer_length: int, weight, k_buffer, stream=None) -> None:
    """k_buffer[:M] = k_latent_buffer[:M, :K] @ weight.T (the up-projection step alone).
    k_latent_buffer is a 2-D tensor with unit column stride (its row stride is passed)."""
    import torch
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [N, K] tensor")
    N, K = weight.shape
    if k_latent_buffer.dim() != 2 or k_latent_buffer.stride(1) != 1 or k_latent_buffer.shape[0] < buffer_length:
        raise ValueError("k_latent_buffer must be a [>= M, >= K] tensor with unit column stride")
    if k_latent_buffer.shape[1] < K or k_latent_buffer.dtype != weight.dtype or k_buffer.dtype != weight.dtype:
        raise ValueError("k_latent_buffer, weight and k_buffer must share a dtype, and K <= latent width")
    if k_buffer.numel() < buffer_length * N or not k_buffer.is_contiguous():
        raise ValueError(f"k_buffer must be contiguous and hold at least [{buffer_length}, {N}]")
    dt = {torch.float32: MLA_DTYPE_F32, torch.bfloat16: MLA_DTYPE_BF16}.get(weight.dtype, -1)
    st = lib().mla_latent_matmul(k_latent_buffer.data_ptr(), k_latent_buffer.stride(0), int(buffer_length),
                                 weight.data_ptr(), N, K, dt, k_buffer.data_ptr(), _stream(stream))
    _check(st, "mla_latent_matmul")


def mla_check_indices(row_offsets, cache_offsets, rows: int, cache: PagedKVCache, stream=None):
    """Debug validation of a call's index arrays (synchronous).  Returns
    (status, first failing request or -1); never raises on a failed check."""
    desc = cache.descriptor()
    bad = ctypes.c_int64(-1)
    st = lib().mla_check_indices(_u32(row_offsets, "row_offsets"),
                                 _u32(cache_offsets, "cache_offsets") if cache_offsets is not None else None,
                                 int(rows), ctypes.byref(desc), ctypes.byref(bad), _stream(stream))
    if st in (1, 7, 8):
        _check(st, "mla_check_indices")
    return st, int(bad.value)


def mla_decompress_k_paged_fp8_workspace_size(buffer_length: int, K: int, k_gran: int = 128) -> int:
    return int(lib().mla_decompress_k_paged_fp8_workspace_size(int(buffer_length), int(K), int(k_gran)))


def mla_decompress_k_paged_fp8(buffer_row_offsets, cache_offsets, buffer_length: int, weight_e4m3,
                               weight_scale, cache: PagedKVCache, layer_idx: int, k_latent_buffer,
                               k_buffer, workspace, m_gran: int = 1, n_gran: int = 128,
                               k_gran: int = 128, stream=None) -> None:
    """The fp8 block-scaled form; ``workspace`` is a uint8 device tensor of at least
    mla_decompress_k_paged_fp8_workspace_size(M, K) bytes."""
    if weight_e4m3.dim() != 2 or not weight_e4m3.is_contiguous():
        raise ValueError("weight_e4m3 must be a contiguous [N, K] tensor")
    N, K = weight_e4m3.shape
    desc = cache.descriptor()
    _check_outputs(buffer_length, desc, N, k_latent_buffer, k_buffer)
    if weight_scale.numel() < -(-N // n_gran) * -(-K // k_gran) or weight_scale.element_size() != 4:
        raise ValueError("weight_scale must hold float32 [N/n_gran, K/k_gran]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().mla_decompress_k_paged_fp8(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                          _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                          weight_e4m3.data_ptr(), weight_scale.data_ptr(), N, K,
                                          m_gran, n_gran, k_gran, ctypes.byref(desc), int(layer_idx),
                                          k_latent_buffer.data_ptr(), k_buffer.data_ptr(),
                                          workspace.data_ptr() if workspace is not None else None,
                                          ws_bytes, _stream(stream))
    _check(st, "mla_decompress_k_paged_fp8")


def _weight_shape(w, name):
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [N, K] tensor")
    return w.shape


def mla_decompress_kv_paged(buffer_row_offsets, cache_offsets, buffer_length: int, w_k, w_v,
                            cache: PagedKVCache, layer_idx: int, k_latent_buffer, k_buffer, v_buffer,
                            stream=None) -> None:
    """One gather, two up-projections: k_buffer = rows @ w_k.T, v_buffer = rows @ w_v.T."""
    N_k, K = _weight_shape(w_k, "w_k")
    N_v, K_v = _weight_shape(w_v, "w_v")
    if K_v != K:
        raise ValueError("w_k and w_v must have the same K")
    desc = cache.descriptor()
    _check_outputs(buffer_length, desc, N_k, k_latent_buffer, k_buffer)
    if v_buffer.numel() < buffer_length * N_v or not v_buffer.is_contiguous():
        raise ValueError(f"v_buffer must be contiguous and hold at least [{buffer_length}, {N_v}]")
    st = lib().mla_decompress_kv_paged(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                       _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                       w_k.data_ptr(), N_k, w_v.data_ptr(), N_v, K, ctypes.byref(desc),
                                       int(layer_idx), k_latent_buffer.data_ptr(), k_buffer.data_ptr(),
                                       v_buffer.data_ptr(), _stream(stream))
    _check(st, "mla_decompress_kv_paged")


def mla_decompress_kv_paged_fp8(buffer_row_offsets, cache_offsets, buffer_length: int, w_k_e4m3, w_k_scale,
                                w_v_e4m3, w_v_scale, cache: PagedKVCache, layer_idx: int, k_latent_buffer,
                                k_buffer, v_buffer, workspace, m_gran: int = 1, n_gran: int = 128,
                                k_gran: int = 128, stream=None) -> None:
    """The fp8 block-scaled fused form (one gather and quantisation, two products)."""
    N_k, K = _weight_shape(w_k_e4m3, "w_k_e4m3")
    N_v, K_v = _weight_shape(w_v_e4m3, "w_v_e4m3")
    if K_v != K:
        raise ValueError("w_k_e4m3 and w_v_e4m3 must have the same K")
    desc = cache.descriptor()
    _check_outputs(buffer_length, desc, N_k, k_latent_buffer, k_buffer)
    if v_buffer.numel() < buffer_length * N_v or not v_buffer.is_contiguous():
        raise ValueError(f"v_buffer must be contiguous and hold at least [{buffer_length}, {N_v}]")
    for sc, n, nm in ((w_k_scale, N_k, "w_k_scale"), (w_v_scale, N_v, "w_v_scale")):
        if sc.numel() < -(-n // n_gran) * -(-K // k_gran) or sc.element_size() != 4:
            raise ValueError(f"{nm} must hold float32 [N/n_gran, K/k_gran]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().mla_decompress_kv_paged_fp8(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                           _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                           w_k_e4m3.data_ptr(), w_k_scale.data_ptr(), N_k,
                                           w_v_e4m3.data_ptr(), w_v_scale.data_ptr(), N_v, K,
                                           m_gran, n_gran, k_gran, ctypes.byref(desc), int(layer_idx),
                                           k_latent_buffer.data_ptr(), k_buffer.data_ptr(), v_buffer.data_ptr(),
                                           workspace.data_ptr() if workspace is not None else None,
                                           ws_bytes, _stream(stream))
    _check(st, "mla_decompress_kv_paged_fp8")


def mla_decompress_k_paged_fp8_cache(buffer_row_offsets, cache_offsets, buffer_length: int, w_k_e4m3, w_k_scale,
                                     cache: PagedKVCache, layer_idx: int, k_latent_buffer, k_latent_scales, k_buffer,
                                     stream=None) -> None:
    """Gather e4m3 rows and their scales from an fp8 cache (bit copies into
    k_latent_buffer / k_latent_scales), then k_buffer = block-scaled rows @ w_k.T."""
    N, K = _weight_shape(w_k_e4m3, "w_k_e4m3")
    desc = cache.descriptor()
    sdesc = cache.scales_descriptor()
    D = desc.num_heads * desc.head_dim
    nblk = -(-D // 128)
    if k_latent_buffer.numel() * k_latent_buffer.element_size() < buffer_length * D or \
            not k_latent_buffer.is_contiguous() or k_latent_buffer.element_size() != 1:
        raise ValueError(f"k_latent_buffer must be a contiguous 1-byte tensor of at least [{buffer_length}, {D}]")
    if k_latent_scales.numel() < buffer_length * nblk or not k_latent_scales.is_contiguous() or \
            k_latent_scales.element_size() != 4:
        raise ValueError(f"k_latent_scales must be a contiguous float32 tensor of at least [{buffer_length}, {nblk}]")
    if k_buffer.numel() < buffer_length * N or not k_buffer.is_contiguous():
        raise ValueError(f"k_buffer must be contiguous and hold at least [{buffer_length}, {N}]")
    if w_k_scale.numel() < -(-N // 128) * -(-K // 128) or w_k_scale.element_size() != 4:
        raise ValueError("w_k_scale must hold float32 [N/128, K/128]")
    st = lib().mla_decompress_k_paged_fp8_cache(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                                _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                                w_k_e4m3.data_ptr(), w_k_scale.data_ptr(), N, K, ctypes.byref(desc),
                                                ctypes.byref(sdesc), int(layer_idx), k_latent_buffer.data_ptr(),
                                                k_latent_scales.data_ptr(), k_buffer.data_ptr(), _stream(stream))
    _check(st, "mla_decompress_k_paged_fp8_cache")


def mla_decompress_kv_paged_fp8_cache(buffer_row_offsets, cache_offsets, buffer_length: int, w_k_e4m3, w_k_scale,
                                      w_v_e4m3, w_v_scale, cache: PagedKVCache, layer_idx: int, k_latent_buffer,
                                      k_latent_scales, k_buffer, v_buffer, stream=None) -> None:
    """mla_decompress_k_paged_fp8_cache for K and, from the same gathered codes and
    scales, v_buffer = block-scaled rows @ w_v.T, in one gather and one product launch."""
    N, K = _weight_shape(w_k_e4m3, "w_k_e4m3")
    Nv, Kv = _weight_shape(w_v_e4m3, "w_v_e4m3")
    if Kv != K:
        raise ValueError("w_k_e4m3 and w_v_e4m3 must have the same K")
    desc = cache.descriptor()
    sdesc = cache.scales_descriptor()
    D = desc.num_heads * desc.head_dim
    nblk = -(-D // 128)
    if k_latent_buffer.numel() * k_latent_buffer.element_size() < buffer_length * D or \
            not k_latent_buffer.is_contiguous() or k_latent_buffer.element_size() != 1:
        raise ValueError(f"k_latent_buffer must be a contiguous 1-byte tensor of at least [{buffer_length}, {D}]")
    if k_latent_scales.numel() < buffer_length * nblk or not k_latent_scales.is_contiguous() or \
            k_latent_scales.element_size() != 4:
        raise ValueError(f"k_latent_scales must be a contiguous float32 tensor of at least [{buffer_length}, {nblk}]")
    for name, buf, n in (("k_buffer", k_buffer, N), ("v_buffer", v_buffer, Nv)):
        if buf.numel() < buffer_length * n or not buf.is_contiguous():
            raise ValueError(f"{name} must be contiguous and hold at least [{buffer_length}, {n}]")
    for name, sc, n in (("w_k_scale", w_k_scale, N), ("w_v_scale", w_v_scale, Nv)):
        if sc.numel() < -(-n // 128) * -(-K // 128) or sc.element_size() != 4:
            raise ValueError(f"{name} must hold float32 [{n}/128, K/128]")
    st = lib().mla_decompress_kv_paged_fp8_cache(_u32(buffer_row_offsets, "buffer_row_offsets"),
                                                 _u32(cache_offsets, "cache_offsets"), int(buffer_length),
                                                 w_k_e4m3.data_ptr(), w_k_scale.data_ptr(), N,
                                                 w_v_e4m3.data_ptr(), w_v_scale.data_ptr(), Nv, K,
                                                 ctypes.byref(desc), ctypes.byref(sdesc), int(layer_idx),
                                                 k_latent_buffer.data_ptr(), k_latent_scales.data_ptr(),
                                                 k_buffer.data_ptr(), v_buffer.data_ptr(), _stream(stream))
    _check(st, "mla_decompress_kv_paged_fp8_cache")


def mla_absorb_q(q, w_uk, q_latent, d_nope: int = 128, copy_rope: bool = True, stream=None) -> None:
    """q_latent[t, h, :L] = q[t, h, :d_nope] @ w_uk[h].T per head (L = kv_latent_dim),
    then, with copy_rope, the rope columns q[t, h, d_nope:] after it."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, H, d_nope + d_rope] tensor")
    if w_uk.dim() != 3 or not w_uk.is_contiguous():
        raise ValueError("w_uk must be a contiguous [H, kv_latent_dim, d_nope] tensor")
    T, H, Dq = q.shape
    if w_uk.shape[0] != H or w_uk.shape[2] != d_nope:
        raise ValueError(f"w_uk must be [{H}, kv_latent_dim, {d_nope}]")
    L = w_uk.shape[1]
    d_rope = Dq - d_nope
    Do = L + (d_rope if copy_rope else 0)
    if tuple(q_latent.shape) != (T, H, Do) or not q_latent.is_contiguous():
        raise ValueError(f"q_latent must be a contiguous [{T}, {H}, {Do}] tensor")
    st = lib().mla_absorb_q(q.data_ptr(), T, H, int(d_nope), int(d_rope), w_uk.data_ptr(), int(L),
                            1 if copy_rope else 0, q_latent.data_ptr(), _stream(stream))
    _check(st, "mla_absorb_q")


def mla_absorb_q_fp8(q, w_uk_e4m3, w_uk_scale, q_latent, d_nope: int = 128, copy_rope: bool = True,
                     stream=None) -> None:
    """The fp8 form: each head's non-rope query part quantised per 1x128 block,
    times the e4m3 w_uk with its 128x128 block scales."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, H, d_nope + d_rope] tensor")
    if w_uk_e4m3.dim() != 3 or not w_uk_e4m3.is_contiguous() or w_uk_e4m3.element_size() != 1:
        raise ValueError("w_uk_e4m3 must be a contiguous 1-byte [H, kv_latent_dim, d_nope] tensor")
    T, H, Dq = q.shape
    if w_uk_e4m3.shape[0] != H or w_uk_e4m3.shape[2] != d_nope:
        raise ValueError(f"w_uk_e4m3 must be [{H}, kv_latent_dim, {d_nope}]")
    L = w_uk_e4m3.shape[1]
    if w_uk_scale.numel() < H * (-(-L // 128)) * (-(-d_nope // 128)) or w_uk_scale.element_size() != 4:
        raise ValueError("w_uk_scale must hold float32 [H, kv_latent_dim / 128, d_nope / 128]")
    d_rope = Dq - d_nope
    Do = L + (d_rope if copy_rope else 0)
    if tuple(q_latent.shape) != (T, H, Do) or not q_latent.is_contiguous():
        raise ValueError(f"q_latent must be a contiguous [{T}, {H}, {Do}] tensor")
    st = lib().mla_absorb_q_fp8(q.data_ptr(), T, H, int(d_nope), int(d_rope), w_uk_e4m3.data_ptr(),
                                w_uk_scale.data_ptr(), int(L), 1, 128, 128, 1 if copy_rope else 0,
                                q_latent.data_ptr(), _stream(stream))
    _check(st, "mla_absorb_q_fp8")


def mla_write_latent_paged(kv_input, input_row_offsets, kv_norm_gamma, epsilon: float, freqs_cis, K: int,
                           cache: PagedKVCache, layer_idx: int, stream=None) -> None:
    """Append new tokens' rows (RMSNorm of the first K columns with kv_norm_gamma,
    the rest rotated by freqs_cis at each token's position) into the cache pages."""
    if kv_input.dim() != 2 or not kv_input.is_contiguous():
        raise ValueError("kv_input must be a contiguous [T, D_c] tensor")
    T = kv_input.shape[0]
    desc = cache.descriptor()
    if kv_input.shape[1] != desc.num_heads * desc.head_dim:
        raise ValueError("kv_input rows must be as wide as the cache rows")
    max_seq = freqs_cis.shape[0] if freqs_cis is not None else 0
    st = lib().mla_write_latent_paged(kv_input.data_ptr(), _u32(input_row_offsets, "input_row_offsets"), T,
                                      kv_norm_gamma.data_ptr(), float(epsilon),
                                      freqs_cis.data_ptr() if freqs_cis is not None else None, int(max_seq),
                                      int(K), ctypes.byref(desc), int(layer_idx), _stream(stream))
    _check(st, "mla_write_latent_paged")


def mla_write_latent_paged_fp8(kv_input, input_row_offsets, kv_norm_gamma, epsilon: float, freqs_cis, K: int,
                               cache: PagedKVCache, layer_idx: int, stream=None) -> None:
    """mla_write_latent_paged into an e4m3 cache: the same fp32 rows, quantised
    per 128 columns (codes into the pool, fp32 scales into the cache's scale pool)."""
    if kv_input.dim() != 2 or not kv_input.is_contiguous():
        raise ValueError("kv_input must be a contiguous [T, D_c] tensor")
    T = kv_input.shape[0]
    desc = cache.descriptor()
    sdesc = cache.scales_descriptor()
    if kv_input.shape[1] != desc.num_heads * desc.head_dim:
        raise ValueError("kv_input rows must be as wide as the cache rows")
    max_seq = freqs_cis.shape[0] if freqs_cis is not None else 0
    st = lib().mla_write_latent_paged_fp8(kv_input.data_ptr(), _u32(input_row_offsets, "input_row_offsets"), T,
                                          kv_norm_gamma.data_ptr(), float(epsilon),
                                          freqs_cis.data_ptr() if freqs_cis is not None else None, int(max_seq),
                                          int(K), ctypes.byref(desc), ctypes.byref(sdesc), int(layer_idx),
                                          _stream(stream))
    _check(st, "mla_write_latent_paged_fp8")


def kv_matmul_paged(hidden_state, input_row_offsets, weight, cache: PagedKVCache, layer_idx: int,
                    stream=None) -> None:
    """Append bf16(hidden_state @ weight) as K ([:HD]) and V ([HD:]) rows into the cache pages."""
    if hidden_state.dim() != 2 or not hidden_state.is_contiguous():
        raise ValueError("hidden_state must be a contiguous [T, hidden] tensor")
    T, Kd = hidden_state.shape
    desc = cache.descriptor()
    hd = desc.num_heads * desc.head_dim
    if tuple(weight.shape) != (Kd, 2 * hd) or not weight.is_contiguous():
        raise ValueError(f"weight must be a contiguous [{Kd}, {2 * hd}] tensor")
    if input_row_offsets.numel() != desc.batch_size + 1:
        raise ValueError("input_row_offsets must have batch_size + 1 entries")
    st = lib().kv_matmul_paged(hidden_state.data_ptr(), _u32(input_row_offsets, "input_row_offsets"),
                               T, Kd, weight.data_ptr(), ctypes.byref(desc), int(layer_idx),
                               _stream(stream))
    _check(st, "kv_matmul_paged")


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().mla_abi_version())
