"""Seeded synthetic inputs for the paged MLA latent-K path.

This module draws random numbers and lays out buffers: paged cache pools, page
tables, ragged row offsets, weights and hidden states.  It holds none of the
method's arithmetic -- no gather, no product, no quantisation of activations --
so that both sides of every parity check (the HIP library and the CPU oracle)
can take identical inputs from it without sharing any computation.

Cache pools are laid out ``[page][layer][kv][slot][head][dim]``, innermost
contiguous, as the paged KV cache collection of the MAX kernel pages is
described (a per-layer paged store addressed through a page table; page
"generic_flare_mla_decompress_k_cache_ragged_paged", Args ``kv_collection`` and
``layer_idx``).  Entries a kernel must never read are filled with a NaN poison
pattern: the other layer, spare pages, page-table slack (``0xFFFFFFFF``) and the
slots of a request's last page that lie beyond its cached length.

Numbers are drawn with numpy's PCG64 (``default_rng(seed)``), which is
reproducible across machines; bf16 and e4m3fn rounding of drawn values is done
by torch's CPU casts (round-to-nearest-even), i.e. input preparation, not the
method.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE_NONE = 0xFFFFFFFF
POISON_BF16 = np.uint16(0x7FC1)       # a quiet NaN in bfloat16
POISON_F32_BITS = np.uint32(0x7FC00001)  # a quiet NaN in binary32
POISON_E4M3 = np.uint8(0x7F)          # NaN in e4m3fn


# --------------------------------------------------------------------------
# element helpers (input preparation only)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (torch CPU cast, RNE) and return the bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP e4m3fn (torch CPU cast, RNE) and return the codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------------
# paged cache pool
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PagedCache:
    """A paged KV pool plus the page table of one batch of requests.

    ``pool`` holds raw element bits: uint16 for bf16, uint32 for f32, uint8
    codes for e4m3.  Shape ``[num_pages, num_layers, num_kv, page_size,
    num_heads, head_dim]``.  An e4m3 pool comes with ``scales``, float32
    ``[num_pages, num_layers, num_kv, page_size, ceil(row / scale_gran)]``:
    element j of a token's scales covers row columns [j*scale_gran, (j+1)*scale_gran).
    """
    pool: np.ndarray
    dtype: str                   # "bf16" | "f32" | "e4m3"
    page_table: np.ndarray       # uint32 [batch, max_pages_per_seq]
    cache_lengths: np.ndarray    # uint32 [batch] tokens already cached per request
    used_pages: int
    scales: Optional[np.ndarray] = None
    scale_gran: int = 128

    @property
    def num_pages(self) -> int: return self.pool.shape[0]
    @property
    def num_layers(self) -> int: return self.pool.shape[1]
    @property
    def num_kv(self) -> int: return self.pool.shape[2]
    @property
    def page_size(self) -> int: return self.pool.shape[3]
    @property
    def num_heads(self) -> int: return self.pool.shape[4]
    @property
    def head_dim(self) -> int: return self.pool.shape[5]
    @property
    def batch(self) -> int: return self.page_table.shape[0]
    @property
    def max_pages_per_seq(self) -> int: return self.page_table.shape[1]

    def strides(self):
        """Element strides (page, layer, kv, token) of the contiguous pool."""
        s = self.pool.strides
        e = self.pool.itemsize
        return s[0] // e, s[1] // e, s[2] // e, s[3] // e

    @property
    def elem_bytes(self) -> int: return self.pool.itemsize

    def scale_strides(self):
        """Element strides (page, layer, kv, token) of the scale pool."""
        s = self.scales.strides
        return s[0] // 4, s[1] // 4, s[2] // 4, s[3] // 4

    @property
    def scale_blocks(self) -> int: return self.scales.shape[4]


def _allocate_pages(rng, pages_needed, spare_frac):
    used = int(sum(pages_needed))
    spare = max(1, int(math.ceil(spare_frac * used)))
    num_pages = used + spare
    perm = rng.permutation(num_pages).astype(np.uint32)
    maxp = max(1, max(pages_needed))
    table = np.full((len(pages_needed), maxp), PAGE_NONE, dtype=np.uint32)
    cur = 0
    for b, n in enumerate(pages_needed):
        table[b, :n] = perm[cur:cur + n]
        cur += n
    return num_pages, table, used


def make_paged_cache(rng, *, cache_lengths, page_size, num_heads, head_dim,
                     dtype="bf16", num_kv=1, num_layers=2, layer_idx=1,
                     value_std=1.0, spare_frac=0.1, fill="normal",
                     extra_tokens=None, scale_gran=128) -> PagedCache:
    """Build a poisoned pool whose referenced pages hold N(0, value_std) values.

    ``extra_tokens[b]`` reserves room for tokens to be appended after the cached
    ones (the write path); those slots start as poison.
    ``fill="tag"`` (f32 only) writes into every element the tag
    ``page<<20 | layer<<19 | kv<<18 | slot<<10 | col`` as raw binary32 bits, so a
    gathered element names where it came from.

    ``dtype="e4m3"``: codes e4m3fn(clip(100 * N(0, 1), -448, 448)) with one fp32
    scale U[0.008, 0.012] per ``scale_gran`` columns of each token row (so the
    stored values are about N(0, 1)); poison is code 0x7F and scale NaN.  With
    ``fill="tag"`` the scale of block j of (page, layer, kv, slot) is the exact
    float ``page*65536 + layer*32768 + kv*16384 + slot*64 + j`` and code c of
    column i is ``(i + 3*slot + 5*page) % 126`` (a finite positive code).
    """
    cache_lengths = np.asarray(cache_lengths, dtype=np.int64)
    extra = np.zeros_like(cache_lengths) if extra_tokens is None else np.asarray(extra_tokens, np.int64)
    pages_needed = [int(math.ceil((int(c) + int(e)) / page_size)) for c, e in zip(cache_lengths, extra)]
    num_pages, table, used = _allocate_pages(rng, pages_needed, spare_frac)
    shape = (num_pages, num_layers, num_kv, page_size, num_heads, head_dim)
    row = num_heads * head_dim

    if dtype == "bf16":
        pool = np.full(shape, POISON_BF16, dtype=np.uint16)
    elif dtype == "f32":
        pool = np.full(shape, POISON_F32_BITS, dtype=np.uint32)
    elif dtype == "e4m3":
        return _make_e4m3_cache(rng, shape, table, cache_lengths, pages_needed, used, layer_idx, fill, scale_gran)
    else:
        raise ValueError(dtype)

    if fill == "tag":
        assert dtype == "f32" and page_size <= 256 and row <= 1024 and num_pages < 4096
        pg = np.arange(num_pages, dtype=np.uint32)[:, None, None, None, None]
        ly = np.arange(num_layers, dtype=np.uint32)[None, :, None, None, None]
        kv = np.arange(num_kv, dtype=np.uint32)[None, None, :, None, None]
        sl = np.arange(page_size, dtype=np.uint32)[None, None, None, :, None]
        col = np.arange(row, dtype=np.uint32)[None, None, None, None, :]
        tag = (pg << 20) | (ly << 19) | (kv << 18) | (sl << 10) | col
        pool[...] = tag.reshape(shape)
        return PagedCache(pool, dtype, table, cache_lengths.astype(np.uint32), used)

    # referenced layer of every used page: random values over all slots, then
    # poison the slots past each request's cached length in its last page
    for b, n in enumerate(pages_needed):
        if n == 0:
            continue
        ids = table[b, :n].astype(np.int64)
        vals = rng.standard_normal((n, num_kv, page_size, row), dtype=np.float32) * np.float32(value_std)
        if dtype == "bf16":
            bits = to_bf16_bits(vals)
        else:
            bits = vals.view(np.uint32)
        pool[ids, layer_idx] = bits.reshape(n, num_kv, page_size, num_heads, head_dim)
        tail = int(cache_lengths[b])
        for p in range(tail, n * page_size):
            pool[ids[p // page_size], layer_idx, :, p % page_size] = (
                POISON_BF16 if dtype == "bf16" else POISON_F32_BITS)
    return PagedCache(pool, dtype, table, cache_lengths.astype(np.uint32), used)


def _make_e4m3_cache(rng, shape, table, cache_lengths, pages_needed, used, layer_idx, fill, gran):
    num_pages, num_layers, num_kv, page_size, num_heads, head_dim = shape
    row = num_heads * head_dim
    nblk = -(-row // gran)
    pool = np.full(shape, POISON_E4M3, dtype=np.uint8)
    sbits = np.full((num_pages, num_layers, num_kv, page_size, nblk), POISON_F32_BITS, dtype=np.uint32)
    scales = sbits.view(np.float32)
    if fill == "tag":
        assert num_pages <= 256 and page_size <= 256 and nblk <= 64
        pg = np.arange(num_pages)[:, None, None, None, None]
        ly = np.arange(num_layers)[None, :, None, None, None]
        kv = np.arange(num_kv)[None, None, :, None, None]
        sl = np.arange(page_size)[None, None, None, :, None]
        j = np.arange(nblk)[None, None, None, None, :]
        scales[...] = (pg * 65536 + ly * 32768 + kv * 16384 + sl * 64 + j).astype(np.float32)
        col = np.arange(row)[None, None, None, None, :]
        codes = (col + 3 * sl + 5 * pg) % 126 + 0 * ly + 0 * kv
        pool[...] = codes.astype(np.uint8).reshape(shape)
        return PagedCache(pool, "e4m3", table, cache_lengths.astype(np.uint32), used, scales, gran)
    for b, n in enumerate(pages_needed):
        if n == 0:
            continue
        ids = table[b, :n].astype(np.int64)
        vals = np.clip(rng.standard_normal((n, num_kv, page_size, row), dtype=np.float32) * np.float32(100.0),
                       -448.0, 448.0)
        pool[ids, layer_idx] = to_e4m3_bits(vals).reshape(n, num_kv, page_size, num_heads, head_dim)
        scales[ids, layer_idx] = rng.uniform(0.008, 0.012, size=(n, num_kv, page_size, nblk)).astype(np.float32)
        tail = int(cache_lengths[b])
        for p in range(tail, n * page_size):
            pool[ids[p // page_size], layer_idx, :, p % page_size] = POISON_E4M3
            sbits[ids[p // page_size], layer_idx, :, p % page_size] = POISON_F32_BITS
    return PagedCache(pool, "e4m3", table, cache_lengths.astype(np.uint32), used, scales, gran)


# --------------------------------------------------------------------------
# decompress cases (gather + up-projection)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DecompressCase:
    name: str
    cache: PagedCache
    layer_idx: int
    buffer_row_offsets: np.ndarray  # uint32 [B+1]
    cache_offsets: np.ndarray       # uint32 [B]
    K: int                          # kv_lora_rank (latent columns used by the product)
    N: int                          # num_heads * qk_nope_head_dim
    weight: Optional[np.ndarray]    # bits [N, K]: uint16 (bf16) or uint32 (f32)
    weight_dtype: str               # "bf16" | "f32" | "e4m3"
    weight_q: Optional[np.ndarray] = None      # uint8 e4m3fn codes [N, K]
    weight_scale: Optional[np.ndarray] = None  # float32 [ceil(N/128), ceil(K/128)]
    n_gran: int = 128
    k_gran: int = 128

    @property
    def M(self) -> int: return int(self.buffer_row_offsets[-1])
    @property
    def D_c(self) -> int: return self.cache.num_heads * self.cache.head_dim
    @property
    def batch(self) -> int: return len(self.buffer_row_offsets) - 1


def decompress_case(name, *, seed, cache_lengths, cache_offsets, page_size,
                    kv_lora_rank, rope_dim, N, dtype="bf16", w_std=0.02,
                    num_layers=2, layer_idx=1, fp8=False, fill="normal",
                    rows=None, spare_frac=0.1) -> DecompressCase:
    """One request batch: ``rows[b]`` latent rows are copied from cache position
    ``cache_offsets[b]`` onward (default: to the end of the cached length)."""
    rng = np.random.default_rng(seed)
    cache_lengths = np.asarray(cache_lengths, dtype=np.int64)
    cache_offsets = np.asarray(cache_offsets, dtype=np.int64)
    if rows is None:
        rows = cache_lengths - cache_offsets
    rows = np.asarray(rows, dtype=np.int64)
    assert np.all(rows >= 0) and np.all(cache_offsets + rows <= cache_lengths)
    D_c = kv_lora_rank + rope_dim
    cache = make_paged_cache(rng, cache_lengths=cache_lengths, page_size=page_size,
                             num_heads=1, head_dim=D_c, dtype=dtype, num_kv=1,
                             num_layers=num_layers, layer_idx=layer_idx, fill=fill,
                             spare_frac=spare_frac)
    bro = np.zeros(len(rows) + 1, dtype=np.uint32)
    bro[1:] = np.cumsum(rows)
    case = DecompressCase(name, cache, layer_idx, bro, cache_offsets.astype(np.uint32),
                          kv_lora_rank, N, None, dtype)
    if fp8:
        assert dtype in ("bf16", "e4m3")
        payload = rng.standard_normal((N, kv_lora_rank), dtype=np.float32)
        case.weight_q = to_e4m3_bits(payload)
        nb, kb = -(-N // 128), -(-kv_lora_rank // 128)
        case.weight_scale = rng.uniform(0.015, 0.025, size=(nb, kb)).astype(np.float32)
        case.weight_dtype = "e4m3"
    else:
        w = rng.standard_normal((N, kv_lora_rank), dtype=np.float32) * np.float32(w_std)
        case.weight = to_bf16_bits(w) if dtype == "bf16" else w.view(np.uint32).copy()
    return case


def with_second_projection(case: DecompressCase, *, seed, N, w_std=0.02) -> DecompressCase:
    """``case`` with its weight replaced by another projection of the same rows
    (W_uv for the fused K and V form): same cache, offsets and K, a new [N, K]
    weight drawn like the first (bf16/f32 N(0, w_std); e4m3 payload N(0,1) with
    128x128 scales U[0.015, 0.025])."""
    rng = np.random.default_rng(seed)
    v = dataclasses.replace(case, name=case.name + "_v", N=N, weight=None, weight_q=None, weight_scale=None)
    if case.weight_dtype == "e4m3":
        v.weight_q = to_e4m3_bits(rng.standard_normal((N, case.K), dtype=np.float32))
        v.weight_scale = rng.uniform(0.015, 0.025, size=(-(-N // 128), -(-case.K // 128))).astype(np.float32)
    else:
        w = rng.standard_normal((N, case.K), dtype=np.float32) * np.float32(w_std)
        v.weight = to_bf16_bits(w) if case.weight_dtype == "bf16" else w.view(np.uint32).copy()
    return v


# --------------------------------------------------------------------------
# write-path cases (projection + scatter into K/V pages)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class KvMatmulCase:
    name: str
    cache: PagedCache               # num_kv == 2, bf16; cache_lengths = start positions
    layer_idx: int
    hidden: np.ndarray              # uint16 bf16 bits [T, hidden_dim]
    input_row_offsets: np.ndarray   # uint32 [B+1]
    weight: np.ndarray              # uint16 bf16 bits [hidden_dim, 2*Hkv*D]

    @property
    def T(self) -> int: return int(self.input_row_offsets[-1])
    @property
    def hidden_dim(self) -> int: return self.hidden.shape[1]
    @property
    def N(self) -> int: return self.weight.shape[1]


def lognormal_lengths(rng, batch, median, sigma, max_len):
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=batch)
    return np.clip(np.round(x), 1, max_len).astype(np.int64)


def kv_matmul_case(name, *, seed, seq_lens, start_lengths, hidden_dim, num_kv_heads,
                   head_dim, page_size, w_std=0.02, num_layers=2, layer_idx=1,
                   weight=None) -> KvMatmulCase:
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    start_lengths = np.asarray(start_lengths, dtype=np.int64)
    cache = make_paged_cache(rng, cache_lengths=start_lengths, page_size=page_size,
                             num_heads=num_kv_heads, head_dim=head_dim, dtype="bf16",
                             num_kv=2, num_layers=num_layers, layer_idx=layer_idx,
                             extra_tokens=seq_lens)
    T = int(seq_lens.sum())
    iro = np.zeros(len(seq_lens) + 1, dtype=np.uint32)
    iro[1:] = np.cumsum(seq_lens)
    hidden = to_bf16_bits(rng.standard_normal((T, hidden_dim), dtype=np.float32))
    N = 2 * num_kv_heads * head_dim
    if weight is None:
        w = rng.standard_normal((hidden_dim, N), dtype=np.float32) * np.float32(w_std)
        weight = to_bf16_bits(w)
    return KvMatmulCase(name, cache, layer_idx, hidden, iro, np.ascontiguousarray(weight))


# --------------------------------------------------------------------------
# latent write-path cases (RMSNorm + RoPE + scatter into the MLA pages)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LatentWriteCase:
    name: str
    cache: PagedCache               # num_kv == 1, bf16; cache_lengths = start positions
    layer_idx: int
    x: np.ndarray                   # uint16 bf16 bits [T, D_c]: latent K then rope R columns
    input_row_offsets: np.ndarray   # uint32 [B+1]
    gamma: np.ndarray               # float32 [K]
    eps: float
    freqs: np.ndarray               # float32 [max_seq_len, R]: (cos, sin) per rope pair
    K: int

    @property
    def T(self) -> int: return int(self.input_row_offsets[-1])


def rope_table(max_seq_len, R, base=10000.0):
    """float32 [max_seq_len, R]: (cos, sin) of position p times base^(-2j/R) for
    rope pair j, interleaved."""
    j = np.arange(R // 2, dtype=np.float64)
    ang = np.arange(max_seq_len, dtype=np.float64)[:, None] * base ** (-2.0 * j / R)[None, :]
    out = np.empty((max_seq_len, R), np.float32)
    out[:, 0::2] = np.cos(ang)
    out[:, 1::2] = np.sin(ang)
    return out


def latent_write_case(name, *, seed, seq_lens, start_lengths, page_size, K=512, R=64, num_layers=2,
                      layer_idx=1, eps=1e-6, max_seq_len=None, dtype="bf16", fill="normal") -> LatentWriteCase:
    """New tokens (latent N(0,1), rope N(0,1), bf16) appended after each request's
    cached ones in an MLA cache of rows K + R; RMSNorm weights U[0.5, 1.5].
    dtype="e4m3": an e4m3 cache with one fp32 scale per 128 columns (fill as
    make_paged_cache)."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    start_lengths = np.asarray(start_lengths, dtype=np.int64)
    cache = make_paged_cache(rng, cache_lengths=start_lengths, page_size=page_size, num_heads=1,
                             head_dim=K + R, dtype=dtype, num_kv=1, num_layers=num_layers,
                             layer_idx=layer_idx, extra_tokens=seq_lens, fill=fill)
    T = int(seq_lens.sum())
    iro = np.zeros(len(seq_lens) + 1, dtype=np.uint32)
    iro[1:] = np.cumsum(seq_lens)
    x = to_bf16_bits(rng.standard_normal((T, K + R), dtype=np.float32))
    gamma = rng.uniform(0.5, 1.5, size=K).astype(np.float32)
    if max_seq_len is None:
        max_seq_len = int((start_lengths + seq_lens).max()) + 1
    return LatentWriteCase(name, cache, layer_idx, x, iro, gamma, float(eps), rope_table(max_seq_len, R), K)


def c5_latent_write_fp8(seed=5) -> LatentWriteCase:
    """The c5 write batch into an e4m3 cache (one fp32 scale per 128 columns)."""
    rng = np.random.default_rng(seed + 1000)
    lens = lognormal_lengths(rng, 128, 512, 1.0, 8192)
    return latent_write_case("c5_latent_write_fp8", seed=seed, seq_lens=lens, start_lengths=np.zeros(128, np.int64),
                             page_size=128, dtype="e4m3")


def c5_latent_write(seed=5) -> LatentWriteCase:
    """The write-path batch shape of the kv projection (128 requests, lengths
    lognormal(ln 512, 1) clipped to [1, 8192], fresh requests) writing 576-wide
    latent rows (512 + 64 rope), page_size 128."""
    rng = np.random.default_rng(seed + 1000)
    lens = lognormal_lengths(rng, 128, 512, 1.0, 8192)
    return latent_write_case("c5_latent_write", seed=seed, seq_lens=lens, start_lengths=np.zeros(128, np.int64),
                             page_size=128)


# --------------------------------------------------------------------------
# query absorption cases (q_nope x w_uk per head)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class AbsorbCase:
    name: str
    q: np.ndarray          # uint16 bf16 bits [T, H, d_nope + d_rope]
    w_uk: np.ndarray       # uint16 bf16 bits [H, kv_latent_dim, d_nope]
    d_nope: int
    copy_rope: bool = True
    w_q: Optional[np.ndarray] = None       # e4m3 form: uint8 codes [H, kv_latent_dim, d_nope]
    w_scale: Optional[np.ndarray] = None   # float32 [H, kv_latent_dim / 128, d_nope / 128]

    @property
    def T(self) -> int: return self.q.shape[0]
    @property
    def H(self) -> int: return self.q.shape[1]
    @property
    def d_rope(self) -> int: return self.q.shape[2] - self.d_nope
    @property
    def kv_latent_dim(self) -> int: return self.w_uk.shape[1]
    @property
    def out_dim(self) -> int: return self.kv_latent_dim + (self.d_rope if self.copy_rope else 0)


def absorb_case(name, *, seed, T, H=128, d_nope=128, d_rope=64, kv_latent_dim=512, w_std=0.05,
                copy_rope=True, fp8=False) -> AbsorbCase:
    """Queries bf16 N(0, 1) [T, H, d_nope + d_rope]; w_uk bf16 N(0, w_std)
    [H, kv_latent_dim, d_nope].  fp8: w_uk as e4m3 codes of N(0, 1) with fp32
    scales U[0.04, 0.06] per 128 x 128 block of each head (about N(0, 0.05))."""
    rng = np.random.default_rng(seed)
    q = to_bf16_bits(rng.standard_normal((T, H, d_nope + d_rope), dtype=np.float32))
    w = to_bf16_bits(rng.standard_normal((H, kv_latent_dim, d_nope), dtype=np.float32) * np.float32(w_std))
    case = AbsorbCase(name, q, w, d_nope, copy_rope)
    if fp8:
        case.w_q = to_e4m3_bits(rng.standard_normal((H, kv_latent_dim, d_nope), dtype=np.float32))
        case.w_scale = rng.uniform(0.04, 0.06, size=(H, -(-kv_latent_dim // 128), -(-d_nope // 128))).astype(np.float32)
    return case


def c7_absorb(seed=7) -> AbsorbCase:
    """A decode step of 128 requests, one new token each: 128 query heads of
    128 nope + 64 rope columns, w_uk [128, 512, 128]."""
    return absorb_case("c7_absorb", seed=seed, T=128)


def c7_absorb_fp8(seed=7) -> AbsorbCase:
    """c7_absorb with an e4m3 w_uk and its 128 x 128 block scales."""
    return absorb_case("c7_absorb_fp8", seed=seed, T=128, fp8=True)


def device_absorb(case: AbsorbCase, device="cuda"):
    t = {"q": _bits_to_torch(case.q, device), "w_uk": _bits_to_torch(case.w_uk, device)}
    if case.w_q is not None:
        t["w_uk_e4m3"] = _bits_to_torch(case.w_q, device)
        t["w_uk_scale"] = torch.from_numpy(np.ascontiguousarray(case.w_scale)).to(device)
    return t


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
def c0_tiny(seed=0) -> DecompressCase:
    """2 requests with 5 and 11 cached tokens, copies starting at 0 and 3;
    page_size 16; one latent head of 80 (64 latent + 16 rope); pool of 8
    permuted pages; W_k [128 = 4 heads x 32, 64]; f32 N(0,1) latents, N(0,0.05) W."""
    return decompress_case("c0_tiny", seed=seed, cache_lengths=[5, 11], cache_offsets=[0, 3],
                           page_size=16, kv_lora_rank=64, rope_dim=16, N=128, dtype="f32",
                           w_std=0.05, spare_frac=(8 - 2) / 2)


def c1_decode(seed=1) -> DecompressCase:
    """64 requests, cached lengths U{256..4096}, copies from position 0,
    page_size 128, rows of 576 (512 latent + 64 rope), W_k [16384, 512] bf16 N(0,0.02)."""
    rng = np.random.default_rng(seed + 1000)
    lens = rng.integers(256, 4096, size=64, endpoint=True)
    return decompress_case("c1_decode", seed=seed, cache_lengths=lens, cache_offsets=np.zeros(64, np.int64),
                           page_size=128, kv_lora_rank=512, rope_dim=64, N=16384)


def c2_prefill(seed=2, fp8=False, name="c2_prefill") -> DecompressCase:
    """4 requests of 16384 rows each; copies start at U{0..8192} (prefix reuse);
    cached length = start + 16384; page_size 128; rows of 576; W_k [16384, 512]."""
    rng = np.random.default_rng(seed + 1000)
    offs = rng.integers(0, 8192, size=4, endpoint=True)
    return decompress_case(name, seed=seed, cache_lengths=offs + 16384, cache_offsets=offs,
                           page_size=128, kv_lora_rank=512, rope_dim=64, N=16384, fp8=fp8)


def c3_fp8(seed=3) -> DecompressCase:
    """The 64K-row prefill shapes with an e4m3fn W_k (payload N(0,1)) and fp32
    128x128 block scales U[0.015, 0.025]; activations quantised per 1x128."""
    return c2_prefill(seed=seed, fp8=True, name="c3_fp8")


def c6_fp8_cache(seed=6) -> DecompressCase:
    """The 64K-row prefill shapes read from an e4m3 cache (codes with one fp32
    scale per 128 columns of each 576-wide row, values about N(0, 1)) with an
    e4m3fn W_k (payload N(0,1), 128x128 scales U[0.015, 0.025])."""
    rng = np.random.default_rng(seed + 1000)
    offs = rng.integers(0, 8192, size=4, endpoint=True)
    return decompress_case("c6_fp8_cache", seed=seed, cache_lengths=offs + 16384, cache_offsets=offs,
                           page_size=128, kv_lora_rank=512, rope_dim=64, N=16384, dtype="e4m3", fp8=True)


def c4_kv_matmul(seed=4, start="zero") -> KvMatmulCase:
    """128 requests of lognormal lengths (median 512, sigma 1, clipped to
    [1, 8192]); hidden [T, 4096] bf16 N(0,1); W [4096, 2*8*128] bf16 N(0,0.02);
    cache of 2 (K,V) x 8 heads x 128, page_size 128, shuffled pages.
    ``start="zero"``: fresh requests; ``"random"``: U{0..1000} tokens already cached."""
    rng = np.random.default_rng(seed + 1000)
    lens = lognormal_lengths(rng, 128, 512, 1.0, 8192)
    starts = np.zeros(128, np.int64) if start == "zero" else rng.integers(0, 1000, size=128, endpoint=True)
    return kv_matmul_case("c4_kv_matmul", seed=seed, seq_lens=lens, start_lengths=starts,
                          hidden_dim=4096, num_kv_heads=8, head_dim=128, page_size=128)


CONFIGS = {
    "c0_tiny": c0_tiny,
    "c1_decode": c1_decode,
    "c2_prefill": c2_prefill,
    "c3_fp8": c3_fp8,
    "c4_kv_matmul": c4_kv_matmul,
}


# --------------------------------------------------------------------------
# small parity shapes: several tiles and ragged tails, seconds for the oracle
# --------------------------------------------------------------------------
def small_decompress(seed, *, batch=5, max_len=300, page_size=16, K=512, rope=64, N=512,
                     dtype="bf16", fp8=False, offsets="random", w_std=0.02) -> DecompressCase:
    rng = np.random.default_rng(seed + 5000)
    lens = rng.integers(1, max_len, size=batch, endpoint=True)
    if offsets == "random":
        offs = np.array([rng.integers(0, l) for l in lens], dtype=np.int64)
    else:
        offs = np.zeros(batch, np.int64)
    return decompress_case(f"small_s{seed}", seed=seed, cache_lengths=lens, cache_offsets=offs,
                           page_size=page_size, kv_lora_rank=K, rope_dim=rope, N=N,
                           dtype=dtype, fp8=fp8, w_std=w_std)


def small_kv_matmul(seed, *, batch=6, max_len=200, hidden_dim=256, num_kv_heads=2,
                    head_dim=128, page_size=16, start="random") -> KvMatmulCase:
    rng = np.random.default_rng(seed + 6000)
    lens = rng.integers(1, max_len, size=batch, endpoint=True)
    starts = rng.integers(0, 40, size=batch, endpoint=True) if start == "random" else np.zeros(batch, np.int64)
    return kv_matmul_case(f"small_kv_s{seed}", seed=seed, seq_lens=lens, start_lengths=starts,
                          hidden_dim=hidden_dim, num_kv_heads=num_kv_heads, head_dim=head_dim,
                          page_size=page_size)


# --------------------------------------------------------------------------
# device copies (torch tensors on the current HIP device)
# --------------------------------------------------------------------------
def _bits_to_torch(bits: np.ndarray, device):
    if bits.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    if bits.dtype == np.uint32:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).to(device)
    if bits.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    raise ValueError(bits.dtype)


def _u32_to_torch(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


@dataclasses.dataclass
class DeviceCache:
    pool: "torch.Tensor"
    page_table: "torch.Tensor"
    cache_lengths: "torch.Tensor"
    scales: Optional["torch.Tensor"] = None


def device_cache(cache: PagedCache, device="cuda") -> DeviceCache:
    sc = None
    if cache.scales is not None:
        sc = torch.from_numpy(np.ascontiguousarray(cache.scales)).to(device)
    return DeviceCache(_bits_to_torch(cache.pool, device), _u32_to_torch(cache.page_table, device),
                       _u32_to_torch(cache.cache_lengths, device), sc)


def device_decompress(case: DecompressCase, device="cuda"):
    """(DeviceCache, dict of device tensors) for a decompress case."""
    dc = device_cache(case.cache, device)
    t = {"buffer_row_offsets": _u32_to_torch(case.buffer_row_offsets, device),
         "cache_offsets": _u32_to_torch(case.cache_offsets, device)}
    if case.weight_dtype == "e4m3":
        t["weight_q"] = _bits_to_torch(case.weight_q, device)
        t["weight_scale"] = torch.from_numpy(case.weight_scale).to(device)
    else:
        t["weight"] = _bits_to_torch(case.weight, device)
    return dc, t


def device_latent_write(case: LatentWriteCase, device="cuda"):
    dc = device_cache(case.cache, device)
    t = {"x": _bits_to_torch(case.x, device),
         "input_row_offsets": _u32_to_torch(case.input_row_offsets, device),
         "gamma": torch.from_numpy(case.gamma).to(device),
         "freqs": torch.from_numpy(case.freqs).to(device)}
    return dc, t


def device_kv(case: KvMatmulCase, device="cuda"):
    dc = device_cache(case.cache, device)
    t = {"hidden": _bits_to_torch(case.hidden, device),
         "input_row_offsets": _u32_to_torch(case.input_row_offsets, device),
         "weight": _bits_to_torch(case.weight, device)}
    return dc, t
