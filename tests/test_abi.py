"""The C-ABI library loads, exports every function include/mla_paged.h declares,
and returns the documented status for every host-side error -- all without a
GPU (no call here reaches a kernel launch: validation fails first, or the
device check refuses a machine without a gfx950)."""
import ctypes
import os
import re

import pytest

import mla_paged_latent_page_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_paged.h")

OK, NULLP, SHAPE, DTYPE, MISAL, RANGE, WS, DEV, HIP = range(9)
FAKE = 0x100000  # an aligned non-null address; never dereferenced by the host checks


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return mp.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:mla_status_t|size_t|const char\s*\*|int32_t)\s+(\w+)\s*\(", text, re.M)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(mp.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_abi_version() == 1


def test_status_strings(lib):
    for s in range(9):
        assert lib.mla_status_string(s)
    assert b"gfx950" in lib.mla_status_string(DEV)


def cache_desc(dtype=1, num_kv=1, heads=1, head_dim=576, page_size=128, layers=2, pages=16, batch=2, maxp=4,
               with_lengths=False):
    d = mp.CacheDesc()
    d.blocks = FAKE
    d.dtype = dtype
    d.num_layers, d.num_pages, d.page_size, d.num_kv = layers, pages, page_size, num_kv
    d.num_heads, d.head_dim = heads, head_dim
    d.page_table = FAKE
    d.batch_size, d.max_pages_per_seq = batch, maxp
    d.cache_lengths = FAKE if with_lengths else None
    assert mp.lib().mla_paged_cache_default_strides(ctypes.byref(d)) == OK
    return d


def decompress(lib, d, M=100, N=512, K=512, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, w=FAKE, lat=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.mla_decompress_k_paged(p["bro"], p["co"], M, p["w"], N, K,
                                      ctypes.byref(d) if d is not None else None, layer, p["lat"], p["out"], None)


def test_default_strides(lib):
    d = cache_desc(num_kv=2, heads=8, head_dim=128, page_size=16, layers=3)
    assert (d.stride_token, d.stride_kv, d.stride_layer, d.stride_page) == (1024, 16 * 1024, 2 * 16 * 1024,
                                                                           3 * 2 * 16 * 1024)
    assert lib.mla_paged_cache_default_strides(None) == NULLP


def test_decompress_error_paths(lib):
    d = cache_desc()
    assert decompress(lib, None) == NULLP
    for k in ("bro", "co", "w", "lat", "out"):
        assert decompress(lib, d, **{k: None}) == NULLP
    assert decompress(lib, d, M=-1) == SHAPE
    assert decompress(lib, d, K=1024) == SHAPE          # K > D_c
    assert decompress(lib, d, K=96) == SHAPE            # bf16 needs K % 64
    assert decompress(lib, d, N=100) == SHAPE           # bf16 needs N % 64
    assert decompress(lib, cache_desc(num_kv=2)) == SHAPE
    assert decompress(lib, cache_desc(page_size=0)) == SHAPE
    assert decompress(lib, cache_desc(dtype=2)) == DTYPE
    assert decompress(lib, d, w=FAKE + 8) == MISAL
    assert decompress(lib, d, out=FAKE + 2) == MISAL
    assert decompress(lib, cache_desc(head_dim=572)) == MISAL   # bf16 row of 1144 bytes
    assert decompress(lib, d, layer=2) == RANGE
    # zero rows: host checks only, nothing enqueued, OK even without pointers
    assert decompress(lib, d, M=0, bro=None, co=None, w=None, lat=None, out=None) == OK
    # a valid call on a machine without a gfx950
    assert decompress(lib, d) == DEV
    assert decompress(lib, cache_desc(dtype=0, head_dim=80, page_size=16), N=128, K=64) == DEV


def fp8(lib, d, M=100, N=512, K=512, grans=(1, 128, 128), ws=None, ws_bytes=None, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, w=FAKE, sw=FAKE, lat=FAKE, out=FAKE)
    p.update(ptrs)
    need = lib.mla_decompress_k_paged_fp8_workspace_size(max(M, 0), K, 128)
    return lib.mla_decompress_k_paged_fp8(p["bro"], p["co"], M, p["w"], p["sw"], N, K, *grans,
                                          ctypes.byref(d), layer, p["lat"], p["out"],
                                          FAKE if ws is None else ws,
                                          need if ws_bytes is None else ws_bytes, None)


def test_fp8_workspace_size(lib):
    assert lib.mla_decompress_k_paged_fp8_workspace_size(65536, 512, 128) == 65536 * 512 + 65536 * 4 * 4
    assert lib.mla_decompress_k_paged_fp8_workspace_size(3, 256, 128) == 768 + 256  # align256(3*256) + align256(3*2*4)
    assert lib.mla_decompress_k_paged_fp8_workspace_size(3, 256, 64) == 0
    assert lib.mla_decompress_k_paged_fp8_workspace_size(-1, 256, 128) == 0


def test_fp8_error_paths(lib):
    d = cache_desc()
    for k in ("bro", "co", "w", "sw", "lat", "out"):
        assert fp8(lib, d, **{k: None}) == NULLP
    assert fp8(lib, d, ws=0) == NULLP
    assert fp8(lib, d, grans=(1, 128, 64)) == SHAPE
    assert fp8(lib, d, grans=(128, 128, 128)) == SHAPE
    assert fp8(lib, d, N=320) == SHAPE
    assert fp8(lib, d, K=640) == SHAPE
    assert fp8(lib, cache_desc(dtype=0)) == DTYPE
    assert fp8(lib, d, ws=FAKE + 16) == MISAL
    assert fp8(lib, d, layer=5) == RANGE
    assert fp8(lib, d, ws_bytes=1000) == WS
    assert fp8(lib, d, M=0, ws_bytes=0) == OK
    assert fp8(lib, d) == DEV


def kv(lib, d, T=50, Kd=4096, layer=1, **ptrs):
    p = dict(h=FAKE, iro=FAKE, w=FAKE)
    p.update(ptrs)
    return lib.kv_matmul_paged(p["h"], p["iro"], T, Kd, p["w"], ctypes.byref(d), layer, None)


def test_kv_matmul_error_paths(lib):
    d = cache_desc(num_kv=2, heads=8, head_dim=128, with_lengths=True)
    for k in ("h", "iro", "w"):
        assert kv(lib, d, **{k: None}) == NULLP
    assert kv(lib, cache_desc(num_kv=2, heads=8, head_dim=128)) == NULLP   # no cache_lengths
    assert kv(lib, d, T=-3) == SHAPE
    assert kv(lib, d, Kd=100) == SHAPE
    assert kv(lib, cache_desc(num_kv=1, heads=8, head_dim=128, with_lengths=True)) == SHAPE
    assert kv(lib, cache_desc(num_kv=2, heads=1, head_dim=96, with_lengths=True)) == SHAPE
    assert kv(lib, cache_desc(dtype=0, num_kv=2, heads=8, head_dim=128, with_lengths=True)) == DTYPE
    assert kv(lib, d, h=FAKE + 4) == MISAL
    assert kv(lib, d, layer=2) == RANGE
    assert kv(lib, d, T=0) == OK
    assert kv(lib, d) == DEV


def test_gather_error_paths(lib):
    d = cache_desc()

    def gather(dd, M=100, layer=1, **ptrs):
        p = dict(bro=FAKE, co=FAKE, lat=FAKE)
        p.update(ptrs)
        return lib.mla_gather_latent_paged(p["bro"], p["co"], M, ctypes.byref(dd) if dd is not None else None,
                                           layer, p["lat"], None)
    assert gather(None) == NULLP
    for k in ("bro", "co", "lat"):
        assert gather(d, **{k: None}) == NULLP
    assert gather(d, M=-1) == SHAPE
    assert gather(cache_desc(num_kv=2)) == SHAPE
    assert gather(cache_desc(dtype=2)) == DTYPE
    assert gather(d, lat=FAKE + 8) == MISAL
    assert gather(d, layer=2) == RANGE
    assert gather(d, M=0, bro=None, co=None, lat=None) == OK
    assert gather(d) == DEV
    assert gather(cache_desc(dtype=0, head_dim=80, page_size=16)) == DEV


def test_latent_matmul_error_paths(lib):
    def mm(M=100, ld=576, N=512, K=512, dtype=1, **ptrs):
        p = dict(lat=FAKE, w=FAKE, out=FAKE)
        p.update(ptrs)
        return lib.mla_latent_matmul(p["lat"], ld, M, p["w"], N, K, dtype, p["out"], None)
    for k in ("lat", "w", "out"):
        assert mm(**{k: None}) == NULLP
    assert mm(M=-1) == SHAPE
    assert mm(ld=256) == SHAPE          # ld < K
    assert mm(ld=1 << 21) == SHAPE
    assert mm(K=96, ld=96) == SHAPE     # bf16 needs K % 64
    assert mm(N=100) == SHAPE
    assert mm(dtype=2) == DTYPE
    assert mm(ld=580) == MISAL          # 1160-byte rows
    assert mm(w=FAKE + 2) == MISAL
    assert mm(M=0, lat=None, w=None, out=None) == OK
    assert mm() == DEV
    assert mm(dtype=0, ld=80, N=128, K=64) == DEV


def test_check_indices_host_paths(lib):
    d = cache_desc(with_lengths=True)
    bad = ctypes.c_int64(7)
    assert lib.mla_check_indices(None, FAKE, 10, ctypes.byref(d), ctypes.byref(bad), None) == NULLP
    assert bad.value == -1
    no_len = cache_desc()
    assert lib.mla_check_indices(FAKE, None, 10, ctypes.byref(no_len), None, None) == NULLP
    assert lib.mla_check_indices(FAKE, FAKE, -1, ctypes.byref(d), None, None) == SHAPE
    assert lib.mla_check_indices(FAKE, FAKE, 10, ctypes.byref(d), None, None) == DEV


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mp, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(mp, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        mp.lib()


def decompress_kv(lib, d, M=100, Nk=512, Nv=512, K=512, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, wk=FAKE, wv=FAKE, lat=FAKE, kout=FAKE, vout=FAKE)
    p.update(ptrs)
    return lib.mla_decompress_kv_paged(p["bro"], p["co"], M, p["wk"], Nk, p["wv"], Nv, K,
                                       ctypes.byref(d) if d is not None else None, layer, p["lat"], p["kout"],
                                       p["vout"], None)


def test_decompress_kv_error_paths(lib):
    """The fused K and V call checks its second weight and output like the first,
    in the documented order (pointers, shapes, dtype, alignment, ranges)."""
    d = cache_desc()
    assert decompress_kv(lib, None) == NULLP
    for k in ("bro", "co", "wk", "wv", "lat", "kout", "vout"):
        assert decompress_kv(lib, d, **{k: None}) == NULLP
    assert decompress_kv(lib, d, wv=None, Nv=100) == NULLP          # pointers come before shapes
    assert decompress_kv(lib, d, Nv=0) == SHAPE
    assert decompress_kv(lib, d, Nv=100) == SHAPE                    # bf16 needs N_v % 64
    assert decompress_kv(lib, d, Nk=100) == SHAPE
    assert decompress_kv(lib, d, K=1024) == SHAPE
    assert decompress_kv(lib, cache_desc(dtype=2)) == DTYPE
    assert decompress_kv(lib, d, wv=FAKE + 8) == MISAL
    assert decompress_kv(lib, d, vout=FAKE + 4) == MISAL
    assert decompress_kv(lib, d, vout=FAKE + 4, Nv=100) == SHAPE     # shapes come before alignment
    assert decompress_kv(lib, d, layer=2) == RANGE
    assert decompress_kv(lib, d, M=0, bro=None, co=None, wk=None, wv=None, lat=None, kout=None, vout=None) == OK
    assert decompress_kv(lib, d) == DEV
    assert decompress_kv(lib, cache_desc(dtype=0, head_dim=80, page_size=16), Nk=128, Nv=68, K=64) == DEV


def fp8_kv(lib, d, M=100, Nk=512, Nv=512, K=512, grans=(1, 128, 128), ws=None, ws_bytes=None, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, wk=FAKE, sk=FAKE, wv=FAKE, sv=FAKE, lat=FAKE, kout=FAKE, vout=FAKE)
    p.update(ptrs)
    need = lib.mla_decompress_k_paged_fp8_workspace_size(max(M, 0), K, 128)
    return lib.mla_decompress_kv_paged_fp8(p["bro"], p["co"], M, p["wk"], p["sk"], Nk, p["wv"], p["sv"], Nv, K,
                                           *grans, ctypes.byref(d), layer, p["lat"], p["kout"], p["vout"],
                                           FAKE if ws is None else ws, need if ws_bytes is None else ws_bytes, None)


def test_decompress_kv_fp8_error_paths(lib):
    d = cache_desc()
    for k in ("bro", "co", "wk", "sk", "wv", "sv", "lat", "kout", "vout"):
        assert fp8_kv(lib, d, **{k: None}) == NULLP
    assert fp8_kv(lib, d, ws=0) == NULLP
    assert fp8_kv(lib, d, Nv=192) == SHAPE                           # N_v % 128
    assert fp8_kv(lib, d, grans=(1, 128, 64)) == SHAPE
    assert fp8_kv(lib, cache_desc(dtype=0, head_dim=576)) == DTYPE
    assert fp8_kv(lib, d, wv=FAKE + 8) == MISAL
    assert fp8_kv(lib, d, sv=FAKE + 2) == MISAL
    assert fp8_kv(lib, d, layer=5) == RANGE
    assert fp8_kv(lib, d, ws_bytes=1000) == WS
    assert fp8_kv(lib, d, M=0, ws_bytes=0) == OK
    assert fp8_kv(lib, d) == DEV


def write_latent(lib, d, T=50, K=512, max_seq=4096, eps=1e-6, layer=1, **ptrs):
    p = dict(x=FAKE, iro=FAKE, g=FAKE, f=FAKE)
    p.update(ptrs)
    return lib.mla_write_latent_paged(p["x"], p["iro"], T, p["g"], eps, p["f"], max_seq, K,
                                      ctypes.byref(d) if d is not None else None, layer, None)


def test_write_latent_error_paths(lib):
    d = cache_desc(with_lengths=True)
    assert write_latent(lib, None) == NULLP
    for k in ("x", "iro", "g", "f"):
        assert write_latent(lib, d, **{k: None}) == NULLP
    assert write_latent(lib, cache_desc()) == NULLP                   # no cache_lengths
    assert write_latent(lib, cache_desc(head_dim=512, with_lengths=True), f=None) == DEV   # no rope part: no freqs needed
    assert write_latent(lib, d, T=-1) == SHAPE
    assert write_latent(lib, d, K=500) == SHAPE                       # K % 8
    assert write_latent(lib, d, K=1024) == SHAPE                      # K > 512 and R < 0
    assert write_latent(lib, d, max_seq=0) == SHAPE
    assert write_latent(lib, d, eps=-1.0) == SHAPE
    assert write_latent(lib, cache_desc(num_kv=2, with_lengths=True)) == SHAPE
    assert write_latent(lib, cache_desc(dtype=0, with_lengths=True)) == DTYPE
    assert write_latent(lib, d, x=FAKE + 8) == MISAL
    assert write_latent(lib, d, g=FAKE + 4) == MISAL
    assert write_latent(lib, d, layer=2) == RANGE
    assert write_latent(lib, d, T=0, x=None, iro=None, g=None, f=None) == OK
    assert write_latent(lib, d) == DEV


def scales_desc(gran=128, nblk=5, page_size=128, layers=2):
    s = mp.ScalesDesc()
    s.scales = FAKE
    s.granularity = gran
    s.stride_token = nblk
    s.stride_kv = nblk * page_size
    s.stride_layer = s.stride_kv
    s.stride_page = s.stride_layer * layers
    return s


def fp8_cache(lib, d, s, M=100, N=512, K=512, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, w=FAKE, ws=FAKE, lat=FAKE, lsc=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.mla_decompress_k_paged_fp8_cache(p["bro"], p["co"], M, p["w"], p["ws"], N, K,
                                                ctypes.byref(d) if d is not None else None,
                                                ctypes.byref(s) if s is not None else None, layer,
                                                p["lat"], p["lsc"], p["out"], None)


def test_fp8_cache_error_paths(lib):
    d = cache_desc(dtype=2)
    s = scales_desc()
    assert fp8_cache(lib, None, s) == NULLP
    assert fp8_cache(lib, d, None) == NULLP
    for k in ("bro", "co", "w", "ws", "lat", "lsc", "out"):
        assert fp8_cache(lib, d, s, **{k: None}) == NULLP
    sn = scales_desc()
    sn.scales = None
    assert fp8_cache(lib, d, sn) == NULLP
    assert fp8_cache(lib, d, s, M=-1) == SHAPE
    assert fp8_cache(lib, d, s, N=500) == SHAPE                     # N % 128
    assert fp8_cache(lib, d, s, K=320) == SHAPE                     # K % 128
    assert fp8_cache(lib, d, s, K=640) == SHAPE                     # K > D_c
    assert fp8_cache(lib, d, scales_desc(gran=64)) == SHAPE         # only 128-column scale blocks
    assert fp8_cache(lib, d, scales_desc(nblk=4)) == SHAPE          # scale rows shorter than ceil(576/128)
    assert fp8_cache(lib, d, s, M=4_000_000) == SHAPE               # M * D_c >= 2^31
    assert fp8_cache(lib, cache_desc(dtype=2, num_kv=2), s) == SHAPE
    assert fp8_cache(lib, cache_desc(dtype=1), s) == DTYPE          # a bf16 pool has no scales
    assert fp8_cache(lib, d, s, w=FAKE + 8) == MISAL
    assert fp8_cache(lib, d, s, lat=FAKE + 8) == MISAL
    assert fp8_cache(lib, d, s, ws=FAKE + 2) == MISAL
    assert fp8_cache(lib, d, s, lsc=FAKE + 2) == MISAL
    assert fp8_cache(lib, cache_desc(dtype=2, head_dim=584), s) == MISAL   # 584-byte rows are not 16-byte granules
    assert fp8_cache(lib, d, s, layer=2) == RANGE
    assert fp8_cache(lib, d, s, M=0, bro=None, co=None, w=None, ws=None, lat=None, lsc=None, out=None) == OK
    assert fp8_cache(lib, d, s) == DEV


def absorb(lib, T=64, H=16, dn=128, dr=64, L=512, copy=1, **ptrs):
    p = dict(q=FAKE, w=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.mla_absorb_q(p["q"], T, H, dn, dr, p["w"], L, copy, p["out"], None)


def test_absorb_error_paths(lib):
    for k in ("q", "w", "out"):
        assert absorb(lib, **{k: None}) == NULLP
    assert absorb(lib, T=-1) == SHAPE
    assert absorb(lib, H=0) == SHAPE
    assert absorb(lib, dn=64) == SHAPE                 # only qk_nope_head_dim 128
    assert absorb(lib, dr=60) == SHAPE                 # rope columns in 16-byte pieces
    assert absorb(lib, L=500) == SHAPE                 # kv_latent_dim % 128
    assert absorb(lib, copy=2) == SHAPE
    assert absorb(lib, T=60000, H=128) == SHAPE        # query offsets past 2^31
    assert absorb(lib, q=FAKE + 8) == MISAL
    assert absorb(lib, w=FAKE + 8) == MISAL
    assert absorb(lib, out=FAKE + 2) == MISAL
    assert absorb(lib, T=0, q=None, w=None, out=None) == OK
    assert absorb(lib, dr=0, copy=0) == DEV
    assert absorb(lib) == DEV


def absorb_fp8(lib, T=64, H=16, dn=128, dr=64, L=512, grans=(1, 128, 128), copy=1, **ptrs):
    p = dict(q=FAKE, w=FAKE, ws=FAKE, out=FAKE)
    p.update(ptrs)
    return lib.mla_absorb_q_fp8(p["q"], T, H, dn, dr, p["w"], p["ws"], L, *grans, copy, p["out"], None)


def test_absorb_fp8_error_paths(lib):
    for k in ("q", "w", "ws", "out"):
        assert absorb_fp8(lib, **{k: None}) == NULLP
    assert absorb_fp8(lib, T=-1) == SHAPE
    assert absorb_fp8(lib, dn=256) == SHAPE
    assert absorb_fp8(lib, L=384 + 64) == SHAPE
    for g in ((2, 128, 128), (1, 64, 128), (1, 128, 64)):
        assert absorb_fp8(lib, grans=g) == SHAPE
    assert absorb_fp8(lib, copy=-1) == SHAPE
    assert absorb_fp8(lib, w=FAKE + 4) == MISAL
    assert absorb_fp8(lib, ws=FAKE + 1) == MISAL
    assert absorb_fp8(lib, T=0, q=None, w=None, ws=None, out=None) == OK
    assert absorb_fp8(lib) == DEV


def write_latent_fp8(lib, d, s, T=50, K=512, max_seq=4096, eps=1e-6, layer=1, **ptrs):
    p = dict(x=FAKE, iro=FAKE, g=FAKE, f=FAKE)
    p.update(ptrs)
    return lib.mla_write_latent_paged_fp8(p["x"], p["iro"], T, p["g"], eps, p["f"], max_seq, K,
                                          ctypes.byref(d) if d is not None else None,
                                          ctypes.byref(s) if s is not None else None, layer, None)


def test_write_latent_fp8_error_paths(lib):
    d = cache_desc(dtype=2, with_lengths=True)
    s = scales_desc()
    assert write_latent_fp8(lib, None, s) == NULLP
    assert write_latent_fp8(lib, d, None) == NULLP
    for k in ("x", "iro", "g", "f"):
        assert write_latent_fp8(lib, d, s, **{k: None}) == NULLP
    bad = scales_desc()
    bad.scales = None
    assert write_latent_fp8(lib, d, bad) == NULLP
    assert write_latent_fp8(lib, d, s, K=448) == SHAPE                # K % 128
    assert write_latent_fp8(lib, d, scales_desc(gran=64)) == SHAPE
    assert write_latent_fp8(lib, d, scales_desc(nblk=4)) == SHAPE     # stride_token < ceil(576 / 128)
    assert write_latent_fp8(lib, d, s, eps=-1.0) == SHAPE
    assert write_latent_fp8(lib, cache_desc(dtype=1, with_lengths=True), s) == DTYPE   # a bf16 cache
    assert write_latent_fp8(lib, d, s, x=FAKE + 8) == MISAL
    mis = scales_desc()
    mis.scales = FAKE + 2
    assert write_latent_fp8(lib, d, mis) == MISAL
    assert write_latent_fp8(lib, d, s, layer=2) == RANGE
    assert write_latent_fp8(lib, d, s, T=0, x=None, iro=None, g=None, f=None) == OK
    assert write_latent_fp8(lib, d, s) == DEV


def fp8_cache_kv(lib, d, s, M=100, Nk=512, Nv=256, K=512, layer=1, **ptrs):
    p = dict(bro=FAKE, co=FAKE, wk=FAKE, sk=FAKE, wv=FAKE, sv=FAKE, lat=FAKE, lsc=FAKE, kout=FAKE, vout=FAKE)
    p.update(ptrs)
    return lib.mla_decompress_kv_paged_fp8_cache(p["bro"], p["co"], M, p["wk"], p["sk"], Nk, p["wv"], p["sv"], Nv, K,
                                                 ctypes.byref(d) if d is not None else None,
                                                 ctypes.byref(s) if s is not None else None, layer,
                                                 p["lat"], p["lsc"], p["kout"], p["vout"], None)


def test_fp8_cache_kv_error_paths(lib):
    d = cache_desc(dtype=2)
    s = scales_desc()
    assert fp8_cache_kv(lib, None, s) == NULLP
    assert fp8_cache_kv(lib, d, None) == NULLP
    for k in ("bro", "co", "wk", "sk", "wv", "sv", "lat", "lsc", "kout", "vout"):
        assert fp8_cache_kv(lib, d, s, **{k: None}) == NULLP
    assert fp8_cache_kv(lib, d, s, Nv=192) == SHAPE                 # N_v % 128
    assert fp8_cache_kv(lib, d, s, Nv=0) == SHAPE
    assert fp8_cache_kv(lib, d, s, K=640) == SHAPE                  # K > D_c
    assert fp8_cache_kv(lib, cache_desc(dtype=1), s) == DTYPE
    assert fp8_cache_kv(lib, d, s, wv=FAKE + 8) == MISAL
    assert fp8_cache_kv(lib, d, s, vout=FAKE + 8) == MISAL
    assert fp8_cache_kv(lib, d, s, sv=FAKE + 2) == MISAL
    assert fp8_cache_kv(lib, d, s, layer=2) == RANGE
    assert fp8_cache_kv(lib, d, s, M=0) == OK
    assert fp8_cache_kv(lib, d, s) == DEV


def test_tile_offsets_that_overflow_32_bits_are_refused(lib):
    """The product kernels address a 256-row tile with 32-bit byte offsets, so a
    row of 2^22 bf16 elements (256 rows = 2^31 bytes) is refused before any
    launch, even where the weight itself (N x K) stays under 2^31 bytes."""
    big = 1 << 22
    d = cache_desc()
    assert decompress(lib, d, N=big, K=64) == SHAPE
    assert decompress(lib, d, N=big - 64, K=64) == DEV          # the largest accepted width
    assert fp8(lib, d, N=big, K=128) == SHAPE
    assert fp8(lib, d, N=big - 128, K=128) == DEV
    assert lib.mla_latent_matmul(FAKE, 576, 100, FAKE, big, 64, 1, FAKE, None) == SHAPE
    dk = cache_desc(num_kv=2, heads=1, head_dim=64, with_lengths=True)
    assert kv(lib, dk, Kd=big) == SHAPE
    assert kv(lib, dk, Kd=big - 64) == DEV
    wide = cache_desc(head_dim=big, page_size=1, pages=2, maxp=2)   # a cache row of 2^22 bf16
    assert decompress(lib, wide, N=512, K=512) == SHAPE


def test_noalloc_fp8_error_paths(lib):
    """The fp8 call without a workspace: the usual checks, and a call whose
    workspace would exceed the library's fixed array is refused."""
    d = cache_desc()

    def call(M=100, N=512, K=512, grans=(1, 128, 128), **ptrs):
        p = dict(bro=FAKE, co=FAKE, w=FAKE, sw=FAKE, lat=FAKE, out=FAKE)
        p.update(ptrs)
        return lib.mla_decompress_k_paged_fp8_noalloc(p["bro"], p["co"], M, p["w"], p["sw"], N, K, *grans,
                                                      ctypes.byref(d), 1, p["lat"], p["out"], None)
    limit = mp.MLA_FP8_NOALLOC_SCRATCH_BYTES
    assert lib.mla_decompress_k_paged_fp8_workspace_size(65536, 512, 128) == limit
    assert call(M=65536) == DEV                 # exactly fills the array
    assert call(M=65537) == WS                  # one row more does not fit
    for k in ("bro", "co", "w", "sw", "lat", "out"):
        assert call(**{k: None}) == NULLP
    assert call(grans=(1, 128, 64)) == SHAPE
    assert call(M=0, bro=None, co=None, w=None, sw=None, lat=None, out=None) == OK
    assert call() == DEV
