// Device-side helpers shared by the gfx950 kernels of the paged MLA library:
// vector types, paged-cache addressing, LDS swizzles and bf16/fp8 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One layer of a paged pool, in bytes.  Token position p of request b is in
// page page_table[b * max_pages + p / page_size], slot p % page_size.
struct PagedLayer {
    const char* base;        // pool base + layer * stride_layer (bytes)
    const uint32_t* page_table;
    int64_t stride_page;     // bytes
    int64_t stride_token;    // bytes
    int64_t stride_kv;       // bytes
    uint32_t num_pages;
    uint32_t page_size;
    uint32_t max_pages;
    uint32_t batch;
};

// Request b holding ragged row r: the largest b < batch with offsets[b] <= r.
// Requires offsets[0] <= r; empty requests (equal neighbouring offsets) are
// skipped because the largest qualifying index is taken.
__device__ inline uint32_t find_request(const uint32_t* __restrict__ offsets, uint32_t batch, uint32_t r)
{
    uint32_t lo = 0, hi = batch;
    while (hi - lo > 1) {
        uint32_t mid = (lo + hi) >> 1;
        if (offsets[mid] <= r)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Byte offset of token position p of request b inside the layer.  The logical
// page and the page id are clamped to the table and the pool, so a bad index
// reads a wrong row of the pool, never memory outside it.
__device__ inline int64_t token_offset(const PagedLayer& L, uint32_t b, uint32_t p)
{
    uint32_t lp = p / L.page_size;
    uint32_t slot = p - lp * L.page_size;
    lp = lp < L.max_pages ? lp : L.max_pages - 1;
    uint32_t pg = L.page_table[(size_t)b * L.max_pages + lp];
    pg = pg < L.num_pages ? pg : L.num_pages - 1;
    return (int64_t)pg * L.stride_page + (int64_t)slot * L.stride_token;
}

// Byte offset of the slot a write path stores token position p of request b
// into, or -1 when the position lies past the request's page table or its page
// id past the pool: the store is then skipped (clamping, as the read paths do,
// would overwrite another token's cached row).
__device__ inline int64_t store_offset(const PagedLayer& L, uint32_t b, uint32_t p)
{
    const uint32_t lp = p / L.page_size;
    if (lp >= L.max_pages)
        return -1;
    const uint32_t pg = L.page_table[(size_t)b * L.max_pages + lp];
    if (pg >= L.num_pages)
        return -1;
    return (int64_t)pg * L.stride_page + (int64_t)(p - lp * L.page_size) * L.stride_token;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bf16 of two values, packed low/high (one
// v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Wait for this wave's LDS operations, then meet the other waves of the block.
// Unlike __syncthreads() this carries no memory fence for global memory, so
// global loads and stores in flight stay in flight.
__device__ inline void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> two OCP e4m3fn codes (round to nearest even) in the low 16 bits.
__device__ inline uint32_t pack_e4m3x2(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ inline void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }

__device__ inline u32x4 lds_ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void lds_st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ inline void lds_st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer access.  A resource covers [base, base + bytes); a 16-byte access
// at or past the end reads zeros / writes nothing, which handles ragged tile
// edges without branches.  Offsets are 32-bit: a per-lane part (VGPR) plus a
// wave-uniform part (SGPR).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every resource we build

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}
__device__ inline u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
// 16 bytes per lane straight from memory into LDS: lane l's bytes land at
// lds + 16 * l (lds is wave-uniform).  No VGPRs are involved.
__device__ inline void buf_ld16_lds(rsrc_t r, void* lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff,
                                             (int)soff, 0, 0);
}

// The same buffer resource as four SGPR words, for inline assembly: base,
// stride 0, num_records = bytes, raw 32-bit format.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 make_srd(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = kRsrcFlags;
    return r;
}
// LDS address (byte offset in the workgroup's LDS) of a __shared__ location.
__device__ inline uint32_t lds_addr(const void* p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// 16 bytes per lane from memory into LDS at lds + 16 * lane, issued from inline
// assembly: the compiler does not know this instruction writes LDS, so it adds
// no waits of its own for it.  The caller orders it against LDS reads with
// explicit s_waitcnt vmcnt and barriers.
__device__ inline void asm_ld16_lds(i32x4 srd, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

// 4 bytes per lane from memory into LDS at lds + 4 * lane (same rules as above).
__device__ inline void asm_ld4_lds(i32x4 srd, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(srd), "s"(soff)
                 : "memory", "m0");
}

// 16 bytes per lane from a per-lane 64-bit address into LDS at lds + 16 * lane,
// from inline assembly (same rules as asm_ld16_lds).
__device__ inline void asm_gld16_lds(const void* src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "memory", "m0");
}

// Non-temporal store: output rows are written once and not read back.
__device__ inline void buf_st16_nt(rsrc_t r, u32x4 v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, 2);
}

// Swizzled position of 16-byte granule g in a tile row with `gpr` granules
// (a power of two): XOR with the row index spreads the rows that one MFMA
// operand read touches over all LDS banks.
__device__ inline int swz(int row, int g, int gpr) { return g ^ (row & (gpr - 1)); }

// Maximum of v over each group of 16 lanes (lanes 16 k .. 16 k + 15), by DPP
// moves inside the 16-lane rows: quad lanes xor 1, xor 2, then the other
// quad of the half row (half-row mirror), then the other half (row mirror).
// Plain VALU work, where shuffles through LDS (ds_bpermute) would each wait
// an LDS round trip.  A maximum is exact in any order.
template <int CTRL>
__device__ inline float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ inline float max16(float v)
{
    v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));   // row_mirror
    return v;
}
// The value lane p (0..15, a constant once unrolled) of this lane's 16-lane
// row holds (DPP row_newbcast).
__device__ inline float row16_lane(float v, int p)
{
    switch (p & 15) {
    case 0: return dpp_f32<0x150>(v);
    case 1: return dpp_f32<0x151>(v);
    case 2: return dpp_f32<0x152>(v);
    case 3: return dpp_f32<0x153>(v);
    case 4: return dpp_f32<0x154>(v);
    case 5: return dpp_f32<0x155>(v);
    case 6: return dpp_f32<0x156>(v);
    case 7: return dpp_f32<0x157>(v);
    case 8: return dpp_f32<0x158>(v);
    case 9: return dpp_f32<0x159>(v);
    case 10: return dpp_f32<0x15A>(v);
    case 11: return dpp_f32<0x15B>(v);
    case 12: return dpp_f32<0x15C>(v);
    case 13: return dpp_f32<0x15D>(v);
    case 14: return dpp_f32<0x15E>(v);
    default: return dpp_f32<0x15F>(v);
    }
}

// Tile-to-block map.  Blocks are dispatched to the 8 XCDs round-robin
// (block i runs on XCD i % 8).  When the N tiles split evenly over the XCDs,
// XCD x takes N-tiles [x*G, (x+1)*G) for every M-tile, so its slice of the
// weight stays in its own L2 while the activation rows stream past; within
// an XCD the G N-tiles of one M-tile run next to each other and share the
// activation tile in L2.
__device__ inline void tile_of_block(int bid, int tiles_m, int tiles_n, bool xcd_map, int& tm, int& tn)
{
    if (xcd_map) {
        int xcd = bid & 7, j = bid >> 3;
        int G = tiles_n >> 3;
        tn = xcd * G + j % G;
        tm = j / G;
    } else {
        tn = bid % tiles_n;
        tm = bid / tiles_n;
    }
    (void)tiles_m;
}

}  // namespace mla
