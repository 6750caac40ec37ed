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

// Round-to-nearest-even float -> bf16 of two values, packed low/high.
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = static_cast<__bf16>(lo);
    __bf16 b = static_cast<__bf16>(hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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

// Swizzled position of 16-byte granule g in a tile row with `gpr` granules
// (a power of two): XOR with the row index spreads the rows that one MFMA
// operand read touches over all LDS banks.
__device__ inline int swz(int row, int g, int gpr) { return g ^ (row & (gpr - 1)); }

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
