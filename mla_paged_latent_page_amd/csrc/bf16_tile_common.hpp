// Pieces shared by the persistent product kernels (decompress_bf16.hip,
// decompress_bf16_ring.hip, decompress_fp8_ring.hip): problem description, the per-block tile list with
// its XCD-aware order, the accumulator drain used by the epilogues, barrier
// helpers and the launch geometry.
#pragma once

#include "launch.hpp"

namespace mla {

struct GemmParams {
    const uint16_t* A;   // [M][lda] bf16 (gathered rows)
    const uint16_t* W;   // [N][K] bf16
    uint16_t* C;         // [M][N] bf16
    int lda;
    int M, N, K;
    int tiles_m, tiles_n;
    int xcd_map;
    // Second projection (fused K and V): N-tiles tiles_n1 .. tiles_n - 1 take
    // their weight rows from W2 [N2][K] and write C2 [M][N2].  tiles_n1 ==
    // tiles_n when there is none.
    const uint16_t* W2;
    uint16_t* C2;
    int N2, tiles_n1;
};

// The projection an N-tile belongs to: its weight, output, width and its
// tile index within that projection.
struct Segment {
    const uint16_t* W;
    uint16_t* C;
    int N, tn;
};
__device__ inline Segment segment_of(const GemmParams& P, int tn)
{
    if (tn < P.tiles_n1)
        return Segment{P.W, P.C, P.N, tn};
    return Segment{P.W2, P.C2, P.N2, tn - P.tiles_n1};
}

// The tiles of one persistent block, in the order it processes them.
// Blocks are dispatched to the 8 XCDs round-robin (block b runs on XCD b % 8).
// xcd_map 1 (weight-stationary): XCD x owns N-tiles [x*G, (x+1)*G) and walks
// the M-tiles, so its 1/8 of W stays in its own L2 while the activation rows
// stream past; the N-tiles of one M-tile, running side by side, share those
// rows in L2.  Suits activations that are re-read cheaply (the decompress
// rows, 1 KB each).
// xcd_map 2 (activation-stationary): XCD x owns M-tiles x, x+8, x+16, ... and
// runs all N-tiles of an M-tile side by side, so each activation tile is
// fetched from HBM once and the whole weight, small enough for the last-level
// cache, is re-read from there.  Suits long activation rows with few N-tiles
// (the kv projection: 8 KB rows, 8 N-tiles) and weights that fit in an XCD's
// L2 (a decompress weight of at most 2 MiB).
// xcd_map 3 (two projections, weight-stationary in two passes): XCD x walks the
// M-tiles over its eighth of the first projection's N-tiles, then over its
// eighth of the second's, so only one projection's eighth of the weight has to
// stay in its L2 at a time (both together would fill it).
// xcd_map 0: plain row-major order.
struct TileList {
    int first, step, count, Gn, x, tiles_n, mode;
    int G2, tiles_n1, pass1;   // xcd_map 3 only
    __device__ void coords(int i, int& tm, int& tn) const
    {
        const int u = first + i * step;
        if (mode == 1 || (mode == 3 && u < pass1)) {
            tm = u / Gn;
            tn = x * Gn + (u - tm * Gn);
        } else if (mode == 3) {
            const int v = u - pass1;
            tm = v / G2;
            tn = tiles_n1 + x * G2 + (v - tm * G2);
        } else if (mode == 2) {
            const int q = u / tiles_n;
            tm = x + 8 * q;
            tn = u - q * tiles_n;
        } else {
            tm = u / tiles_n;
            tn = u - tm * tiles_n;
        }
        tm = __builtin_amdgcn_readfirstlane(tm);
        tn = __builtin_amdgcn_readfirstlane(tn);
    }
};

// N-tiles of the first projection (all of them unless the block has two).
template <class PT>
__device__ inline int first_projection_tiles(const PT& P) { return P.tiles_n; }
__device__ inline int first_projection_tiles(const GemmParams& P) { return P.tiles_n1; }

// PT: any parameter block with tiles_m, tiles_n and xcd_map.
template <class PT>
__device__ inline TileList make_tiles(const PT& P)
{
    TileList L;
    L.tiles_n = P.tiles_n;
    L.mode = P.xcd_map;
    L.G2 = 0;
    L.tiles_n1 = first_projection_tiles(P);
    L.pass1 = 0;
    int total;
    if (L.mode == 3) {
        L.x = blockIdx.x & 7;
        L.first = blockIdx.x >> 3;
        L.step = gridDim.x >> 3;
        L.Gn = L.tiles_n1 >> 3;
        L.G2 = (P.tiles_n - L.tiles_n1) >> 3;
        L.pass1 = P.tiles_m * L.Gn;
        total = L.pass1 + P.tiles_m * L.G2;
    } else if (L.mode == 1) {
        L.x = blockIdx.x & 7;
        L.first = blockIdx.x >> 3;
        L.step = gridDim.x >> 3;
        L.Gn = P.tiles_n >> 3;
        total = P.tiles_m * L.Gn;
    } else if (L.mode == 2) {
        L.x = blockIdx.x & 7;
        L.first = blockIdx.x >> 3;
        L.step = gridDim.x >> 3;
        L.Gn = 1;
        total = (P.tiles_m > L.x ? (P.tiles_m - L.x + 7) / 8 : 0) * P.tiles_n;
    } else {
        L.x = 0;
        L.Gn = 1;
        L.first = blockIdx.x;
        L.step = gridDim.x;
        total = P.tiles_m * P.tiles_n;
    }
    L.count = L.first < total ? (total - L.first + L.step - 1) / L.step : 0;
    // Every field is wave-uniform; say so, so that the tile walk stays in
    // scalar registers and its branches stay scalar branches.
    L.first = __builtin_amdgcn_readfirstlane(L.first);
    L.step = __builtin_amdgcn_readfirstlane(L.step);
    L.count = __builtin_amdgcn_readfirstlane(L.count);
    L.Gn = __builtin_amdgcn_readfirstlane(L.Gn);
    L.x = __builtin_amdgcn_readfirstlane(L.x);
    L.G2 = __builtin_amdgcn_readfirstlane(L.G2);
    L.pass1 = __builtin_amdgcn_readfirstlane(L.pass1);
    return L;
}

// Order this wave's LDS writes before its later LDS reads (a wave's LDS
// operations are performed in order; this only stops compiler reordering).
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Read accumulator element E of a 32x32 block.  The volatile asm keeps the
// reads in program order with the LDS writes that consume them, so a tile is
// drained block by block instead of copying all 256 accumulators out at once.
template <int E>
__device__ inline float acc_read(const f32x16& a)
{
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(a[E]));
    return x;
}

// Accumulators 4Q..4Q+3 of a block (4 consecutive output columns) as bf16.
template <int Q>
__device__ inline u32x2 acc_pack4(const f32x16& a)
{
    u32x2 v;
    v[0] = pack_bf16x2(acc_read<4 * Q + 0>(a), acc_read<4 * Q + 1>(a));
    v[1] = pack_bf16x2(acc_read<4 * Q + 2>(a), acc_read<4 * Q + 3>(a));
    return v;
}

// Wait until at most N of this thread's vector-memory operations are in
// flight and its LDS operations are done, then meet at the block barrier.
template <int N>
__device__ inline void vm_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Launch geometry: one block per CU; with the XCD map every XCD gets the same
// number of blocks (surplus blocks find no tile and exit at once).
inline GemmParams make_gemm_params(const DecompressArgs& a, int BM, int BN, int cus)
{
    GemmParams P;
    P.A = static_cast<const uint16_t*>(a.lat);
    P.W = static_cast<const uint16_t*>(a.W);
    P.C = static_cast<uint16_t*>(a.out);
    P.lda = a.D;
    P.M = a.M;
    P.N = a.N;
    P.K = a.K;
    P.tiles_m = (a.M + BM - 1) / BM;
    P.tiles_n = (a.N + BN - 1) / BN;
    P.tiles_n1 = P.tiles_n;
    P.W2 = static_cast<const uint16_t*>(a.W2);
    P.C2 = static_cast<uint16_t*>(a.out2);
    P.N2 = a.N2;
    if (a.N2 > 0) {   // the first projection's width is then a multiple of BN
        P.tiles_n += (a.N2 + BN - 1) / BN;
        P.xcd_map = (P.tiles_n1 % 8 == 0 && (P.tiles_n - P.tiles_n1) % 8 == 0 && cus % 8 == 0) ? 3 : 0;
    } else if ((int64_t)a.N * a.K * 2 <= (int64_t(2) << 20) && cus % 8 == 0) {
        // The whole weight fits in half of one XCD's L2 (a tensor-parallel
        // share of the heads): each XCD owns whole M-tiles, so every activation
        // row is read from HBM once instead of once per XCD.
        P.xcd_map = 2;
    } else {
        P.xcd_map = (P.tiles_n % 8 == 0 && cus % 8 == 0) ? 1 : 0;
    }
    return P;
}

inline int gemm_grid(const GemmParams& P, int cus)
{
    const int tiles = P.tiles_m * P.tiles_n;
    if (P.xcd_map)
        return cus;
    return tiles < cus ? tiles : cus;
}

hipError_t launch_product_bf16_ring(const DecompressArgs& a, int cus, hipStream_t s);

}  // namespace mla
