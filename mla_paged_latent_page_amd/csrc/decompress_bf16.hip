// Fused paged gather + bf16 up-projection for gfx950.
//
// Computes, for the rows of one batch (page "generic_flare_mla_decompress_k_cache_ragged_paged",
// summary; weight layout from page "mla_prefill_decode_graph_fp8", Args w_k):
//   k_latent[r][0:D] = cache row of request b at position cache_offsets[b] + (r - row_offsets[b])
//   k_buffer[r][n]   = sum_{k<K} k_latent[r][k] * W[n][k]      (fp32 accumulate, bf16 RNE out)
//
// Design (one block per BM x BN output tile):
//  * The block first resolves its BM rows to byte offsets in the pool (request
//    search over the ragged offsets, then page table) and keeps them in LDS; the
//    A-tile loads then read the paged rows directly -- the gather is fused into
//    the operand loads and the gathered rows are never re-read from HBM.
//  * One block per M-tile also writes the gathered rows (all D columns, rope
//    included) to k_latent as a by-product of its A loads.
//  * K is walked in stages of 64 through two LDS buffers; every 16-byte granule
//    is XOR-swizzled by row so operand reads are free of bank conflicts.
//  * v_mfma_f32_32x32x16_bf16 with the weight as the row operand: each lane's
//    accumulators then hold 4 consecutive output columns of one row, which pack
//    into 8-byte LDS writes; the tile is re-read row-contiguously and written with
//    16-byte non-temporal stores (the output is written once and never re-read).
//  * XCD-aware tile order (see tile_of_block).
#include "launch.hpp"

namespace mla {
namespace {

template <int BM, int BN, int WM, int WN>
struct Bf16Tile {
    static constexpr int BK = 64;
    static constexpr int GPR = BK / 8;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int RP = NT / GPR;
    static constexpr int AR = BM / RP;
    static constexpr int BR = BN / RP;
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int FM = TM / 32;
    static constexpr int FN = TN / 32;
    static constexpr int A_STAGE = BM * BK;   // elements
    static constexpr int B_STAGE = BN * BK;
    static constexpr int MAIN_LDS = 2 * (A_STAGE + B_STAGE) * 2;
    static constexpr int EPI_LDS = BM * BN * 2;
    static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
    static constexpr int CG = BN / 8;         // 16-byte granules per output tile row
    static_assert(NT % GPR == 0 && BM % RP == 0 && BN % RP == 0, "loader shape");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
    static_assert((CG & (CG - 1)) == 0, "output tile width");
};

struct Bf16Params {
    DecompressArgs a;
    int tiles_m, tiles_n;
    int xcd_map;
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
decompress_bf16_kernel(Bf16Params P)
{
    using T = Bf16Tile<BM, BN, WM, WN>;
    constexpr int BK = T::BK, GPR = T::GPR, NT = T::NT, RP = T::RP;
    __shared__ __attribute__((aligned(16))) char smem[T::LDS + BM * 8];
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);
    uint16_t* Bs = As + 2 * T::A_STAGE;
    int64_t* rowoff = reinterpret_cast<int64_t*>(smem + T::LDS);

    const DecompressArgs& a = P.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of_block(blockIdx.x, P.tiles_m, P.tiles_n, P.xcd_map, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool write_latent = (tn == tm % P.tiles_n);
    const uint16_t* W = static_cast<const uint16_t*>(a.W);
    uint16_t* lat = static_cast<uint16_t*>(a.lat);
    uint16_t* out = static_cast<uint16_t*>(a.out);

    // Resolve the tile's rows to pool byte offsets (-1: row past M).
    for (int r = tid; r < BM; r += NT) {
        const int m = m0 + r;
        int64_t off = -1;
        if (m < a.M) {
            const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)m);
            const uint32_t p = a.co[b] + ((uint32_t)m - a.bro[b]);
            off = token_offset(a.L, b, p);
        }
        rowoff[r] = off;
    }
    __syncthreads();

    const int gcol = tid % GPR, rsub = tid / GPR;
    const char* arow[T::AR];
    bool avalid[T::AR];
#pragma unroll
    for (int j = 0; j < T::AR; ++j) {
        const int64_t off = rowoff[rsub + j * RP];
        avalid[j] = off >= 0;
        arow[j] = a.L.base + (off >= 0 ? off : 0) + gcol * 16;
    }
    uint32_t boff[T::BR];
#pragma unroll
    for (int j = 0; j < T::BR; ++j) {
        int n = n0 + rsub + j * RP;
        n = n < a.N ? n : a.N - 1;
        boff[j] = (uint32_t)(((int64_t)n * a.K + gcol * 8) * 2);
    }
    const char* wbase = reinterpret_cast<const char*>(W);

    u32x4 ra[T::AR], rb[T::BR];
    auto gload = [&](int kt) {
        const int kb = kt * BK * 2;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) ra[j] = ld16(arow[j] + kb);
#pragma unroll
        for (int j = 0; j < T::BR; ++j) rb[j] = ld16(wbase + boff[j] + kb);
    };
    auto lstore = [&](int buf) {
        uint16_t* as = As + buf * T::A_STAGE;
        uint16_t* bs = Bs + buf * T::B_STAGE;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) {
            const int r = rsub + j * RP;
            lds_st16(as + r * BK + swz(r, gcol, GPR) * 8, ra[j]);
        }
#pragma unroll
        for (int j = 0; j < T::BR; ++j) {
            const int r = rsub + j * RP;
            lds_st16(bs + r * BK + swz(r, gcol, GPR) * 8, rb[j]);
        }
    };
    auto latent_store = [&](int kt) {
#pragma unroll
        for (int j = 0; j < T::AR; ++j)
            if (avalid[j])
                st16(lat + (int64_t)(m0 + rsub + j * RP) * a.D + kt * BK + gcol * 8, ra[j]);
    };

    f32x16 acc[T::FN][T::FM];
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
            acc[i][j] = f32x16{};

    const int KT = a.K / BK;
    gload(0);
    if (write_latent) latent_store(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint16_t* as = As + buf * T::A_STAGE;
        const uint16_t* bs = Bs + buf * T::B_STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int g = 2 * ks + (lane >> 5);
            bf16x8 fa[T::FN], fb[T::FM];
#pragma unroll
            for (int i = 0; i < T::FN; ++i) {
                const int n = wn * T::TN + i * 32 + (lane & 31);
                fa[i] = as_bf16x8(lds_ld16(bs + n * BK + swz(n, g, GPR) * 8));
            }
#pragma unroll
            for (int j = 0; j < T::FM; ++j) {
                const int m = wm * T::TM + j * 32 + (lane & 31);
                fb[j] = as_bf16x8(lds_ld16(as + m * BK + swz(m, g, GPR) * 8));
            }
#pragma unroll
            for (int i = 0; i < T::FN; ++i)
#pragma unroll
                for (int j = 0; j < T::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) {
            if (write_latent) latent_store(kt + 1);
            lstore(buf ^ 1);
        }
        __syncthreads();
    }

    // Rope (and any other) columns past K complete the gathered rows.
    if (write_latent && a.D > a.K) {
        const int rg = (a.D - a.K) / 8;
        for (int idx = tid; idx < BM * rg; idx += NT) {
            const int r = idx / rg, g = idx - r * rg;
            const int64_t off = rowoff[r];
            if (off >= 0)
                st16(lat + (int64_t)(m0 + r) * a.D + a.K + g * 8,
                     ld16(a.L.base + off + (int64_t)(a.K + g * 8) * 2));
        }
    }

    // Epilogue: accumulators (rows n, columns m of the MFMA result) -> bf16 ->
    // LDS tile [BM][BN] with swizzled granules -> row-contiguous global stores.
    uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);
    constexpr int CG = T::CG;
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wm * T::TM + j * 32 + (lane & 31);
                const int n = wn * T::TN + i * 32 + 8 * q + 4 * (lane >> 5);
                u32x2 v;
                v[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                v[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                lds_st8(Cs + m * BN + swz(m, n >> 3, CG) * 8 + (n & 7), v);
            }
    __syncthreads();
    for (int idx = tid; idx < BM * CG; idx += NT) {
        const int r = idx / CG, g = idx - r * CG;
        const int m = m0 + r, n = n0 + g * 8;
        const u32x4 v = lds_ld16(Cs + r * BN + swz(r, g, CG) * 8);
        if (m < a.M && n < a.N)
            st16_nt(out + (int64_t)m * a.N + n, v);
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const DecompressArgs& a, hipStream_t s)
{
    Bf16Params P;
    P.a = a;
    P.tiles_m = (a.M + BM - 1) / BM;
    P.tiles_n = (a.N + BN - 1) / BN;
    P.xcd_map = (P.tiles_n % 8 == 0) ? 1 : 0;
    const int grid = P.tiles_m * P.tiles_n;
    hipLaunchKernelGGL((decompress_bf16_kernel<BM, BN, WM, WN>), dim3(grid), dim3(64 * WM * WN), 0, s, P);
    return hipGetLastError();
}

}  // namespace

// Tile configurations (BM x BN, waves WM x WN).  MLA_PAGED_BF16_TILE picks one
// explicitly (for tuning); the default is the fastest measured on MI355X.
hipError_t launch_decompress_bf16(const DecompressArgs& a, hipStream_t s)
{
    static const int cfg = [] {
        const char* e = getenv("MLA_PAGED_BF16_TILE");
        return e ? atoi(e) : 0;
    }();
    switch (cfg) {
    case 1: return launch_cfg<256, 256, 2, 4>(a, s);
    case 2: return launch_cfg<256, 128, 2, 2>(a, s);
    case 3: return launch_cfg<128, 256, 2, 2>(a, s);
    case 4: return launch_cfg<128, 128, 2, 2>(a, s);
    default: return launch_cfg<256, 256, 2, 2>(a, s);
    }
}

}  // namespace mla
