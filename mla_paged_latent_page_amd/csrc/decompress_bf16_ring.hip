// LDS-ring variant of the persistent bf16 product (k_buffer = k_latent[:, :K] W^T;
// page "generic_flare_mla_decompress_k_cache_ragged_paged", summary, and page
// "mla_prefill_decode_graph_fp8", Args w_k), used when K is a multiple of 128.
//
//  * Same 256 x 256 tiles, epilogue, buffer resources and XCD-aware tile order
//    as the register-staged kernel in decompress_bf16.hip; 8 waves of 128 x 64
//    (128 accumulators, two waves per SIMD, so one wave's LDS and memory
//    stalls are covered by the other's MFMAs).
//  * K advances in 64-wide stages through two LDS slots of 64 KB (256 rows of
//    128 bytes for each operand).  Operand tiles go from memory straight into
//    LDS (buffer loads with an LDS destination, 16 bytes per lane, no VGPR
//    staging); the stream of stages runs straight across tile boundaries.
//  * Per stage, with its k step 0 fragments already in registers: k steps 0..2
//    run while the fragments of the step after each are read; then the block
//    meets (this thread's loads of the next stage have landed, and every wave
//    has read all of the current slot), the loads two stages ahead go into the
//    current slot, one per MFMA of k step 3, and the next stage's step-0
//    fragments are read under those MFMAs.  The matrix pipe has work as soon as
//    the barrier opens.
//  * The loads are issued from inline assembly, so the compiler adds no waits
//    of its own for them; the waits before the barrier are explicit.
//  * Rows of 128 bytes hold eight 16-byte granules XOR-swizzled by (row / 2) % 8:
//    a 1 KB load chunk covers 8 rows, and the MFMA operand reads of 16 lanes
//    (16 rows, one logical granule column) touch each of the 64 LDS banks once.
//  * K is a multiple of 128, so every tile spans an even number of stages and
//    the slot of each stage is known at compile time.
//  * Epilogue per wave through a private LDS strip of 32 rows x 64 columns:
//    bf16 pairs in, 16-byte row pieces out, non-temporal stores; after a tile
//    the first stage of the next one waits only for its loads, not the stores.
#include <type_traits>

#include "bf16_tile_common.hpp"

namespace mla {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NBUF = 2;
static_assert(BN == kRingTileN, "tile width the launchers assume");
constexpr int ROWB = BK * 2;                  // bytes per tile row in a stage
constexpr int CHUNK_ROWS = 1024 / ROWB;       // rows covered by one 1 KB load chunk
constexpr int A_BYTES = BM * ROWB, SLOT_BYTES = (BM + BN) * ROWB;
constexpr int EPI_ROWS = 32;

template <int WAVES_M, int WAVES_N>
struct RingCfg {
    static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int CA = BM / CHUNK_ROWS / NW, CB = BN / CHUNK_ROWS / NW;  // load chunks per wave
    static constexpr int LOADS = CA + CB;     // vector-memory operations per thread per stage
    static constexpr int EPI = EPI_ROWS * WTN;             // elements of one wave's epilogue strip
    static constexpr int EG = WTN / 8;                     // 16-byte granules per strip row
    static constexpr int EPI_PER_LANE = EPI_ROWS * EG / 64;
    static constexpr int STORES_PER_TILE = FM * EPI_PER_LANE;  // buffer stores per thread per tile
    static_assert(NBUF * SLOT_BYTES + NW * EPI * 2 <= 163840, "LDS budget");
    static_assert(CA * NW * CHUNK_ROWS == BM && CB * NW * CHUNK_ROWS == BN, "loader shape");
    static_assert(LOADS + STORES_PER_TILE <= 63, "vmcnt range");
    static_assert(CA % 2 == 0 && CB % 2 == 0, "chunks alternate between the two swizzle phases");
};

// Scheduling pattern for one k step of NMF MFMAs: one LDS read after each of
// the first NDS MFMAs and one memory load after each of the NVM MFMAs that
// follow them (or alongside them when there are not enough MFMAs).  Spreading
// the memory instructions over the MFMAs keeps the waves, released together by
// the barrier, from flooding the LDS and address queues while the matrix pipe
// idles.
template <int NMF, int NDS, int NVM>
__device__ inline void interleave()
{
    constexpr bool split = NDS + NVM <= NMF;
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        if (i < NDS)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        if (split ? (i >= NDS && i < NDS + NVM) : (i < NVM))
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
}

// Where the loader of the next stages stands.
struct LoadCursor {
    int tile, ks;
    i32x4 ar, wr;   // operand tiles, as resources for the inline-assembly loads
};

template <int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1) gemm_bf16_ring(GemmParams P)
{
    using C = RingCfg<WAVES_M, WAVES_N>;
    constexpr int WTM = C::WTM, WTN = C::WTN, FM = C::FM, FN = C::FN, CA = C::CA, CB = C::CB;
    constexpr int EPI = C::EPI, EG = C::EG, EPI_PER_LANE = C::EPI_PER_LANE;
    constexpr int LOADS = C::LOADS, STORES_PER_TILE = C::STORES_PER_TILE;
    __shared__ __attribute__((aligned(1024))) char slot0[SLOT_BYTES];
    __shared__ __attribute__((aligned(1024))) char slot1[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) uint16_t strips[C::NW * EPI];
    auto slot = [&](auto b) __attribute__((always_inline)) -> char* {
        constexpr int i = decltype(b)::value;
        if constexpr (i == 0) return slot0;
        else return slot1;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived offsets in SGPRs
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const TileList tl = make_tiles(P);
    const int KT = P.K / BK;
    if (tl.count == 0)
        return;

    // Loader lane offsets: in a 1 KB chunk (8 rows of 128 bytes) lane l fills
    // row l/8 at granule position l%8, i.e. logical granule (l%8) ^ ((row/2)%8)
    // of that row.  Chunk c starts at row 8c, so (row/2)%8 has 4 added in odd
    // chunks: two lane offsets, for even and odd chunks.
    const int lrow = lane >> 3;
    const int lg_even = (lane & 7) ^ ((lrow >> 1) & 7), lg_odd = (lane & 7) ^ (((lrow >> 1) + 4) & 7);
    const uint32_t a_lane[2] = {(uint32_t)(lrow * P.lda * 2 + lg_even * 16), (uint32_t)(lrow * P.lda * 2 + lg_odd * 16)};
    const uint32_t w_lane[2] = {(uint32_t)(lrow * P.K * 2 + lg_even * 16), (uint32_t)(lrow * P.K * 2 + lg_odd * 16)};
    const uint32_t a_chunk = (uint32_t)(CHUNK_ROWS * P.lda * 2), w_chunk = (uint32_t)(CHUNK_ROWS * P.K * 2);

    auto cursor_at = [&](int tile, LoadCursor& c) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const Segment sg = segment_of(P, tn);
        const int mrows = min(P.M - tm * BM, BM), nrows = min(sg.N - sg.tn * BN, BN);
        c.tile = tile;
        c.ks = 0;
        c.ar = make_srd(P.A + (int64_t)tm * BM * P.lda, (uint32_t)(mrows * P.lda * 2));
        c.wr = make_srd(sg.W + (int64_t)sg.tn * BN * P.K, (uint32_t)(nrows * P.K * 2));
    };
    // Load q (of LOADS) of the cursor's stage into ring slot b.  The loads are
    // issued from inline assembly, so the compiler adds no waits of its own for
    // them; every wait is explicit.  Past the last tile the last stage is
    // loaded again (never read).
    auto load_one = [&](auto b, const LoadCursor& c, int q) __attribute__((always_inline)) {
        const uint32_t s = lds_addr(slot(b));
        const uint32_t kb = c.ks * BK * 2;
        if (q < CA) {
            const int ch = wave * CA + q;
            asm_ld16_lds(c.ar, s + ch * 1024, a_lane[q & 1], ch * a_chunk + kb);
        } else {
            const int ch = wave * CB + (q - CA);
            asm_ld16_lds(c.wr, s + A_BYTES + ch * 1024, w_lane[(q - CA) & 1], ch * w_chunk + kb);
        }
    };
    auto issue = [&](auto b, LoadCursor& c) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            load_one(b, c, q);
        ++c.ks;
    };
    // Move a cursor that ran off its tile to the next tile (kept out of the
    // stage's MFMA block so the loads can interleave with the MFMAs).
    auto settle = [&](LoadCursor& c) __attribute__((always_inline)) {
        if (c.ks == KT) {
            if (c.tile + 1 < tl.count)
                cursor_at(c.tile + 1, c);
            else
                c.ks = KT - 1;
        }
    };

    f32x16 acc[FN][FM];

    // Fragment byte offsets (lane part) for the four 16-wide k steps of a stage.
    const int frow = lane & 31;
    int fr_off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        fr_off[kk] = frow * ROWB + ((2 * kk + (lane >> 5)) ^ ((frow >> 1) & 7)) * 16;

    bf16x8 fa0[FN], fb0[FM], fa1[FN], fb1[FM];
    auto load_frags = [&](auto b, int kk, bf16x8 (&fa)[FN], bf16x8 (&fb)[FM]) {
        const char* s = slot(b);
        const char* as = s + wm * WTM * ROWB + fr_off[kk];
        const char* bs = s + A_BYTES + wn * WTN * ROWB + fr_off[kk];
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fa[i] = as_bf16x8(lds_ld16(bs + i * 32 * ROWB));
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fb[j] = as_bf16x8(lds_ld16(as + j * 32 * ROWB));
    };
    auto mfmas = [&](const bf16x8 (&fa)[FN], const bf16x8 (&fb)[FM], auto first) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                if constexpr (decltype(first)::value)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], f32x16{}, 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
    };

    // Write the finished tile through this wave's strip.
    auto epilogue = [&](int tile) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const int mrows = min(P.M - tm * BM, BM);
        const Segment sg = segment_of(P, tn);
        const rsrc_t cr = make_rsrc(sg.C + (int64_t)tm * BM * sg.N, (uint32_t)(mrows * sg.N * 2));
        uint16_t* E = strips + wave * EPI;
        const int ncol0 = sg.tn * BN + wn * WTN;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const int row = lane & 31;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int col = i * 32 + 4 * (lane >> 5);
                uint16_t* e = E + row * WTN + (col & 7);
                lds_st8(e + swz(row, (col >> 3) + 0, EG) * 8, acc_pack4<0>(acc[i][j]));
                lds_st8(e + swz(row, (col >> 3) + 1, EG) * 8, acc_pack4<1>(acc[i][j]));
                lds_st8(e + swz(row, (col >> 3) + 2, EG) * 8, acc_pack4<2>(acc[i][j]));
                lds_st8(e + swz(row, (col >> 3) + 3, EG) * 8, acc_pack4<3>(acc[i][j]));
            }
            wave_lds_sync();
            u32x4 v[EPI_PER_LANE];
#pragma unroll
            for (int p = 0; p < EPI_PER_LANE; ++p) {
                const int idx = p * 64 + lane;
                const int r = idx / EG, g = idx % EG;
                v[p] = lds_ld16(E + r * WTN + swz(r, g, EG) * 8);
            }
            wave_lds_sync();
#pragma unroll
            for (int p = 0; p < EPI_PER_LANE; ++p) {
                const int idx = p * 64 + lane;
                const int r = idx / EG, g = idx % EG;
                const int n = ncol0 + g * 8;
                const uint32_t off = n < sg.N ? (uint32_t)(((wm * WTM + j * 32 + r) * sg.N + n) * 2) : kOutOfRange;
                buf_st16_nt(cr, v[p], off, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using first_t = std::integral_constant<bool, true>;
    using rest_t = std::integral_constant<bool, false>;

    // Prologue: stage 0 landed and visible, stage 1 in flight, stage 0's first
    // fragments read.
    LoadCursor lc;
    cursor_at(0, lc);
    issue(I0{}, lc);
    settle(lc);
    vm_barrier<0>();
    issue(I1{}, lc);
    settle(lc);
    load_frags(I0{}, 0, fa0, fb0);

    // One stage in slot B, its k step 0 fragments already in registers.  Steps
    // 0..2 run while the fragments of the step after each are read; then the
    // block meets: this thread's loads of the next stage have landed (after the
    // first stage of a tile other than the first, the previous tile's stores
    // are queued behind them and may stay in flight: `relaxed`), so the next
    // stage is complete in LDS, and every wave has read all of slot B.  The
    // loads two stages ahead go into slot B, the next stage's step-0 fragments
    // are read, and step 3's MFMAs cover that read: the matrix pipe has work
    // as soon as the barrier opens.
    auto stage = [&](auto b, auto first, auto relaxed) __attribute__((always_inline)) {
        constexpr int B = decltype(b)::value;
        using Bn = std::integral_constant<int, (B + 1) % NBUF>;
        load_frags(b, 1, fa1, fb1);
        mfmas(fa0, fb0, first);
        interleave<FN * FM, FN + FM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(b, 2, fa0, fb0);
        mfmas(fa1, fb1, rest_t{});
        interleave<FN * FM, FN + FM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(b, 3, fa1, fb1);
        mfmas(fa0, fb0, rest_t{});
        interleave<FN * FM, FN + FM, 0>();
        __builtin_amdgcn_sched_barrier(0);
        static_assert(LOADS <= FN * FM, "one load per step-3 MFMA");
        if constexpr (decltype(relaxed)::value)
            vm_barrier<STORES_PER_TILE>();
        else
            vm_barrier<0>();
        load_frags(Bn{}, 0, fa0, fb0);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1[j], acc[i][j], 0, 0, 0);
                const int q = i * FM + j;
                if (q < LOADS)
                    load_one(b, lc, q);
            }
        ++lc.ks;
        __builtin_amdgcn_sched_barrier(0);
        settle(lc);
    };
    using yes_t = std::integral_constant<bool, true>;
    using no_t = std::integral_constant<bool, false>;
    // K is a multiple of 128: a tile is an even number of 64-wide stages.
    for (int tile = 0; tile < tl.count; ++tile) {
        if (tile == 0)
            stage(I0{}, first_t{}, no_t{});
        else
            stage(I0{}, first_t{}, yes_t{});
        stage(I1{}, rest_t{}, no_t{});
        for (int ks = 2; ks < KT; ks += 2) {
            stage(I0{}, rest_t{}, no_t{});
            stage(I1{}, rest_t{}, no_t{});
        }
        epilogue(tile);
    }
    // The last stage's spare loads may still be landing in LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

hipError_t launch_product_bf16_ring(const DecompressArgs& a, int cus, hipStream_t s)
{
    GemmParams P = make_gemm_params(a, BM, BN, cus);
    log_launch("gemm_bf16_ring<2,4>", gemm_grid(P, cus), 512, "M=%d N=%d N2=%d K=%d tiles=%dx%d xcd_map=%d", P.M, P.N,
               P.N2, P.K, P.tiles_m, P.tiles_n, P.xcd_map);
    hipLaunchKernelGGL((gemm_bf16_ring<2, 4>), dim3(gemm_grid(P, cus)), dim3(512), 0, s, P);
    return hipGetLastError();
}

}  // namespace mla
