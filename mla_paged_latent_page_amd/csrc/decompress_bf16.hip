// bf16 up-projection of gathered latent rows for gfx950 (page
// "generic_flare_mla_decompress_k_cache_ragged_paged", summary: the gathered rows are
// multiplied by the weight; weight layout [num_heads*qk_nope_head_dim, kv_latent_dim]
// from page "mla_prefill_decode_graph_fp8", Args w_k):
//   k_buffer[r][n] = sum_{k<K} k_latent[r][k] * W[n][k]   (fp32 accumulate, bf16 RNE out)
//
// Up to 256 rows (decode-sized calls) take the single fused kernel of
// decompress_small.hip.  Otherwise the call runs the paged gather (gather.hip)
// into k_latent_buffer, then a persistent product kernel over k_latent_buffer:
// the LDS-ring kernel of decompress_bf16_ring.hip when K is a multiple of 128,
// else the register-staged kernel below.
//
// Design of the register-staged product (one block of 4 waves per CU,
// persistent over tiles):
//  * 256 x 256 output tiles, each wave 128 x 128 with its 16 32x32 accumulators
//    (256 fp32 per lane) held in AGPRs; v_mfma_f32_32x32x16_bf16 with the weight
//    as the row operand, so a lane's accumulators hold 4 consecutive output
//    columns of one row.
//  * K advances in 64-wide stages through two LDS buffers (2 x 64 KB).  Within
//    a stage the four 16-wide k steps are software-pipelined: the operand
//    fragments of step kk+1 are read while step kk's 16 MFMAs run; the next
//    stage goes from registers into the other LDS buffer during step 1, the
//    stage after it is fetched from memory during step 2, and the single block
//    barrier sits before step 3, whose MFMAs cover the first fragment reads of
//    the next stage.  The stage sequence runs straight across tile boundaries.
//  * Global traffic uses buffer resources built per tile in SGPRs: each lane
//    keeps one fixed 32-bit offset, the uniform parts ride in SGPRs, and rows
//    past M (or columns past N) fall outside the resource, so partial tiles
//    need no clamping or branches (reads return zeros, writes are dropped).
//  * 16-byte LDS granules are XOR-swizzled by row pairs, which keeps the
//    16-byte writes and the MFMA operand reads free of bank conflicts.
//  * Epilogue per wave through a private 8 KB LDS strip (32 rows x 128 columns),
//    so writing a tile needs no block-wide barrier; accumulators are drained
//    block by block, converted with v_cvt_pk_bf16_f32, and stored as 16-byte
//    non-temporal writes.  The first k step of each tile takes a zero
//    accumulator operand instead of clearing the accumulators.
//  * Tile order: block b runs on XCD b % 8; XCD x owns N-tiles [x*G, (x+1)*G)
//    and walks the M-tiles, so its 2 MiB slice of W stays in its L2 and the
//    N-tiles of one M-tile, running side by side, share the A rows in L2.
#include <type_traits>

#include "bf16_tile_common.hpp"

namespace mla {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int GPR = BK / 8;                   // 16-byte granules per tile row
constexpr int RP = NT / GPR;                  // tile rows per loader pass
constexpr int LA = BM / RP;                   // A granules per thread per stage
constexpr int LB = BN / RP;                   // W granules per thread per stage
constexpr int WTM = 128, WTN = 128;           // wave tile (rows m, columns n)
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int A_STAGE = BM * BK;              // elements
constexpr int STAGE = (BM + BN) * BK;         // elements per LDS stage
constexpr int EPI_ROWS = 32;
constexpr int EPI = EPI_ROWS * WTN;           // elements of one wave's epilogue strip
constexpr int LDS_ELEMS = 2 * STAGE + 4 * EPI;
static_assert(LDS_ELEMS * 2 <= 163840, "LDS budget");
static_assert(BK == 64, "the stage body is written for four 16-wide k steps");

__global__ void __launch_bounds__(NT, 1) gemm_bf16_persistent(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived offsets in SGPRs
    const int wm = wave >> 1, wn = wave & 1;
    const int gcol = tid % GPR, rsub = tid / GPR;

    const TileList tl = make_tiles(P);
    const int KT = P.K / BK;
    const int S = tl.count * KT;
    if (S == 0)
        return;

    // Per-lane byte offsets of this thread's granule within a tile's first row
    // pass; row passes and k stages add wave-uniform offsets.
    const uint32_t a_voff = (uint32_t)(rsub * P.lda + gcol * 8) * 2;
    const uint32_t w_voff = (uint32_t)(rsub * P.K + gcol * 8) * 2;
    const uint32_t a_pass = (uint32_t)(RP * P.lda * 2), w_pass = (uint32_t)(RP * P.K * 2);

    u32x4 ra[LA], rb[LB];
    // Global loads of stage `sigma` (tile sigma / KT, k-stage sigma % KT); past
    // the last stage the last one is loaded again (never used).
    auto gload = [&](int sigma) {
        sigma = sigma < S ? sigma : S - 1;
        const int i = sigma / KT, ks = sigma - i * KT;
        int tm, tn;
        tl.coords(i, tm, tn);
        const int mrows = min(P.M - tm * BM, BM), nrows = min(P.N - tn * BN, BN);
        const rsrc_t ar = make_rsrc(P.A + (int64_t)tm * BM * P.lda, (uint32_t)(mrows * P.lda * 2));
        const rsrc_t wr = make_rsrc(P.W + (int64_t)tn * BN * P.K, (uint32_t)(nrows * P.K * 2));
        const uint32_t kb = ks * BK * 2;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            ra[j] = buf_ld16(ar, a_voff, j * a_pass + kb);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            rb[j] = buf_ld16(wr, w_voff, j * w_pass + kb);
    };

    // LDS row r holds granule g at position g ^ ((r >> 1) & 7); every row a thread
    // writes or a lane reads has the same (r >> 1) & 7, so one lane offset plus
    // compile-time row offsets addresses all of them.
    const int lw_off = rsub * BK + (gcol ^ ((rsub >> 1) & 7)) * 8;
    auto lwrite = [&](int buf) {
        uint16_t* as = smem + buf * STAGE + lw_off;
        uint16_t* bs = as + A_STAGE;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            lds_st16(as + j * RP * BK, ra[j]);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            lds_st16(bs + j * RP * BK, rb[j]);
    };

    f32x16 acc[FN][FM];

    const int lrow = lane & 31;
    int fr_off[BK / 16];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
        fr_off[kk] = lrow * BK + ((2 * kk + (lane >> 5)) ^ ((lrow >> 1) & 7)) * 8;

    // Fragments of one 16-wide k step: FN weight rows and FM activation rows.
    bf16x8 fa0[FN], fb0[FM], fa1[FN], fb1[FM];
    auto load_frags = [&](int buf, int kk, bf16x8 (&fa)[FN], bf16x8 (&fb)[FM]) {
        const uint16_t* as = smem + buf * STAGE + wm * WTM * BK + fr_off[kk];
        const uint16_t* bs = smem + buf * STAGE + A_STAGE + wn * WTN * BK + fr_off[kk];
#pragma unroll
        for (int i = 0; i < FN; ++i)
            fa[i] = as_bf16x8(lds_ld16(bs + i * 32 * BK));
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fb[j] = as_bf16x8(lds_ld16(as + j * 32 * BK));
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
    using first_t = std::integral_constant<bool, true>;
    using rest_t = std::integral_constant<bool, false>;

    // One stage (see the header comment for the schedule).
    auto stage = [&](int sigma, auto first) {
        const int buf = sigma & 1;
        load_frags(buf, 1, fa1, fb1);
        mfmas(fa0, fb0, first);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(buf, 2, fa0, fb0);
        lwrite(buf ^ 1);
        mfmas(fa1, fb1, rest_t{});
        __builtin_amdgcn_sched_barrier(0);
        load_frags(buf, 3, fa1, fb1);
        gload(sigma + 2);
        mfmas(fa0, fb0, rest_t{});
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        load_frags(buf ^ 1, 0, fa0, fb0);
        mfmas(fa1, fb1, rest_t{});
        __builtin_amdgcn_sched_barrier(0);
    };

    // Write the finished tile through this wave's strip.
    auto epilogue = [&](int tile) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const int mrows = min(P.M - tm * BM, BM);
        const rsrc_t cr = make_rsrc(P.C + (int64_t)tm * BM * P.N, (uint32_t)(mrows * P.N * 2));
        uint16_t* E = smem + 2 * STAGE + wave * EPI;
        const int ncol0 = tn * BN + wn * WTN;
        constexpr int EG = WTN / 8;  // granules per strip row
        constexpr int PER_LANE = EPI_ROWS * EG / 64;
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
            u32x4 v[PER_LANE];
#pragma unroll
            for (int p = 0; p < PER_LANE; ++p) {
                const int idx = p * 64 + lane;
                const int r = idx / EG, g = idx % EG;
                v[p] = lds_ld16(E + r * WTN + swz(r, g, EG) * 8);
            }
            wave_lds_sync();
#pragma unroll
            for (int p = 0; p < PER_LANE; ++p) {
                const int idx = p * 64 + lane;
                const int r = idx / EG, g = idx % EG;
                const int n = ncol0 + g * 8;
                const uint32_t off = n < P.N ? (uint32_t)(((wm * WTM + j * 32 + r) * P.N + n) * 2) : kOutOfRange;
                buf_st16_nt(cr, v[p], off, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: stage 0 into LDS buffer 0 and its first fragments into
    // registers, stage 1 in flight.
    gload(0);
    lwrite(0);
    gload(1);
    lds_barrier();
    load_frags(0, 0, fa0, fb0);

    int sigma = 0;
    for (int tile = 0; tile < tl.count; ++tile) {
        stage(sigma++, first_t{});
        for (int ks = 1; ks < KT; ++ks)
            stage(sigma++, rest_t{});
        epilogue(tile);
    }
}

}  // namespace

int num_cus()
{
    static int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            v = 256;
        return v > 0 ? v : 256;
    }();
    return n;
}

// K a multiple of 128: the LDS-ring kernel; otherwise the register-staged one.
hipError_t launch_product_bf16(const DecompressArgs& a, hipStream_t s)
{
    if (small_bf16_fits(a))
        return launch_small_bf16(a, 0, s);
    const int cus = num_cus();
    if (a.K % 128 == 0)
        return launch_product_bf16_ring(a, cus, s);
    GemmParams P = make_gemm_params(a, BM, BN, cus);
    log_launch("gemm_bf16_persistent", gemm_grid(P, cus), NT, "M=%d N=%d K=%d tiles=%dx%d xcd_map=%d", P.M, P.N, P.K,
               P.tiles_m, P.tiles_n, P.xcd_map);
    hipLaunchKernelGGL(gemm_bf16_persistent, dim3(gemm_grid(P, cus)), dim3(NT), 0, s, P);
    return hipGetLastError();
}

hipError_t launch_decompress_bf16(const DecompressArgs& a, hipStream_t s)
{
    if (small_bf16_fits(a))
        return launch_small_bf16(a, 1, s);
    hipError_t e = launch_gather_rows(a, 2, s);
    if (e != hipSuccess)
        return e;
    return launch_product_bf16(a, s);
}

// Fused K and V: the rows are gathered once.  With K a multiple of 128 and the
// first projection a whole number of 256-column tiles, both projections run in
// one product launch whose N-tiles span W and then W2 (each activation tile is
// then read from L2 for both); otherwise the two products are launched in turn.
// Few rows: the single-launch few-rows kernel gathers with the first projection
// and the second reads the gathered rows back.
hipError_t launch_decompress_kv_bf16(const DecompressArgs& a, hipStream_t s)
{
    const DecompressArgs k = first_projection(a), v = second_projection(a);
    if (small_bf16_fits(k) && small_bf16_fits(v)) {
        hipError_t e = launch_small_bf16(k, 1, s);
        return e != hipSuccess ? e : launch_small_bf16(v, 0, s);
    }
    hipError_t e = launch_gather_rows(a, 2, s);
    if (e != hipSuccess)
        return e;
    if (a.K % 128 == 0 && a.N % kRingTileN == 0)
        return launch_product_bf16_ring(a, num_cus(), s);
    e = launch_product_bf16(k, s);
    return e != hipSuccess ? e : launch_product_bf16(v, s);
}

}  // namespace mla
