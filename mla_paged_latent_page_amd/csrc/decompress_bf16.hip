// bf16 up-projection of gathered latent rows for gfx950 (page
// "generic_flare_mla_decompress_k_cache_ragged_paged", summary: the gathered rows are
// multiplied by the weight; weight layout [num_heads*qk_nope_head_dim, kv_latent_dim]
// from page "mla_prefill_decode_graph_fp8", Args w_k):
//   k_buffer[r][n] = sum_{k<K} k_latent[r][k] * W[n][k]   (fp32 accumulate, bf16 RNE out)
//
// The call runs the paged gather (gather.hip) into k_latent_buffer, then this
// persistent product kernel over k_latent_buffer.
//
// Design of the product (one block of 4 waves per CU, persistent over tiles):
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

#include "launch.hpp"

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

struct GemmParams {
    const uint16_t* A;   // [M][lda] bf16 (gathered rows)
    const uint16_t* W;   // [N][K] bf16
    uint16_t* C;         // [M][N] bf16
    int lda;
    int M, N, K;
    int tiles_m, tiles_n;
    int xcd_map;
};

// The tiles of one persistent block, in the order it processes them.
struct TileList {
    int first, step, count, Gn, x, tiles_n;
    bool xcd;
    __device__ void coords(int i, int& tm, int& tn) const
    {
        const int u = first + i * step;
        if (xcd) {
            tm = u / Gn;
            tn = x * Gn + (u - tm * Gn);
        } else {
            tm = u / tiles_n;
            tn = u - tm * tiles_n;
        }
    }
};

__device__ inline TileList make_tiles(const GemmParams& P)
{
    TileList L;
    L.tiles_n = P.tiles_n;
    L.xcd = P.xcd_map != 0;
    int total;
    if (L.xcd) {
        L.x = blockIdx.x & 7;
        L.first = blockIdx.x >> 3;
        L.step = gridDim.x >> 3;
        L.Gn = P.tiles_n >> 3;
        total = P.tiles_m * L.Gn;
    } else {
        L.x = 0;
        L.Gn = 1;
        L.first = blockIdx.x;
        L.step = gridDim.x;
        total = P.tiles_m * P.tiles_n;
    }
    L.count = L.first < total ? (total - L.first + L.step - 1) / L.step : 0;
    return L;
}

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

template <int Q>
__device__ inline u32x2 acc_pack4(const f32x16& a)
{
    u32x2 v;
    v[0] = pack_bf16x2(acc_read<4 * Q + 0>(a), acc_read<4 * Q + 1>(a));
    v[1] = pack_bf16x2(acc_read<4 * Q + 2>(a), acc_read<4 * Q + 3>(a));
    return v;
}

__global__ void __launch_bounds__(NT, 1) gemm_bf16_persistent(GemmParams P)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

}  // namespace

hipError_t launch_product_bf16(const DecompressArgs& a, hipStream_t s)
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
    const int cus = num_cus();
    P.xcd_map = (P.tiles_n % 8 == 0 && cus % 8 == 0) ? 1 : 0;
    const int tiles = P.tiles_m * P.tiles_n;
    int grid = tiles < cus ? tiles : cus;
    if (P.xcd_map)
        grid = cus;  // every XCD gets the same number of blocks; idle blocks exit at once
    hipLaunchKernelGGL(gemm_bf16_persistent, dim3(grid), dim3(NT), 0, s, P);
    return hipGetLastError();
}

hipError_t launch_decompress_bf16(const DecompressArgs& a, hipStream_t s)
{
    hipError_t e = launch_gather_rows(a, 2, s);
    if (e != hipSuccess)
        return e;
    return launch_product_bf16(a, s);
}

}  // namespace mla
