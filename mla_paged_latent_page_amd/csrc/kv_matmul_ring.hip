// Persistent projection of hidden states into the paged K/V cache for gfx950
// (page "kv_matmul_ragged_paged", summary and Args hidden_state, input_row_offsets,
// weight, kv_collection, layer_idx):
//
//   out[t][n] = sum_k H[t][k] * W[k][n]   (fp32 accumulate, bf16 RNE into the cache)
//   token t of request b goes to position cache_lengths[b] + (t - row_offsets[b]);
//   columns [0, HD) form its K row, [HD, 2HD) its V row.
//
// Same pipeline as the LDS-ring decompress product (decompress_bf16_ring.hip):
// one 512-thread block per CU walks 256 x 256 output tiles in XCD-aware order
// (activation-stationary: each XCD runs all N-tiles of its M-tiles side by
// side; 8 waves of 128 x 64), and 64-wide K stages go from memory straight into two
// LDS slots (buffer loads with an LDS destination).  The difference is the
// weight: it is [K][N] with N contiguous, while the MFMA operand wants 8
// consecutive k values per lane.  Its stage tile is kept in LDS as it lies in
// memory (64 k-rows of 256 columns, 512 bytes each) and read with
// ds_read_b64_tr_b16: in each group of 16 lanes, lane c addresses the 4 columns
// 4(c%4) .. +3 of k-row c/4 of a 4 x 16 block, and lane i receives column i of
// all 4 rows.  Two such reads give the 8 k values of a fragment.  The 16-byte
// granules of a k-row are XOR-swizzled by 4 * (row % 4), so the 4 rows one read
// touches fall in different banks.
//
// Epilogue: the destination of every tile row (request search, page table) is
// resolved once per tile into LDS; each wave then writes its 128 x 64 piece
// through a private strip, 16 rows at a time, as 16-byte pieces of the token
// rows in the pages (a 64-column slice lies inside the K or the V half).
#include <type_traits>

#include "bf16_tile_common.hpp"

namespace mla {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = 2, WAVES_N = 4, NW = WAVES_M * WAVES_N, NT = 64 * NW;
constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 128 x 64 per wave
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int A_ROWB = BK * 2;                   // bytes per hidden-state row per stage
constexpr int W_ROWB = BN * 2;                   // bytes per weight k-row per stage
constexpr int A_BYTES = BM * A_ROWB, W_BYTES = BK * W_ROWB, SLOT_BYTES = A_BYTES + W_BYTES;
constexpr int CA = A_BYTES / 1024 / NW, CB = W_BYTES / 1024 / NW;   // 1 KB load chunks per wave
constexpr int LOADS = CA + CB;
constexpr int EPI_ROWS = 16, EPI = EPI_ROWS * WTN, EG = WTN / 8, EPI_PER_LANE = EPI_ROWS * EG / 64;
static_assert(2 * SLOT_BYTES + NW * EPI * 2 + BM * 8 <= 163840, "LDS budget");
static_assert(CA * NW * 1024 == A_BYTES && CB * NW * 1024 == W_BYTES, "loader shape");
static_assert(CA % 2 == 0 && CB % 2 == 0, "chunks alternate between two swizzle phases");

struct KvRingParams {
    KvMatmulArgs a;
    int tiles_m, tiles_n;
    int xcd_map;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ inline v4i16 lds_read_tr16(const char* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(__attribute__((address_space(3))) void*)p);
}

__global__ void __launch_bounds__(NT, 1) kv_matmul_ring(KvRingParams P)
{
    __shared__ __attribute__((aligned(1024))) char slot0[SLOT_BYTES];
    __shared__ __attribute__((aligned(1024))) char slot1[SLOT_BYTES];
    __shared__ __attribute__((aligned(16))) uint16_t strips[NW * EPI];
    __shared__ int64_t rowoff[BM];
    auto slot = [&](auto b) __attribute__((always_inline)) -> char* {
        if constexpr (decltype(b)::value == 0) return slot0;
        else return slot1;
    };

    const KvMatmulArgs& a = P.a;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const TileList tl = make_tiles(P);
    const int KT = a.Kd / BK;
    if (tl.count == 0)
        return;

    // Hidden-state loader: a 1 KB chunk is 8 rows of 128 bytes; lane l fills
    // row l/8 at granule position l%8, i.e. logical granule (l%8) ^ ((row/2)%8).
    const int lrow = lane >> 3;
    const int lg_even = (lane & 7) ^ ((lrow >> 1) & 7), lg_odd = (lane & 7) ^ (((lrow >> 1) + 4) & 7);
    const uint32_t a_lane[2] = {(uint32_t)(lrow * a.Kd * 2 + lg_even * 16), (uint32_t)(lrow * a.Kd * 2 + lg_odd * 16)};
    const uint32_t a_chunk = (uint32_t)(8 * a.Kd * 2);
    // Weight loader: a 1 KB chunk is 2 k-rows of 512 bytes; lane l fills k-row
    // l/32 of the chunk at granule position l%32, i.e. logical granule
    // (l%32) ^ (4 * (krow % 4)); chunk c starts at k-row 2c, so even and odd
    // chunks differ in krow % 4.
    const int wrow = lane >> 5;
    const int wg_even = (lane & 31) ^ (4 * (wrow & 3)), wg_odd = (lane & 31) ^ (4 * ((wrow + 2) & 3));
    const uint32_t w_lane[2] = {(uint32_t)(wrow * a.N * 2 + wg_even * 16), (uint32_t)(wrow * a.N * 2 + wg_odd * 16)};
    const uint32_t w_chunk = (uint32_t)(2 * a.N * 2);

    struct Cursor {
        int tile, ks;
        i32x4 ar, wr;   // operand tiles, as resources for the inline-assembly loads
    };
    auto cursor_at = [&](int tile, Cursor& c) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const int mrows = min(a.T - tm * BM, BM);
        c.tile = tile;
        c.ks = 0;
        c.ar = make_srd(a.H + (int64_t)tm * BM * a.Kd, (uint32_t)(mrows * a.Kd * 2));
        c.wr = make_srd(a.W + (int64_t)tn * BN, (uint32_t)((int64_t)a.Kd * a.N * 2 - (int64_t)tn * BN * 2));
    };
    // Load q (of LOADS) of the cursor's stage into ring slot b, from inline
    // assembly: the compiler adds no waits of its own for these loads.
    auto load_one = [&](auto b, const Cursor& c, int q) __attribute__((always_inline)) {
        const uint32_t s = lds_addr(slot(b));
        if (q < CA) {
            const int ch = wave * CA + q;
            asm_ld16_lds(c.ar, s + ch * 1024, a_lane[q & 1], ch * a_chunk + c.ks * BK * 2);
        } else {
            const int ch = wave * CB + (q - CA);
            asm_ld16_lds(c.wr, s + A_BYTES + ch * 1024, w_lane[(q - CA) & 1], (c.ks * BK) * a.N * 2 + ch * w_chunk);
        }
    };
    auto issue = [&](auto b, Cursor& c) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            load_one(b, c, q);
        ++c.ks;
    };
    auto settle = [&](Cursor& c) __attribute__((always_inline)) {
        if (c.ks == KT) {
            if (c.tile + 1 < tl.count)
                cursor_at(c.tile + 1, c);
            else
                c.ks = KT - 1;
        }
    };

    // Hidden-state fragments (the MFMA column operand): lane l reads row l%32 of
    // a 32-row block, granule 2 kk + l/32 of the stage's 8, swizzled.
    const int frow = lane & 31;
    int a_off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        a_off[kk] = frow * A_ROWB + ((2 * kk + (lane >> 5)) ^ ((frow >> 1) & 7)) * 16;
    // Weight fragments (the MFMA row operand) by transposing reads: in 16-lane
    // group G = l/16, lane c = l%16 addresses k-row 8 (G/2) + c/4 (+4 for the
    // second read, + 16 kk for the k step) and columns 16 (G%2) + 4 (c%4) .. +3
    // of the wave's 32-column block i.
    const int G = (lane >> 4) & 3, c16 = lane & 15;
    int w_off[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        const int gbase = (wn * WTN + i * 32) / 8;   // multiple of 4
        const int g = (gbase ^ (4 * (c16 >> 2))) + 2 * (G & 1) + ((c16 & 3) >> 1);
        w_off[i] = A_BYTES + (8 * (G >> 1) + (c16 >> 2)) * W_ROWB + g * 16 + (c16 & 1) * 8;
    }

    bf16x8 fw0[FN], fb0[FM], fw1[FN], fb1[FM];
    auto load_frags = [&](auto b, int kk, bf16x8 (&fw)[FN], bf16x8 (&fb)[FM]) __attribute__((always_inline)) {
        const char* s = slot(b);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const v4i16 lo = lds_read_tr16(s + w_off[i] + (16 * kk) * W_ROWB);
            const v4i16 hi = lds_read_tr16(s + w_off[i] + (16 * kk + 4) * W_ROWB);
            fw[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
            fb[j] = as_bf16x8(lds_ld16(s + (wm * WTM + j * 32) * A_ROWB + a_off[kk]));
    };

    f32x16 acc[FN][FM];
    auto mfmas = [&](const bf16x8 (&fw)[FN], const bf16x8 (&fb)[FM], auto first) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                if constexpr (decltype(first)::value)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fb[j], f32x16{}, 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fb[j], acc[i][j], 0, 0, 0);
            }
    };

    // Destinations of the tile's rows: byte offset of the token's K row in the
    // layer (-1 past the last token).
    auto resolve_rows = [&](int tile) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        for (int r = tid; r < BM; r += NT) {
            const int t = tm * BM + r;
            int64_t off = -1;
            if (t < a.T) {
                const uint32_t b = find_request(a.iro, a.L.batch, (uint32_t)t);
                const uint32_t p = a.cache_len[b] + ((uint32_t)t - a.iro[b]);
                off = store_offset(a.L, b, p);
            }
            rowoff[r] = off;
        }
    };

    auto epilogue = [&](int tile) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        resolve_rows(tile);
        lds_barrier();
        uint16_t* E = strips + wave * EPI;
        const int n0 = tn * BN + wn * WTN;             // first output column of this wave
        const int kv = n0 >= a.HD ? 1 : 0;
        char* dst0 = const_cast<char*>(a.L.base) + kv * a.L.stride_kv + (int64_t)(n0 - kv * a.HD) * 2;
        const int row = lane & (EPI_ROWS - 1), part = (lane & 31) / EPI_ROWS;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
#pragma unroll
            for (int h = 0; h < 32 / EPI_ROWS; ++h) {
                __builtin_amdgcn_sched_barrier(0);
                if (part == h) {
#pragma unroll
                    for (int i = 0; i < FN; ++i) {
                        const int col = i * 32 + 4 * (lane >> 5);
                        uint16_t* e = E + row * WTN + (col & 7);
                        lds_st8(e + swz(row, (col >> 3) + 0, EG) * 8, acc_pack4<0>(acc[i][j]));
                        lds_st8(e + swz(row, (col >> 3) + 1, EG) * 8, acc_pack4<1>(acc[i][j]));
                        lds_st8(e + swz(row, (col >> 3) + 2, EG) * 8, acc_pack4<2>(acc[i][j]));
                        lds_st8(e + swz(row, (col >> 3) + 3, EG) * 8, acc_pack4<3>(acc[i][j]));
                    }
                }
                wave_lds_sync();
#pragma unroll
                for (int p = 0; p < EPI_PER_LANE; ++p) {
                    const int idx = p * 64 + lane;
                    const int r = idx / EG, g = idx % EG;
                    const u32x4 v = lds_ld16(E + r * WTN + swz(r, g, EG) * 8);
                    const int64_t off = rowoff[wm * WTM + j * 32 + h * EPI_ROWS + r];
                    if (off >= 0)
                        st16_nt(dst0 + off + g * 16, v);
                }
                wave_lds_sync();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rowoff is rewritten by the next tile's epilogue only after the next
        // tile's stage barriers, which every wave passes after finishing here.
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using first_t = std::integral_constant<bool, true>;
    using rest_t = std::integral_constant<bool, false>;

    // Prologue: stage 0 landed and visible, stage 1 in flight, stage 0's first
    // fragments read.
    Cursor lc;
    cursor_at(0, lc);
    issue(I0{}, lc);
    settle(lc);
    vm_barrier<0>();
    issue(I1{}, lc);
    settle(lc);
    load_frags(I0{}, 0, fw0, fb0);

    // One stage in slot B, its k step 0 fragments already in registers (the
    // order of decompress_bf16_ring.hip): k steps 0..2 run while the fragments
    // of the step after each are read; the block meets once this thread's
    // loads of the next stage (and any stores) are done; then the loads two
    // stages ahead go into slot B, one per MFMA of k step 3, and the next
    // stage's step-0 fragments are read under those MFMAs.
    auto stage = [&](auto b, auto first) __attribute__((always_inline)) {
        constexpr int B = decltype(b)::value;
        using Bn = std::integral_constant<int, (B + 1) % 2>;
        load_frags(b, 1, fw1, fb1);
        mfmas(fw0, fb0, first);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(b, 2, fw0, fb0);
        mfmas(fw1, fb1, rest_t{});
        __builtin_amdgcn_sched_barrier(0);
        load_frags(b, 3, fw1, fb1);
        mfmas(fw0, fb0, rest_t{});
        __builtin_amdgcn_sched_barrier(0);
        vm_barrier<0>();
        load_frags(Bn{}, 0, fw0, fb0);
        static_assert(LOADS <= FN * FM, "one load per step-3 MFMA");
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw1[i], fb1[j], acc[i][j], 0, 0, 0);
                const int q = i * FM + j;
                if (q < LOADS)
                    load_one(b, lc, q);
            }
        ++lc.ks;
        __builtin_amdgcn_sched_barrier(0);
        settle(lc);
    };
    // Kd is a multiple of 128: a tile is an even number of 64-wide stages.
    for (int tile = 0; tile < tl.count; ++tile) {
        stage(I0{}, first_t{});
        stage(I1{}, rest_t{});
        for (int ks = 2; ks < KT; ks += 2) {
            stage(I0{}, rest_t{});
            stage(I1{}, rest_t{});
        }
        epilogue(tile);
    }
    // The last stage's spare loads may still be landing in LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// Used when the shapes fit its tiling (hidden_dim % 128 == 0, HD % 256 == 0);
// returns hipErrorInvalidValue otherwise so the caller can use the general kernel.
hipError_t launch_kv_matmul_ring(const KvMatmulArgs& a, int cus, hipStream_t s)
{
    if (a.Kd % 128 != 0 || a.HD % 256 != 0)
        return hipErrorInvalidValue;
    KvRingParams P;
    P.a = a;
    P.tiles_m = (a.T + BM - 1) / BM;
    P.tiles_n = a.N / BN;
    // Hidden rows are 8 KB and T is large: keep each activation tile in one
    // XCD's L2 and re-read the (small) weight from the last-level cache.
    P.xcd_map = (cus % 8 == 0 && P.tiles_m >= 8) ? 2 : 0;
    const int tiles = P.tiles_m * P.tiles_n;
    const int grid = P.xcd_map ? cus : (tiles < cus ? tiles : cus);
    log_launch("kv_matmul_ring", grid, NT, "tiles=%dx%d", P.tiles_m, P.tiles_n);
    hipLaunchKernelGGL(kv_matmul_ring, dim3(grid), dim3(NT), 0, s, P);
    return hipGetLastError();
}

}  // namespace mla
