// Persistent fp8 block-scaled product for gfx950 (page "mla_prefill_decode_graph_fp8":
// Parameters fp8_dtype, fp8_scale_dtype, m/n/k_scale_granularity; Args w_k, w_k_scale):
//
//   k_buffer[m][n] = bf16( sum_kb s_a[m][kb] * s_w[n/128][kb] * sum_{k in kb} q_a[m][k] * q_w[n][k] )
//
// with q_a, s_a the e4m3fn codes and fp32 scales the gather pass wrote to the
// workspace (1 x 128 blocks) and q_w, s_w the weight codes and 128 x 128 scales.
//
//  * One 512-thread block per CU walks 256 x 128 output tiles in the XCD-aware
//    order of the bf16 kernels; 8 waves in a 4 x 2 grid own 64 x 64 each.
//  * K advances one scale block (128 codes = 128 bytes per row) per stage.  A
//    stage's operand tiles (256 + 128 rows of 128 bytes) and its scales go from
//    memory straight into one of three LDS slots (buffer loads with an LDS
//    destination), two stages ahead, so a load has two stage times to land;
//    rows are 8 granules of 16 bytes XOR-swizzled by (row / 2) % 8.  The stream
//    of stages runs straight across tile boundaries.
//  * v_mfma_scale_f32_32x32x64_f8f6f4: two per 32 x 32 block and scale block.
//    The fp32 scales are not powers of two, so they cannot ride on the MFMA's
//    E8M0 scale inputs; instead the accumulators are kept in units of the
//    current stage's scale sig = s_a * s_w: before a stage's MFMAs add its
//    products, the accumulators are multiplied by ref / sig (ref: the previous
//    stage's scale), and the epilogue multiplies by the last ref.  A tile's
//    first stage starts its accumulators from zero instead.  The weight is
//    the MFMA's row operand, so a lane's 16 results lie in one output row (one
//    s_a per 32-row block) and a wave's 64 columns lie in one 128-wide weight
//    block (s_w is uniform).  A zero s_w makes its stage add nothing: the MFMAs
//    then run with E8M0 operand scales 2^-127 each, so every product underflows
//    to zero, and the accumulators keep their scale.  A zero activation scale
//    (an fp8 cache may hold one) does the same for its row alone, through that
//    lane's own E8M0 scale.
//  * Epilogue as in the bf16 ring kernel (bf16 pairs into a per-wave LDS strip,
//    read back as 16-byte row pieces, non-temporal stores), 32 rows at a time;
//    the strips live in the ring slot the tile's last stage consumed.
//    The product is bound by these stores: 2 bytes out per 1024 flop of fp8 work.
#include <type_traits>

#include "bf16_tile_common.hpp"

namespace mla {
namespace {

constexpr int BM = 256, BN = 128, BK = 128;       // BK: codes (bytes) per row per stage = one scale block
constexpr int WAVES_M = 4, WAVES_N = 2, NW = WAVES_M * WAVES_N, NT = 64 * NW;
constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 64 x 64 per wave
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int ROWB = BK;
constexpr int CHUNK_ROWS = 1024 / ROWB;           // rows per 1 KB load chunk
// A slot holds one stage: the activation rows, the weight rows, the stage's
// activation scales (one float per row) and 64 copies of its weight scale.
constexpr int A_BYTES = BM * ROWB, W_BYTES = BN * ROWB, SA_OFF = A_BYTES + W_BYTES, SW_OFF = SA_OFF + BM * 4;
constexpr int SLOT_BYTES = SW_OFF + 256, NSLOT = 3;
constexpr int CA = BM / CHUNK_ROWS / NW, CB = BN / CHUNK_ROWS / NW;
constexpr int EPI_ROWS = 32, EPI = EPI_ROWS * WTN, EG = WTN / 8, EPI_PER_LANE = EPI_ROWS * EG / 64;
constexpr int STORES_PER_TILE = (WTM / EPI_ROWS) * EPI_PER_LANE;
static_assert(NSLOT * SLOT_BYTES <= 163840, "LDS budget");
static_assert(NW * EPI * 2 <= SLOT_BYTES, "the strips fit in one ring slot");
static_assert(CA * NW * CHUNK_ROWS == BM && CB * NW * CHUNK_ROWS == BN, "loader shape");
static_assert(CA % 2 == 0 && CB % 2 == 0, "chunks alternate between the two swizzle phases");
static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns sit inside one weight scale block");
static_assert(STORES_PER_TILE <= 63, "vmcnt range");
static_assert(SLOT_BYTES % 256 == 0 && BM / 64 < NW, "slot layout");
constexpr int LOADS = CA + CB + 1;  // loads per wave per stage

struct Fp8GemmParams {
    const uint8_t* A;     // [M][lda] activation codes (the first K of each row used)
    const float* SA;      // [M][sas] activation scales (the first K/128 used)
    const uint8_t* W;     // [N][K] weight codes
    const float* SW;      // [N/128][K/128] weight scales
    uint16_t* C;          // [M][N] bf16
    int M, N, K;
    int lda, sas;         // row strides of A (bytes) and SA (floats)
    int tiles_m, tiles_n;
    int xcd_map;
    // Second projection (fused K and V): N-tiles tiles_n1 .. tiles_n - 1 use
    // W2 [N2][K] with scales SW2 and write C2 [M][N2].
    const uint8_t* W2;
    const float* SW2;
    uint16_t* C2;
    int N2, tiles_n1;
};

// The projection an N-tile belongs to, and the tile's index within it.
struct Fp8Segment {
    const uint8_t* W;
    const float* SW;
    uint16_t* C;
    int N, tn;
};
__device__ inline Fp8Segment segment_of(const Fp8GemmParams& P, int tn)
{
    if (tn < P.tiles_n1)
        return Fp8Segment{P.W, P.SW, P.C, P.N, tn};
    return Fp8Segment{P.W2, P.SW2, P.C2, P.N2, tn - P.tiles_n1};
}
__device__ inline int first_projection_tiles(const Fp8GemmParams& P) { return P.tiles_n1; }

struct Cursor {
    int tile, ks, tn, row0;     // tn: the tile's index within its projection
    i32x4 ar, wr, swr;   // operand tiles and weight scales, as resources for the inline-assembly loads
};
// Every load of the main loop is issued from inline assembly into LDS, so the
// compiler sees no vector-memory loads there and inserts no waits of its own:
// the only waits are the explicit ones before each stage's barrier.

__device__ inline u32x2 pack4(float a, float b, float c, float d)
{
    return u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ inline i32x8 join(u32x4 lo, u32x4 hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__global__ void __launch_bounds__(NT, 1) gemm_fp8_ring(Fp8GemmParams P)
{
    __shared__ __attribute__((aligned(1024))) char ring[NSLOT * SLOT_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const TileList tl = make_tiles(P);
    const int KT = P.K / BK;
    if (tl.count == 0)
        return;
    const int total = tl.count * KT;  // stages this block runs
    // Waves w and w + 4 share a SIMD.  At equal priority the older wave wins
    // the issue slots, and waves 4..7 reached each stage's barrier some 600
    // cycles after waves 0..3 (per-stage timestamps); priority for the later
    // waves evens that out (2-3 % on the whole call).
    if (wave >= 4)
        __builtin_amdgcn_s_setprio(1);

    // Loader lanes: in a 1 KB chunk (8 rows of 128 bytes) lane l fills row l/8 at
    // granule position l%8, i.e. logical granule (l%8) ^ ((row/2)%8); odd chunks
    // start 8 rows further, which adds 4 to (row/2)%8.
    const int lrow = lane >> 3;
    const int lg_even = (lane & 7) ^ ((lrow >> 1) & 7), lg_odd = (lane & 7) ^ (((lrow >> 1) + 4) & 7);
    const uint32_t k_lane[2] = {(uint32_t)(lrow * P.K + lg_even * 16), (uint32_t)(lrow * P.K + lg_odd * 16)};
    const uint32_t chunk = (uint32_t)(CHUNK_ROWS * P.K);
    const uint32_t a_lane[2] = {(uint32_t)(lrow * P.lda + lg_even * 16), (uint32_t)(lrow * P.lda + lg_odd * 16)};
    const uint32_t a_chunk = (uint32_t)(CHUNK_ROWS * P.lda);
    const i32x4 sar = make_srd(P.SA, (uint32_t)((int64_t)P.M * P.sas * 4));
    const uint32_t ring_lds = lds_addr(ring);

    auto cursor_at = [&](int tile, Cursor& c) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const int mrows = min(P.M - tm * BM, BM);
        c.tile = tile;
        c.ks = 0;
        const Fp8Segment sg = segment_of(P, tn);
        c.tn = sg.tn;
        c.row0 = tm * BM;
        c.ar = make_srd(P.A + (int64_t)tm * BM * P.lda, (uint32_t)(mrows * P.lda));
        c.wr = make_srd(sg.W + (int64_t)sg.tn * BN * P.K, (uint32_t)(BN * P.K));
        c.swr = make_srd(sg.SW, (uint32_t)((sg.N / 128) * KT * 4));
    };
    // The cursor's stage into ring slot `sl`: operand tiles, the activation
    // scales of the tile's rows (0 past M; waves 0..3 take 64 rows each) and
    // the weight scale (wave 4, every lane the same value).  Past the last tile
    // the last stage is loaded again (never used).
    auto issue = [&](int sl, Cursor& c) __attribute__((always_inline)) {
        const uint32_t s = ring_lds + sl * SLOT_BYTES;
        const uint32_t kb = c.ks * BK;
#pragma unroll
        for (int q = 0; q < CA; ++q) {
            const int ch = wave * CA + q;
            asm_ld16_lds(c.ar, s + ch * 1024, a_lane[q & 1], ch * a_chunk + kb);
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int ch = wave * CB + q;
            asm_ld16_lds(c.wr, s + A_BYTES + ch * 1024, k_lane[q & 1], ch * chunk + kb);
        }
        // Every wave issues the same number of loads (the weight-scale copies
        // of waves 4..7 are identical), so one vmcnt value fits all waves.
        if (wave < BM / 64)
            asm_ld4_lds(sar, s + SA_OFF + wave * 256, (uint32_t)((c.row0 + wave * 64 + lane) * P.sas) * 4,
                        (uint32_t)c.ks * 4);
        else
            asm_ld4_lds(c.swr, s + SW_OFF, 0u, (uint32_t)(c.tn * KT + c.ks) * 4);
        if (++c.ks == KT) {
            if (c.tile + 1 < tl.count)
                cursor_at(c.tile + 1, c);
            else
                c.ks = KT - 1;
        }
    };

    // Fragment byte offsets (lane part): k step kk of a stage covers codes
    // [64 kk, 64 kk + 64); lane l takes row l%32, codes 32*(l/32) .. +32 of it,
    // i.e. granules 4 kk + 2 (l/32) + h, h = 0, 1.
    const int frow = lane & 31;
    int fr_off[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fr_off[kk][h] = frow * ROWB + (((4 * kk + 2 * (lane >> 5) + h) ^ ((frow >> 1) & 7)) * 16);

    // This stage's fragments and scales.
    i32x8 fw[2][FN], fa[2][FM];
    float sa_c[FM], sw_c;
    // The stage's scales (KK == 0) and the fragments of its k step KK.
    auto load_frags = [&](int sl, auto kk_c) __attribute__((always_inline)) {
        constexpr int kk = decltype(kk_c)::value;
        const char* s = ring + sl * SLOT_BYTES;
        if constexpr (kk == 0) {
#pragma unroll
            for (int j = 0; j < FM; ++j)
                sa_c[j] = *reinterpret_cast<const float*>(s + SA_OFF + (wm * WTM + j * 32 + (lane & 31)) * 4);
            sw_c = *reinterpret_cast<const float*>(s + SW_OFF + lane * 4);
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const char* p = s + A_BYTES + (wn * WTN + i * 32) * ROWB;
            fw[kk][i] = join(lds_ld16(p + fr_off[kk][0]), lds_ld16(p + fr_off[kk][1]));
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const char* p = s + (wm * WTM + j * 32) * ROWB;
            fa[kk][j] = join(lds_ld16(p + fr_off[kk][0]), lds_ld16(p + fr_off[kk][1]));
        }
    };

    f32x16 acc[FN][FM];
    float ref[FM];  // scale the accumulators are expressed in (0: nothing added yet)
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
            acc[i][j] = f32x16{};
#pragma unroll
    for (int j = 0; j < FM; ++j)
        ref[j] = 0.0f;

    // Write the finished tile through per-wave strips of 32 rows x 64 columns
    // in ring slot `sl`, which the tile's last stage has just consumed: every
    // wave has read it once the block meets, and it is not refilled before the
    // next stage's barrier.
    auto epilogue = [&](int tile, int sl) __attribute__((always_inline)) {
        int tm, tn;
        tl.coords(tile, tm, tn);
        const int mrows = min(P.M - tm * BM, BM);
        const Fp8Segment sg = segment_of(P, tn);
        const rsrc_t cr = make_rsrc(sg.C + (int64_t)tm * BM * sg.N, (uint32_t)(mrows * sg.N * 2));
        uint16_t* E = reinterpret_cast<uint16_t*>(ring + sl * SLOT_BYTES) + wave * EPI;
        const int ncol0 = sg.tn * BN + wn * WTN;
        // The lane's addresses are recomputed per tile from an opaque copy of
        // the lane id: hoisted out of the stage loop they would hold registers
        // for the whole kernel.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int row = ln & 31;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int col = i * 32 + 4 * (ln >> 5);
                uint16_t* e = E + row * WTN + (col & 7);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    lds_st8(e + swz(row, (col >> 3) + q, EG) * 8,
                            pack4(acc[i][j][4 * q] * ref[j], acc[i][j][4 * q + 1] * ref[j],
                                  acc[i][j][4 * q + 2] * ref[j], acc[i][j][4 * q + 3] * ref[j]));
            }
            wave_lds_sync();
            u32x4 v[EPI_PER_LANE];
#pragma unroll
            for (int p = 0; p < EPI_PER_LANE; ++p) {
                const int idx = p * 64 + ln;
                const int r = idx / EG, g = idx % EG;
                v[p] = lds_ld16(E + r * WTN + swz(r, g, EG) * 8);
            }
            wave_lds_sync();
#pragma unroll
            for (int p = 0; p < EPI_PER_LANE; ++p) {
                const int idx = p * 64 + ln;
                const int r = idx / EG, g = idx % EG;
                const uint32_t off = (uint32_t)(((wm * WTM + j * 32 + r) * sg.N + ncol0 + g * 8) * 2);
                buf_st16_nt(cr, v[p], off, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
            ref[j] = 0.0f;
    };

    // Prologue: stages 0 and 1 in flight.
    Cursor lc;
    cursor_at(0, lc);
    issue(0, lc);
    issue(1, lc);

    int slot = 0;      // ring slot of the current stage
    int ks = 0, tile = 0;

    // Stage g: wait for its loads (issued two stages earlier; stage g+1's may
    // stay in flight, and after the first stage of a tile other than the first
    // so may the previous tile's stores); the barrier makes the slot visible to
    // all waves and frees the slot of stage g-1, which stage g+2's loads refill.
    while (true) {
        if (ks == 0 && tile > 0)
            vm_barrier<LOADS + STORES_PER_TILE>();
        else
            vm_barrier<LOADS>();
        load_frags(slot, std::integral_constant<int, 0>{});
        const int after = slot == 0 ? 2 : slot - 1;
        issue(after, lc);
        const bool skip = sw_c == 0.0f;
        const int e8 = skip ? 0 : 127;
        float rho[FM], ref_next[FM];
        int e8a[FM];   // E8M0 scale of this lane's activation row in this stage
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const float sig = sa_c[j] * sw_c;
            // A zero (or subnormal) activation scale: the row's block adds
            // nothing.  Its codes go in with E8M0 scale 2^-127, so each of its
            // products is below 2^-109 (exactly zero when nothing was added
            // before: the accumulators stay in units of ref = 0), and the
            // accumulators keep their scale, as for a zero weight scale.
            const bool dead = skip || __builtin_fabsf(sig) < 1.17549435e-38f;
            const float r = ref[j] * __builtin_amdgcn_rcpf(sig);
            rho[j] = dead ? 1.0f : (ref[j] == 0.0f ? 0.0f : r);
            ref_next[j] = dead ? ref[j] : sig;
            e8a[j] = dead ? 0 : 127;
        }
        // Per block: its rescale (none in a tile's first stage: the
        // accumulators start from zero there), its first-step MFMA and one of
        // the second step's fragments read; then the second step.  Fences keep
        // that order, so no MFMA waits for the one before it on the same block.
        const char* sb = ring + slot * SLOT_BYTES;
        auto read_k1 = [&](int b) __attribute__((always_inline)) {
            if (b < FN) {
                const char* p = sb + A_BYTES + (wn * WTN + b * 32) * ROWB;
                fw[1][b] = join(lds_ld16(p + fr_off[1][0]), lds_ld16(p + fr_off[1][1]));
            } else {
                const char* p = sb + (wm * WTM + (b - FN) * 32) * ROWB;
                fa[1][b - FN] = join(lds_ld16(p + fr_off[1][0]), lds_ld16(p + fr_off[1][1]));
            }
        };
        static_assert(FN + FM == FN * FM, "one second-step fragment read per block");
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[0][i], fa[0][j], f32x16{}, 0, 0, 0,
                                                                                e8, 0, e8a[j]);
                    read_k1(i * FM + j);
                    __builtin_amdgcn_sched_barrier(0);
                }
        } else {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[i][j][e] *= rho[j];
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[0][i], fa[0][j], acc[i][j], 0, 0, 0,
                                                                                e8, 0, e8a[j]);
                    read_k1(i * FM + j);
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[1][i], fa[1][j], acc[i][j], 0, 0, 0, e8,
                                                                            0, e8a[j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < FM; ++j)
            ref[j] = ref_next[j];
        const int done = slot;
        slot = slot == NSLOT - 1 ? 0 : slot + 1;
        if (++ks == KT) {
            epilogue(tile, done);
            ks = 0;
            if (++tile == tl.count)
                break;
        }
    }
    // The spare loads of the last stages may still be landing in LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

hipError_t launch_product_fp8_ring(const DecompressArgs& a, int cus, hipStream_t s)
{
    Fp8GemmParams P;
    P.A = static_cast<const uint8_t*>(a.q);
    P.SA = a.q_scale;
    P.W = static_cast<const uint8_t*>(a.W);
    P.SW = a.W_scale;
    P.C = static_cast<uint16_t*>(a.out);
    P.M = a.M;
    P.N = a.N;
    P.K = a.K;
    P.lda = a.q_ld ? a.q_ld : a.K;
    P.sas = a.qs_ld ? a.qs_ld : a.K / 128;
    P.tiles_m = (a.M + BM - 1) / BM;
    P.tiles_n = a.N / BN;
    P.tiles_n1 = P.tiles_n;
    P.W2 = static_cast<const uint8_t*>(a.W2);
    P.SW2 = a.W2_scale;
    P.C2 = static_cast<uint16_t*>(a.out2);
    P.N2 = a.N2;
    P.tiles_n += a.N2 / BN;
    if (a.N2 > 0) {
        // Two projections: both eighths of the weight at once would take half
        // of an XCD's L2 and get evicted by the streaming rows, so each XCD
        // walks the rows over its eighth of one projection, then the other's.
        P.xcd_map = (P.tiles_n1 % 8 == 0 && (P.tiles_n - P.tiles_n1) % 8 == 0 && cus % 8 == 0) ? 3 : 0;
    } else {
        P.xcd_map = (P.tiles_n % 8 == 0 && cus % 8 == 0) ? 1 : 0;
    }
    const int tiles = P.tiles_m * P.tiles_n;
    const int grid = P.xcd_map ? cus : (tiles < cus ? tiles : cus);
    log_launch("gemm_fp8_ring", grid, NT, "M=%d N=%d N2=%d K=%d tiles=%dx%d xcd_map=%d", P.M, P.N, P.N2, P.K, P.tiles_m,
               P.tiles_n, P.xcd_map);
    hipLaunchKernelGGL(gemm_fp8_ring, dim3(grid), dim3(NT), 0, s, P);
    return hipGetLastError();
}

}  // namespace mla
