// Few-rows fp8 block-scaled product (page "mla_prefill_decode_graph_fp8": Parameters fp8_dtype,
// fp8_scale_dtype, m/n/k_scale_granularity; Args w_k, w_k_scale), for decode-sized calls:
//
//   k_buffer[m][n] = bf16( sum_kb s_a[m][kb] * s_w[n/128][kb] * sum_{k in kb} q_a[m][k] * q_w[n][k] )
//
// for at most 192 rows of activation codes and their 1 x 128 scales (written
// by the quantising gather, or copied from an e4m3 cache) at K = 512.  At these
// sizes the call is bound by reading the weight (N x 512 codes, 8 MiB at
// N = 16384) once, so the whole weight has to be in flight from the start:
//  * one 256-thread block per 64 weight rows (256 blocks at N = 16384), which
//    lie in one 128-row weight scale block;
//  * at kernel start every wave puts its share of everything the block needs
//    in flight into LDS, scale block by scale block: the 64 x 128 weight codes,
//    the rows' 128 codes, their scales and the weight scale of that block
//    (buffer loads with an LDS destination, from inline assembly; rows past M
//    load as zeros).  Rows of 128 bytes hold 8 granules of 16 bytes
//    XOR-swizzled by (row / 2) % 8, as in the large fp8 product;
//  * the block then meets once per scale block, after waiting for that block's
//    loads only: later blocks' weight is still arriving while the first ones
//    are multiplied;
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with the weight as the row operand (two
//    per 32 x 32 output block and scale block), so a lane's 16 results lie in
//    one output row.  The fp32 scales are not powers of two: the accumulators
//    are kept in units of the current scale sig = s_a * s_w, multiplied by
//    ref / sig before a scale block's MFMAs (ref: the previous block's scale)
//    and by the last ref in the epilogue; a zero scale adds nothing (its
//    operand goes in with E8M0 scale 2^-127), as in the large fp8 product;
//  * wave w owns weight rows 32 (w % 2) .. +32 and the 32-row blocks w / 2,
//    w / 2 + 2, ... of the M rows; the outputs go through LDS so that each
//    store writes whole 128-byte row segments.
#include "bf16_tile_common.hpp"

namespace mla {
namespace {

constexpr int FS_N = 64;                 // weight rows per block
constexpr int FS_K = 512;                // codes per row
constexpr int FS_KB = FS_K / 128;        // scale blocks along K
constexpr int FS_ROWB = 128;             // bytes of a row in one scale block
constexpr int FS_WAVES = 4, FS_NT = 64 * FS_WAVES;
constexpr int FS_MAX_MB = 6;             // 192 rows (the large product is as fast from 224 on)
constexpr int FS_W_BYTES = FS_N * FS_ROWB;   // 8 KB of weight codes per scale block
constexpr int FS_W_CHUNKS_PER_WAVE = FS_W_BYTES / 1024 / FS_WAVES;

template <int MB>
struct FsCfg {
    static constexpr int ROWS = 32 * MB;
    static constexpr int A_BYTES = ROWS * FS_ROWB;               // one scale block of every row
    static constexpr int A_CHUNKS_PER_WAVE = ROWS / 8 / FS_WAVES;
    // Per wave and scale block: weight chunks, row chunks, one load of 64 row
    // scales and one of 64 copies of the weight scale.
    static constexpr int LOADS = FS_W_CHUNKS_PER_WAVE + A_CHUNKS_PER_WAVE + 2;
    static_assert(ROWS % (8 * FS_WAVES) == 0, "row chunks split evenly over the waves");
    static_assert(FS_KB * LOADS <= 63, "vmcnt range");
    static_assert(ROWS <= 64 * FS_WAVES, "one scale load per wave covers 64 rows");
    static_assert(FS_KB * (FS_W_BYTES + A_BYTES) + FS_KB * (256 + FS_WAVES * 64) * 4 <= 163840, "LDS budget");
};

template <int N>
__device__ inline void fs_vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline i32x8 fs_join(u32x4 lo, u32x4 hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// The product of a block's 64 weight rows with the rows' codes, scale block by
// scale block.  ready(kb) returns once scale block kb's weight codes, row codes
// and row scales are in LDS for every wave; wscale(kb) is the weight scale of
// the block's rows in scale block kb.  Wave w owns weight rows 32 (w % 2) ..
// +32 and the 32-row blocks w / 2, w / 2 + 2, ... of the rows.  On return the
// accumulators are in units of ref[t].
template <int MB, int ABYTES, int SA_LD, class Ready, class WScale>
__device__ inline void fs_product(f32x16 (&acc)[(MB + 1) / 2], float (&ref)[(MB + 1) / 2],
                                  const char (*wq)[FS_W_BYTES], const char (*aq)[ABYTES],
                                  const float (*sa)[SA_LD], Ready ready, WScale wscale, int wave, int lane)
{
    constexpr int NTM = (MB + 1) / 2;        // row blocks of wave 0 / 1 (waves 2 / 3 may have one fewer)
    const int wb = wave & 1, j0 = wave >> 1;
    const int nt = (MB - j0 + 1) / 2;
    const int frow = lane & 31;
    int fr_off[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fr_off[kk][h] = frow * FS_ROWB + (((4 * kk + 2 * (lane >> 5) + h) ^ ((frow >> 1) & 7)) * 16);

#pragma unroll
    for (int t = 0; t < NTM; ++t) {
        acc[t] = f32x16{};
        ref[t] = 0.0f;
    }
#pragma unroll
    for (int kb = 0; kb < FS_KB; ++kb) {
        ready(kb);
        const float sw = wscale(kb);
        const bool skip = sw == 0.0f;
        const int e8 = skip ? 0 : 127;
        float rho[NTM];
        int e8a[NTM];
#pragma unroll
        for (int t = 0; t < NTM; ++t) {
            const float sig = sa[kb][32 * (j0 + 2 * t) + frow] * sw;
            // A zero (or subnormal) scale: the row's block adds nothing and
            // the accumulators keep their scale.
            const bool dead = skip || __builtin_fabsf(sig) < 1.17549435e-38f;
            const float r = ref[t] * __builtin_amdgcn_rcpf(sig);
            rho[t] = dead ? 1.0f : (ref[t] == 0.0f ? 0.0f : r);
            ref[t] = dead ? ref[t] : sig;
            e8a[t] = dead ? 0 : 127;
        }
        const char* ws = wq[kb] + wb * 32 * FS_ROWB;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const i32x8 fw = fs_join(lds_ld16(ws + fr_off[kk][0]), lds_ld16(ws + fr_off[kk][1]));
#pragma unroll
            for (int t = 0; t < NTM; ++t) {
                if (t < nt) {
                    const char* as = aq[kb] + (j0 + 2 * t) * 32 * FS_ROWB;
                    const i32x8 fa = fs_join(lds_ld16(as + fr_off[kk][0]), lds_ld16(as + fr_off[kk][1]));
                    if (kk == 0 && kb > 0) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[t][e] *= rho[t];
                    }
                    acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw, fa, acc[t], 0, 0, 0, e8, 0, e8a[t]);
                }
            }
        }
    }
}

// The outputs through LDS (stg: 32 MB rows of 128 bytes that no wave reads any
// more once every wave is past the barrier here): lane l holds row
// 32 j + l % 32, columns 32 wb + 8 q + 4 (l / 32) .. +3 (q < 4) of the block's
// 64; then each store writes whole 128-byte row segments.
template <int MB>
__device__ inline void fs_store(const f32x16 (&acc)[(MB + 1) / 2], const float (&ref)[(MB + 1) / 2], char* stg,
                                const DecompressArgs& a, int n0, int wave, int lane)
{
    constexpr int NTM = (MB + 1) / 2;
    const int wb = wave & 1, j0 = wave >> 1;
    const int nt = (MB - j0 + 1) / 2;
    const int frow = lane & 31, lrow = lane >> 3;
    const int M = a.M;
    lds_barrier();
#pragma unroll
    for (int t = 0; t < NTM; ++t) {
        if (t < nt) {
            const int m = 32 * (j0 + 2 * t) + frow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v = {pack_bf16x2(acc[t][4 * q] * ref[t], acc[t][4 * q + 1] * ref[t]),
                                 pack_bf16x2(acc[t][4 * q + 2] * ref[t], acc[t][4 * q + 3] * ref[t])};
                lds_st8(stg + m * FS_ROWB + swz(m, 4 * wb + q, 8) * 16 + (lane >> 5) * 8, v);
            }
        }
    }
    lds_barrier();
    const rsrc_t cr = make_rsrc(a.out, (uint32_t)((int64_t)M * a.N * 2));
    for (int s = wave; s * 8 < M; s += FS_WAVES) {
        const int m = 8 * s + lrow, g = lane & 7;
        const u32x4 v = lds_ld16(stg + m * FS_ROWB + swz(m, g, 8) * 16);
        const uint32_t off = m < M ? (uint32_t)((m * a.N + n0 + 8 * g) * 2) : kOutOfRange;
        buf_st16_nt(cr, v, off, 0);
    }
}

template <int MB>
__global__ void __launch_bounds__(FS_NT, 1) decompress_small_fp8(DecompressArgs a)
{
    using C = FsCfg<MB>;
    constexpr int ROWS = C::ROWS;
    __shared__ __attribute__((aligned(1024))) char wq[FS_KB][FS_W_BYTES];
    __shared__ __attribute__((aligned(1024))) char aq[FS_KB][C::A_BYTES];
    __shared__ __attribute__((aligned(256))) float sa[FS_KB][64 * FS_WAVES];
    __shared__ __attribute__((aligned(256))) float swc[FS_KB][FS_WAVES][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * FS_N;
    const int M = a.M;

    // 1. Every load of the block, scale block by scale block.  A 1 KB chunk is
    //    8 rows of 128 bytes: lane l fills row l / 8 at granule position l % 8,
    //    which holds logical granule (l % 8) ^ ((row / 2) % 8).
    const int lrow = lane >> 3;
    const i32x4 wr = make_srd(static_cast<const uint8_t*>(a.W) + (int64_t)n0 * FS_K, (uint32_t)(FS_N * FS_K));
    const i32x4 ar = make_srd(a.q, (uint32_t)((int64_t)M * a.q_ld));
    const i32x4 sar = make_srd(a.q_scale, (uint32_t)((int64_t)M * a.qs_ld * 4));
    const i32x4 swr = make_srd(a.W_scale, (uint32_t)((a.N / 128) * FS_KB * 4));
    auto voff = [&](int chunk, int stride) __attribute__((always_inline)) {
        const int r = 8 * chunk + lrow;
        const int g = (lane & 7) ^ ((r >> 1) & 7);
        return (uint32_t)(r * stride + g * 16);
    };
#pragma unroll
    for (int kb = 0; kb < FS_KB; ++kb) {
#pragma unroll
        for (int i = 0; i < FS_W_CHUNKS_PER_WAVE; ++i) {
            const int c = wave * FS_W_CHUNKS_PER_WAVE + i;
            asm_ld16_lds(wr, lds_addr(wq[kb]) + c * 1024, voff(c, FS_K), (uint32_t)(kb * FS_ROWB));
        }
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS_PER_WAVE; ++i) {
            const int c = wave * C::A_CHUNKS_PER_WAVE + i;
            asm_ld16_lds(ar, lds_addr(aq[kb]) + c * 1024, voff(c, a.q_ld), (uint32_t)(kb * FS_ROWB));
        }
        asm_ld4_lds(sar, lds_addr(sa[kb]) + wave * 256, (uint32_t)((wave * 64 + lane) * a.qs_ld * 4),
                    (uint32_t)(kb * 4));
        asm_ld4_lds(swr, lds_addr(swc[kb][wave]), 0u, (uint32_t)(((n0 >> 7) * FS_KB + kb) * 4));
    }

    // 2. The product, each scale block once its loads have landed, then the
    //    outputs (staged in the first scale block's row codes, read by then).
    constexpr int NTM = (MB + 1) / 2;
    f32x16 acc[NTM];
    float ref[NTM];
    auto ready = [&](int kb) __attribute__((always_inline)) {
        switch (kb) {
        case 0: fs_vm_wait<3 * C::LOADS>(); break;
        case 1: fs_vm_wait<2 * C::LOADS>(); break;
        case 2: fs_vm_wait<1 * C::LOADS>(); break;
        default: fs_vm_wait<0>(); break;
        }
        lds_barrier();
    };
    auto wscale = [&](int kb) __attribute__((always_inline)) { return swc[kb][0][lane]; };
    fs_product<MB>(acc, ref, wq, aq, sa, ready, wscale, wave, lane);
    fs_store<MB>(acc, ref, aq[0], a, n0, wave, lane);
}

// ---------------------------------------------------------------------------
// At most 64 rows from a bf16 cache: the gather, the quantisation and the
// product in one launch.  The quantising gather would otherwise be a launch of
// its own, whose chain of index loads (offsets, page table, rows) runs while
// no weight is in flight; here the weight streams in under it.
//  * wave 3 resolves the rows' cache addresses into a table in LDS, as the
//    bf16 few-rows kernel does: one lane per request reads its offsets, and a
//    page table of at most FG_PT_MAX entries is first copied whole into LDS
//    (the rows' area, unused until then), so the page lookups are LDS reads;
//  * waves 0..2 put the first E scale blocks of the block's 32 KB
//    weight share in flight once the first index loads have gone out (a CU
//    serves its waves' vector loads in issue order); once the row table is
//    built, the rows' first 512 columns (four rows of 256 bytes per
//    instruction, scale block by scale block), then the rest of the weight,
//    which streams in while the rows are quantised;
//  * wave 3 meanwhile copies the block's own rows (r % grid == block) whole
//    into k_latent_buffer, through registers;
//  * every block quantises all the rows in LDS exactly as the quantising
//    gather does (amax over 128 columns, s = amax / 448, codes =
//    e4m3(x * (448 / amax)), binary32, round to nearest even; an all-zero
//    block takes s = 1), one 16-lane group per row and scale block, with one
//    pair of divisions per lane whose results the group's lanes take by DPP
//    row broadcast; wave 3 writes its own rows' codes and scales to the
//    workspace;
//  * then the product and the outputs as in decompress_small_fp8.
// Rows past M take row M - 1's address: loaded and quantised, never stored.
constexpr int FG_MAX_ROWS = 64;
constexpr int FG_XS_BYTES = FG_MAX_ROWS * FS_K * 2;   // the rows' first 512 columns, bf16
constexpr int FG_PT_MAX = FG_XS_BYTES / 4;            // page-table entries copied into LDS
// Weight scale blocks issued before the rows: half for at most 32 rows, all of
// them above (measured: 6.05 against 6.3 us per call at 4 rows, 8.55 against
// 8.86 us at 64).
template <int MB>
constexpr int fg_early_kb() { return MB == 1 ? 2 : 4; }
constexpr int FG_W_CHUNKS = FS_KB * FS_W_BYTES / 1024;

// Weight chunks t in [8 E, FG_W_CHUNKS) that wave w (0..2) issues after its
// rows: t % 3 == w.
template <int E, int W>
constexpr int fg_late_chunks()
{
    int n = 0;
    for (int t = 8 * E; t < FG_W_CHUNKS; ++t)
        n += t % 3 == W;
    return n;
}

// Maximum over each 16-lane group of values that are >= 0 and not NaN, on
// their bit patterns (for such floats the integer order is the float order):
// one DPP maximum per step, where a float maximum also canonicalises its
// operand first.
__device__ inline float fg_max16_nonneg(float v)
{
    int x = __float_as_int(v);
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));    // quad_perm [1, 0, 3, 2]
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));    // quad_perm [2, 3, 0, 1]
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true));   // row_half_mirror
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true));   // row_mirror
    return __int_as_float(x);
}

// Four floats -> four e4m3fn codes in one dword (hardware conversion, round
// to nearest even): the second pair is converted straight into the high half.
__device__ inline uint32_t fg_e4m3x4(float a, float b, float c, float d)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int MB, bool CACHE8>
__device__ inline void fg_body(const DecompressArgs& a)
{
    constexpr int ROWS = 32 * MB;
    constexpr int RB = ROWS * 256;            // one scale block of every row, bf16
    constexpr int NP = ROWS / 16;             // rows per 16-lane group and scale block
    constexpr int NU = FS_KB * NP;            // (row, scale block) units per 16-lane group
    constexpr int E = fg_early_kb<MB>();
    static_assert(NU <= 16, "one division pair per lane");
    __shared__ __attribute__((aligned(1024))) char wq[FS_KB][FS_W_BYTES];
    __shared__ __attribute__((aligned(1024))) char aq[FS_KB][ROWS * FS_ROWB];
    __shared__ __attribute__((aligned(1024))) char xs[FG_XS_BYTES];
    __shared__ __attribute__((aligned(256))) float sa[FS_KB][ROWS];
    __shared__ __attribute__((aligned(16))) uint64_t rowaddr[ROWS];
    __shared__ __attribute__((aligned(16))) uint64_t scaleaddr[ROWS];   // e4m3 cache: the rows' scales
    __shared__ uint32_t row_req[ROWS], row_pos[ROWS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * FS_N;
    const int M = a.M;
    const int grid = gridDim.x;
    const PagedLayer& L = a.L;
    const uint32_t pt_entries = L.batch * L.max_pages;
    const bool pt_staged = (uint64_t)L.batch * L.max_pages <= (uint64_t)FG_PT_MAX;

    // Weight chunk t = 8 kb + c (1 KB: tile rows 8 c .. 8 c + 7 of scale
    // block kb, granules swizzled as the product reads them).
    const i32x4 wr = make_srd(static_cast<const uint8_t*>(a.W) + (int64_t)n0 * FS_K, (uint32_t)(FS_N * FS_K));
    auto issue_w = [&](int t) __attribute__((always_inline)) {
        const int kb = t >> 3, c = t & 7;
        const int r = 8 * c + (lane >> 3);
        const uint32_t voff = (uint32_t)(r * FS_K + (((lane & 7) ^ ((r >> 1) & 7)) * 16));
        asm_ld16_lds(wr, lds_addr(wq[kb]) + c * 1024, voff, (uint32_t)(kb * FS_ROWB));
    };

    // 1. Index loads (wave 3) first, the weight (waves 0..2) after them.
    uint32_t lo = 0, c0 = 0, last = 0;
    auto load_round = [&](uint32_t b0) __attribute__((always_inline)) {
        const uint32_t b = b0 + lane;
        const uint32_t bc = b < L.batch ? b : L.batch - 1;
        const uint32_t bend = b0 + 64 < L.batch ? b0 + 64 : L.batch;
        lo = a.bro[bc];
        c0 = a.co[bc];
        last = a.bro[bend];
    };
    if (wave == 3) {
        if (pt_staged) {
            const i32x4 ptr = make_srd(L.page_table, pt_entries * 4);
            for (uint32_t c = 0; c < (pt_entries * 4 + 1023) / 1024; ++c)
                asm_ld16_lds(ptr, lds_addr(xs) + c * 1024, (uint32_t)lane * 16, c * 1024);
        }
        load_round(0);
        asm volatile("s_barrier" ::: "memory");
        for (int r = lane; r < ROWS; r += 64)
            row_req[r] = ~0u;
        for (uint32_t b0 = 0;;) {
            // One use of all three here keeps the compiler from sinking a
            // load into the branch that needs it.
            asm volatile("" : "+v"(lo), "+v"(c0), "+v"(last));
            const uint32_t b = b0 + lane;
            const uint32_t next = (uint32_t)__shfl_down((int)lo, 1);
            const uint32_t hi0 = lane == 63 || b + 1 >= L.batch ? last : next;
            const uint32_t hi = b >= L.batch ? lo : hi0 < (uint32_t)M ? hi0 : (uint32_t)M;
            for (uint32_t r = lo; r < hi; ++r) {
                row_req[r] = b;
                row_pos[r] = c0 + (r - lo);
            }
            b0 += 64;
            if (b0 >= L.batch)
                break;
            load_round(b0);
        }
        // The page table's copy (older than the offsets' loads) has landed.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        const int r = lane;
        if (r < ROWS) {
            const int re = r < M ? r : M - 1;
            const uint32_t b = row_req[re];
            const bool valid = b != ~0u;
            const uint32_t pos = valid ? row_pos[re] : 0u, bb = valid ? b : 0u;
            uint32_t lp = pos / L.page_size;
            const uint32_t slot = pos - lp * L.page_size;
            lp = lp < L.max_pages ? lp : L.max_pages - 1;
            const size_t e = (size_t)bb * L.max_pages + lp;
            const uint32_t pgv = pt_staged ? reinterpret_cast<const uint32_t*>(xs)[e] : L.page_table[e];
            const uint32_t pg = pgv < L.num_pages ? pgv : L.num_pages - 1;
            const int64_t off = valid ? (int64_t)pg * L.stride_page + (int64_t)slot * L.stride_token : 0;
            rowaddr[r] = (uint64_t)(L.base + off);
            if constexpr (CACHE8) {
                const int64_t soff = valid ? (int64_t)pg * a.Ls.stride_page + (int64_t)slot * a.Ls.stride_token : 0;
                scaleaddr[r] = (uint64_t)(a.Ls.base + soff);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        asm volatile("s_barrier" ::: "memory");
        // The first E scale blocks of the weight; the rest goes out behind
        // the rows, so the rows land (and are quantised) while it streams in.
        for (int t = wave; t < 8 * E; t += 3)
            issue_w(t);
    }
    lds_barrier();              // row table written; the page table's copy read

    // 2. The rows (waves 0..2; instruction t = (ROWS / 4) kb + c: rows
    //    4 c .. 4 c + 3, 256 bytes of scale block kb each), and wave 3's
    //    k_latent_buffer copies.
    if (wave < 3) {
        if constexpr (CACHE8) {
            // e4m3 rows: the codes straight into the product's layout
            // (instruction t = (ROWS / 8) kb + c: rows 8 c .. 8 c + 7, lane l
            // filling position l % 8 of row 8 c + l / 8 with its logical
            // granule (l % 8) ^ ((row / 2) % 8) of scale block kb).
            for (int t = wave; t < FS_KB * (ROWS / 8); t += 3) {
                const int kb = t / (ROWS / 8), c = t - kb * (ROWS / 8);
                const int r = 8 * c + (lane >> 3);
                const int g = (lane & 7) ^ ((r >> 1) & 7);
                const char* src = reinterpret_cast<const char*>(rowaddr[r]) + kb * FS_ROWB + g * 16;
                asm_gld16_lds(src, lds_addr(aq[kb]) + c * 1024);
            }
        } else {
            for (int t = wave; t < FS_KB * (ROWS / 4); t += 3) {
                const int kb = t / (ROWS / 4), c = t - kb * (ROWS / 4);
                const int r = 4 * c + (lane >> 4);
                const char* src = reinterpret_cast<const char*>(rowaddr[r]) + kb * 256 + (lane & 15) * 16;
                asm_gld16_lds(src, lds_addr(xs) + kb * RB + c * 1024);
            }
        }
        const int t0 = 8 * E + (wave - 8 * E % 3 + 3) % 3;
        for (int t = t0; t < FG_W_CHUNKS; t += 3)
            issue_w(t);
        // This wave's rows have landed (its later weight chunks may not have).
        switch (wave) {
        case 0: fs_vm_wait<fg_late_chunks<E, 0>()>(); break;
        case 1: fs_vm_wait<fg_late_chunks<E, 1>()>(); break;
        default: fs_vm_wait<fg_late_chunks<E, 2>()>(); break;
        }
    } else {
        constexpr int EB = CACHE8 ? 1 : 2;       // bytes per cache element
        if constexpr (CACHE8) {
            // The rows' scales of the first K columns, one row per lane.
            if (lane < ROWS) {
                const float* sp = reinterpret_cast<const float*>(scaleaddr[lane]);
#pragma unroll
                for (int kb = 0; kb < FS_KB; ++kb)
                    sa[kb][lane] = sp[kb];
            }
        }
        const int gpr = a.D * EB / 16;           // 16-byte granules per cache row
        for (int r = blockIdx.x; r < M; r += grid) {
            const char* src = reinterpret_cast<const char*>(rowaddr[r]);
            char* dst = static_cast<char*>(a.lat) + (int64_t)r * a.D * EB;
            for (int g = lane; g < gpr; g += 64)
                st16(dst + g * 16, ld16(src + g * 16));
            if constexpr (CACHE8) {
                const float* sp = reinterpret_cast<const float*>(scaleaddr[r]);
                for (int j = lane; j < a.nblk; j += 64)
                    a.lat_scale[(int64_t)r * a.nblk + j] = sp[j];
            }
        }
    }
    lds_barrier();

    if constexpr (!CACHE8) {
        // 3. Quantisation: lanes 16 k .. 16 k + 15 of wave w hold row
        //    16 p + 4 w + k of scale block kb, 8 values each.
        const int lg = lane & 15, lr = lane >> 4;
        u32x4 qv[FS_KB][NP];
#pragma unroll
        for (int kb = 0; kb < FS_KB; ++kb)
#pragma unroll
            for (int p = 0; p < NP; ++p)
                qv[kb][p] = lds_ld16(xs + kb * RB + (16 * p + 4 * wave + lr) * 256 + lg * 16);
        float my_am = 0.0f;
#pragma unroll
        for (int kb = 0; kb < FS_KB; ++kb)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const u32x4 v = qv[kb][p];
                // am starts at 0 and fmaxf passes over NaN: am >= 0, not NaN.
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    am = fmaxf(am, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
                am = fg_max16_nonneg(am);
                my_am = lg % NU == kb * NP + p ? am : my_am;
            }
        float my_s = 1.0f, my_inv = 1.0f;
        if (my_am > 0.0f) {
            my_s = my_am / 448.0f;
            my_inv = 448.0f / my_am;
        }
#pragma unroll
        for (int kb = 0; kb < FS_KB; ++kb)
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int r = 16 * p + 4 * wave + lr;
                const u32x4 v = qv[kb][p];
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = bf16_lo(v[i]);
                    x[2 * i + 1] = bf16_hi(v[i]);
                }
                const float inv = row16_lane(my_inv, kb * NP + p);
                const u32x2 codes = {fg_e4m3x4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv),
                                     fg_e4m3x4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv)};
                lds_st8(aq[kb] + r * FS_ROWB + (((lg >> 1) ^ ((r >> 1) & 7)) * 16) + (lg & 1) * 8, codes);
                const float sq = row16_lane(my_s, kb * NP + p);
                if (lg == 0)
                    sa[kb][r] = sq;
            }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);       // the rest of the weight has landed
    lds_barrier();

    // Wave 3: its own rows' codes and scales into the workspace.
    if (!CACHE8 && wave == 3) {
        for (int r = blockIdx.x; r < M; r += grid) {
            if (lane < 32) {
                const int kb = lane >> 3, g = lane & 7;
                const u32x4 v = lds_ld16(aq[kb] + r * FS_ROWB + ((g ^ ((r >> 1) & 7)) * 16));
                st16(static_cast<uint8_t*>(a.q) + (int64_t)r * FS_K + kb * FS_ROWB + g * 16, v);
            }
            if (lane < FS_KB)
                a.q_scale[(int64_t)r * FS_KB + lane] = sa[lane][r];
        }
    }

    // 4. The product (everything is in LDS) and the outputs, staged in the
    //    rows' area.
    constexpr int NTM = (MB + 1) / 2;
    f32x16 acc[NTM];
    float ref[NTM];
    const float* ws_row = a.W_scale + (n0 >> 7) * FS_KB;
    auto ready = [](int) __attribute__((always_inline)) {};
    auto wscale = [&](int kb) __attribute__((always_inline)) { return ws_row[kb]; };
    fs_product<MB>(acc, ref, wq, aq, sa, ready, wscale, wave, lane);
    fs_store<MB>(acc, ref, xs, a, n0, wave, lane);
}

template <int MB>
__global__ void __launch_bounds__(FS_NT, 1) decompress_small_fp8_gq(DecompressArgs a)
{
    fg_body<MB, false>(a);
}

// The same call on an e4m3 cache: the rows' codes go straight into the
// product's layout and their scales into LDS (no quantisation); block b
// copies rows b, b + grid, ... and their scales into k_latent_buffer and
// k_latent_scales.
template <int MB>
__global__ void __launch_bounds__(FS_NT, 1) decompress_small_fp8_gc(DecompressArgs a)
{
    fg_body<MB, true>(a);
}

}  // namespace

bool small_fp8_fits(const DecompressArgs& a)
{
    return a.M >= 1 && a.M <= 32 * FS_MAX_MB && a.K == FS_K && a.N % 128 == 0 && a.N2 == 0;
}

// a.q / a.q_scale (row strides a.q_ld bytes and a.qs_ld floats; 0: the
// workspace's own K and K / 128): the activation codes and scales of the M rows.
hipError_t launch_small_fp8(const DecompressArgs& args, hipStream_t s)
{
    DecompressArgs a = args;
    a.q_ld = a.q_ld ? a.q_ld : a.K;
    a.qs_ld = a.qs_ld ? a.qs_ld : a.K / 128;
    const dim3 grid(a.N / FS_N), block(FS_NT);
    const int mb = (a.M + 31) / 32;
    log_launch("decompress_small_fp8", grid.x, block.x, "M=%d N=%d K=%d row_blocks=%d", a.M, a.N, a.K, mb);
    switch (mb) {
    case 1: hipLaunchKernelGGL(decompress_small_fp8<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(decompress_small_fp8<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(decompress_small_fp8<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(decompress_small_fp8<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(decompress_small_fp8<5>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(decompress_small_fp8<6>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

bool small_fp8_gq_fits(const DecompressArgs& a)
{
    return a.M >= 1 && a.M <= FG_MAX_ROWS && a.K == FS_K && a.N % 128 == 0 && a.N2 == 0 && a.D % 8 == 0 &&
           a.D >= FS_K;
}

// The rows from the bf16 cache; codes and scales to a.q / a.q_scale (row
// strides K and K / 128), k_latent_buffer and k_buffer written.
hipError_t launch_small_fp8_gq(const DecompressArgs& a, hipStream_t s)
{
    const dim3 grid(a.N / FS_N), block(FS_NT);
    log_launch("decompress_small_fp8_gq", grid.x, block.x, "M=%d N=%d K=%d D=%d", a.M, a.N, a.K, a.D);
    if (a.M <= 32)
        hipLaunchKernelGGL(decompress_small_fp8_gq<1>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(decompress_small_fp8_gq<2>, grid, block, 0, s, a);
    return hipGetLastError();
}

bool small_fp8_gc_fits(const DecompressArgs& a)
{
    return a.M >= 1 && a.M <= FG_MAX_ROWS && a.K == FS_K && a.N % 128 == 0 && a.N2 == 0 && a.D % 16 == 0 &&
           a.D >= FS_K && a.lat_scale != nullptr && a.nblk >= FS_KB;
}

// The rows' codes and scales from the e4m3 cache (a.L, a.Ls); k_latent_buffer,
// k_latent_scales and k_buffer written.
hipError_t launch_small_fp8_gc(const DecompressArgs& a, hipStream_t s)
{
    const dim3 grid(a.N / FS_N), block(FS_NT);
    log_launch("decompress_small_fp8_gc", grid.x, block.x, "M=%d N=%d K=%d D=%d", a.M, a.N, a.K, a.D);
    if (a.M <= 32)
        hipLaunchKernelGGL(decompress_small_fp8_gc<1>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(decompress_small_fp8_gc<2>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
