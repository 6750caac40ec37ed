// Decompress for few rows (decode-sized calls: a handful of new tokens per
// request), bf16, kv_lora_rank 512 (page "generic_flare_mla_decompress_k_cache_ragged_paged",
// summary and Args; weight [num_heads*qk_nope_head_dim, kv_latent_dim] from page
// "mla_prefill_decode_graph_fp8", Args w_k).
//
// With M <= 256 rows the call is bound by reading the weight (N x 512 bf16,
// 16 MiB at N = 16384) once from HBM, so the whole weight must be in flight at
// once and the call must be one launch.  One block of 4 waves per 64 weight
// rows (256 blocks at N = 16384, one per CU):
//  * waves 1..3 put the block's 64 x 512 weight tile (64 KB) in flight first,
//    while wave 0 resolves the rows' cache addresses (one lane per request:
//    its offsets, then the page-table entries of its rows; gathering form);
//  * then the rows' first 512 columns, 64 columns (128 bytes) per chunk, go
//    straight into LDS (loads with an LDS destination: the weight as a buffer,
//    the rows by per-lane addresses, 8 rows of 128 bytes per load).  As many
//    row chunks as fit (all 8 for 64 rows, 3 for 256) are in flight together;
//    the rest follow as chunks are consumed;
//  * v_mfma_f32_32x32x16_bf16 with the weight as the row operand: wave w owns
//    weight rows 32 (w % 2) .. +32 and the 32-row blocks w/2, w/2 + 2, ... of
//    the M rows; outputs go straight to k_buffer (4 consecutive columns per
//    lane);
//  * in the gathering form, block b finally copies rows b, b + grid, ... into
//    k_latent_buffer (whole cache rows), by the lanes that loaded them.
// All loads into LDS are issued from inline assembly and ordered by explicit
// waits and barriers (the compiler adds none of its own for them).
#include "launch.hpp"

namespace mla {
namespace {

constexpr int SBN = 64, SNT = 256, SK = 512, SMAX_M = 256;
constexpr int W_BYTES = SBN * SK * 2;            // 64 KB weight tile, rows of 1 KB
constexpr int CHUNK_K = 64, CHUNKS = SK / CHUNK_K, CROWB = CHUNK_K * 2;
constexpr int A_AREA = 96 * 1024;                // row chunks (and, first, the row table)

template <int MB>
struct SmallCfg {
    static constexpr int ROWS = 32 * MB;                         // rows loaded (M rounded up)
    static constexpr int CHUNK_BYTES = ROWS * CROWB;
    static constexpr int SLOTS = (A_AREA / CHUNK_BYTES) < CHUNKS ? (A_AREA / CHUNK_BYTES) : CHUNKS;
    static constexpr int LOADS_PER_CHUNK = ROWS / 8 / 4;         // per wave (8 rows per load, 4 waves)
    static_assert(SLOTS >= 2 && LOADS_PER_CHUNK >= 1 && ROWS % 32 == 0, "chunk ring");
    static_assert(W_BYTES + A_AREA <= 163840 && SMAX_M * 8 <= CHUNK_BYTES * SLOTS, "LDS budget");
};

// s_waitcnt vmcnt(n) for a value known only after unrolling.
__device__ inline void vm_wait(int n)
{
    switch (n) {
#define MLA_VMW(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        MLA_VMW(1) MLA_VMW(2) MLA_VMW(3) MLA_VMW(4) MLA_VMW(5) MLA_VMW(6) MLA_VMW(7) MLA_VMW(8)
        MLA_VMW(9) MLA_VMW(10) MLA_VMW(11) MLA_VMW(12) MLA_VMW(14) MLA_VMW(15) MLA_VMW(16)
        MLA_VMW(18) MLA_VMW(20) MLA_VMW(21) MLA_VMW(24)
#undef MLA_VMW
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

template <int MB>
__global__ void __launch_bounds__(SNT, 1) decompress_small_bf16(DecompressArgs a, int gather)
{
    using C = SmallCfg<MB>;
    constexpr int SLOTS = C::SLOTS, LPC = C::LOADS_PER_CHUNK;
    __shared__ __attribute__((aligned(1024))) char wt[W_BYTES];
    __shared__ __attribute__((aligned(1024))) char at[A_AREA];
    // The row table lives at the start of the chunk area until every lane has
    // copied the addresses it loads from into registers.
    uint64_t* rowaddr = reinterpret_cast<uint64_t*>(at);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * SBN;
    const int M = a.M;

    // 1. The weight tile does not depend on the rows: waves 1..3 put all of it
    //    in flight first (row c is one 1 KB load; lane l fills physical granule
    //    l, which holds logical granule l ^ (c % 16)), while wave 0 resolves the
    //    rows.  Wave 0 issues none of these loads, so the waits the compiler
    //    puts on its index loads do not wait for the weight.
    const uint32_t wt_lds = lds_addr(wt), at_lds = lds_addr(at);
    if (wave > 0) {
        const i32x4 wr = make_srd(a.W, (uint32_t)((int64_t)a.N * SK * 2));
        for (int c = wave - 1; c < SBN; c += 3)
            asm_ld16_lds(wr, wt_lds + c * 1024, (uint32_t)((lane ^ (c & 15)) * 16), (uint32_t)((n0 + c) * SK * 2));
    }

    // 2. Row addresses (wave 0): the first columns of row r start at
    //    rowaddr[r]; rows M .. ROWS-1 repeat row M-1 (loaded, never stored).
    if (wave > 0) {
    } else if (gather) {
        for (uint32_t b = lane; b < a.L.batch; b += 64) {
            const uint32_t lo = a.bro[b], hi0 = a.bro[b + 1], c0 = a.co[b];
            const uint32_t hi = hi0 < (uint32_t)M ? hi0 : (uint32_t)M;
            for (uint32_t r = lo; r < hi; ++r)
                rowaddr[r] = (uint64_t)(a.L.base + token_offset(a.L, b, c0 + (r - lo)));
        }
    } else {
        for (int r = lane; r < M; r += 64)
            rowaddr[r] = (uint64_t)(static_cast<const char*>(a.lat) + (int64_t)r * a.D * 2);
    }
    lds_barrier();
    if (tid >= M && tid < C::ROWS)
        rowaddr[tid] = rowaddr[M - 1];
    lds_barrier();

    // Row chunks: chunk q holds columns 64 q .. 64 q + 63 of every row, rows of
    // 128 bytes (8 granules XOR-swizzled by (row / 2) % 8).  A load covers 8
    // rows: lane l takes row 8 i + l / 8, physical granule l % 8.
    const int lrow = lane >> 3, lpos = lane & 7;
    const char* src_row[LPC];
#pragma unroll
    for (int i = 0; i < LPC; ++i) {
        const int r = (wave * LPC + i) * 8 + lrow;
        src_row[i] = reinterpret_cast<const char*>(rowaddr[r]) + (lpos ^ ((r >> 1) & 7)) * 16;
    }
    lds_barrier();
    auto issue_chunk = [&](int q, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const int r8 = (wave * LPC + i) * 8;
            asm_gld16_lds(src_row[i] + q * CROWB, at_lds + slot * C::CHUNK_BYTES + r8 * CROWB);
        }
    };
#pragma unroll
    for (int q = 0; q < SLOTS - 1; ++q)
        issue_chunk(q, q);

    // 3. The product.
    const int nb = wave & 1, mb0 = wave >> 1;
    const int frow = lane & 31, half = lane >> 5;
    const char* wrow = wt + (nb * 32 + frow) * (SK * 2);
    const int wsw = frow & 15;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = f32x16{};

#pragma unroll
    for (int q = 0; q < CHUNKS; ++q) {
        // Chunk q (and, at q = 0, the weight tile) has landed for this thread;
        // younger loads are the chunks issued after it.
        vm_wait((q + SLOTS - 2 < CHUNKS - 1 ? SLOTS - 2 : CHUNKS - 1 - q) * LPC);
        lds_barrier();
        // Everyone is done with chunk q-1: refill its slot.
        if (q + SLOTS - 1 < CHUNKS)
            issue_chunk(q + SLOTS - 1, (q + SLOTS - 1) % SLOTS);
        const char* as = at + (q % SLOTS) * C::CHUNK_BYTES;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int g = q * 8 + 2 * kk + half;     // weight logical granule
            const bf16x8 wf = as_bf16x8(lds_ld16(wrow + (((g & ~15) | ((g & 15) ^ wsw)) * 16)));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (mb0 + 2 * i < MB) {
                    const int r = (mb0 + 2 * i) * 32 + frow;
                    const bf16x8 af = as_bf16x8(lds_ld16(as + r * CROWB + ((2 * kk + half) ^ ((r >> 1) & 7)) * 16));
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc[i], 0, 0, 0);
                }
        }
    }

    // 4. Outputs: lane holds rows 32 mb + frow, columns 8q + 4 half + 0..3.
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = (mb0 + 2 * i) * 32 + frow;
        if (mb0 + 2 * i < MB && m < M) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + nb * 32 + 8 * q + 4 * half;
                const u32x2 v = {pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]),
                                 pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3])};
                *reinterpret_cast<u32x2*>(out + (int64_t)m * a.N + n) = v;
            }
        }
    }

    // 5. Gathering form: this block's rows of k_latent_buffer (rows r with
    //    r % grid == block), whole cache rows.  The 8 lanes that loaded row r
    //    still hold its address; each copies every 8th granule.
    if (gather) {
        const int gpr = a.D * 2 / 16;
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const int r = (wave * LPC + i) * 8 + lrow;
            if (r < M && r % (int)gridDim.x == (int)blockIdx.x) {
                const char* base = src_row[i] - (lpos ^ ((r >> 1) & 7)) * 16;
                char* dst = static_cast<char*>(a.lat) + (int64_t)r * a.D * 2;
                for (int g = lpos; g < gpr; g += 8)
                    st16(dst + g * 16, ld16(base + g * 16));
            }
        }
    }
}

}  // namespace

bool small_bf16_fits(const DecompressArgs& a)
{
    return a.M <= SMAX_M && a.K == SK && a.N % SBN == 0;
}

// gather != 0: rows come from the paged cache and are also written to
// k_latent_buffer; gather == 0: rows are read from k_latent_buffer.
hipError_t launch_small_bf16(const DecompressArgs& a, int gather, hipStream_t s)
{
    const dim3 grid(a.N / SBN), block(SNT);
    switch ((a.M + 31) / 32) {
    case 1: hipLaunchKernelGGL(decompress_small_bf16<1>, grid, block, 0, s, a, gather); break;
    case 2: hipLaunchKernelGGL(decompress_small_bf16<2>, grid, block, 0, s, a, gather); break;
    case 3: hipLaunchKernelGGL(decompress_small_bf16<3>, grid, block, 0, s, a, gather); break;
    case 4: hipLaunchKernelGGL(decompress_small_bf16<4>, grid, block, 0, s, a, gather); break;
    case 5: hipLaunchKernelGGL(decompress_small_bf16<5>, grid, block, 0, s, a, gather); break;
    case 6: hipLaunchKernelGGL(decompress_small_bf16<6>, grid, block, 0, s, a, gather); break;
    case 7: hipLaunchKernelGGL(decompress_small_bf16<7>, grid, block, 0, s, a, gather); break;
    default: hipLaunchKernelGGL(decompress_small_bf16<8>, grid, block, 0, s, a, gather); break;
    }
    return hipGetLastError();
}

}  // namespace mla
