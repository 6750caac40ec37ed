// Decompress for few rows (decode-sized calls: a handful of new tokens per
// request), bf16, kv_lora_rank 512 (page "generic_flare_mla_decompress_k_cache_ragged_paged",
// summary and Args; weight [num_heads*qk_nope_head_dim, kv_latent_dim] from page
// "mla_prefill_decode_graph_fp8", Args w_k).
//
// With M <= 256 rows the call is bound by reading the weight (N x 512 bf16,
// 16 MiB at N = 16384) once from HBM, so the weight must stream in from the
// start, the product must run while it streams in, and the call must be one
// launch.  One block of 8 waves per 64 weight rows (256 blocks at N = 16384,
// one per CU).  The block's 64 x 512 weight tile (64 KB) and the rows' first
// 512 columns go into LDS in K order, in chunks of 64 columns (128-byte row
// pieces; weight chunk q is 8 KB):
//  * at kernel start the compute waves 0..3 put the first weight chunks in
//    flight, chunk after chunk, while wave 4 resolves the rows' cache
//    addresses (one lane per request reads its offsets, then one lane per row
//    of waves 4..7 its page-table entry; a small page table is copied into
//    LDS in the same round of loads as the offsets) into a table in LDS.
//    The weight is the one HBM stream of the call: it starts at once and is
//    not held up by the index loads' round trip;
//  * then waves 4..7 each issue, chunk after chunk, their share of the row
//    chunks (the rows are read by every block, so mostly from L2).  Row
//    chunks that do not fit in LDS at once go through a ring of slots
//    refilled as chunks are consumed (for 129..192 rows the weight chunks
//    after the first few go through the same slots, beside their rows);
//  * waves 0..3 run v_mfma_f32_32x32x16_bf16 on chunk q as soon as its pieces
//    have landed, with the weight as the row operand: up to 160 rows, wave w
//    owns weight rows 32 (w % 2) .. +32 and the 32-row blocks w/2, w/2 + 2, ...
//    of the M rows; above that, both weight blocks and the M blocks w, w + 4
//    (fewer LDS fragment reads per MFMA);
//  * wave 4 also puts this block's share of the k_latent_buffer copy (whole
//    cache rows r with r % grid == block) in flight into registers early and
//    stores it at the end.
// The accumulators go through LDS so that every k_buffer store writes whole
// 128-byte row segments.  Every wave that issued loads of chunk q (the
// compute waves its weight pieces, the loader waves its row pieces) waits for
// them with an explicit vmcnt wait before the chunk's barrier; the
// loads into LDS are issued from inline assembly, so the compiler adds no
// waits of its own for them.
#include "launch.hpp"

namespace mla {
namespace {

constexpr int SBN = 64, SK = 512, SMAX_M = 256;
constexpr int SNT = 512;                         // 8 waves
constexpr int W_BYTES = SBN * SK * 2;            // 64 KB weight tile
constexpr int CHUNK_K = 64, CHUNKS = SK / CHUNK_K, CROWB = CHUNK_K * 2;
constexpr int SLOTS_MAX = 6;                      // row chunks in LDS at once (ring slots)
constexpr int W_CHUNK_BYTES = SBN * CROWB;       // 8 KB: one chunk of the weight tile
constexpr int A_AREA = 96 * 1024;                // row chunks (first the row table, last the output staging)
constexpr int W_PIECES = W_CHUNK_BYTES / 1024;   // 1 KB loads per weight chunk
constexpr int COMPUTE_WAVES = 4, LOADER_WAVES = 4;
constexpr int W_PER_WAVE = W_PIECES / COMPUTE_WAVES;   // weight loads per chunk per wave (either role)
constexpr int EARLY_COPY_ROWS = 2;               // k_latent_buffer rows per block copied through registers
constexpr int EARLY_COPY_GRANULES = 128;         // up to 2048-byte cache rows
constexpr int PT_STAGE_MAX = 16384;              // page tables up to 64 KB are copied into LDS whole
constexpr int ROW_TABLE = A_AREA - SMAX_M * 16;  // row table: rowaddr, row_req, row_pos (4 KB)
constexpr int LDS_BYTES = 160 * 1024;

// vmcnt is a 6-bit counter: a wave never has more than 63 vector memory
// operations outstanding (issue waits instead), so a wait for at most 63
// younger operations is the weakest one needed.
template <int N>
__device__ inline void vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Loads and stores through global (not flat) addresses: pointers read back
// from LDS are generic, and flat accesses would also count against lgkmcnt,
// which every LDS wait here would then wait for.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
__device__ inline u32x4 gld16(const void* p) { return *(const g_u32x4*)p; }
__device__ inline void gst16(void* p, u32x4 v) { *(g_u32x4*)p = v; }

constexpr int cmin(int x, int y) { return x < y ? x : y; }

// LDS layout.  The whole 64 KB weight tile stays in LDS and the row chunks go
// through the remaining 96 KB (at most SLOTS_MAX chunks of rows at once: with
// fewer rows in flight at the start, the first chunks' rows and the weight
// land sooner); or, where that leaves room for fewer chunks of rows than
// LDS could hold with the weight streamed beside them (160 or 192 rows), each
// ring slot holds a chunk of rows and the same chunk of the weight (WRING).
// The rows then have one more chunk in flight: with every block reading the
// same rows, their loads take long to land, and chunks in flight set the
// pace.  Only weight chunks with a free slot can go early, so the streamed
// layout is used only where at least four can (five slots): with three, the
// weight stream starts too thin to cover the index round trip of many rows
// (224 and 256 rows ran 2 % slower streamed than resident).
template <int MB>
struct SmallCfg {
    static constexpr int ROWS = 32 * MB;                         // rows loaded (M rounded up)
    static constexpr int CHUNK_BYTES = ROWS * CROWB;
    static constexpr int FIT_RESIDENT = cmin(A_AREA / CHUNK_BYTES, SLOTS_MAX);
    static constexpr int FIT_STREAMED = cmin(LDS_BYTES / (CHUNK_BYTES + W_CHUNK_BYTES), SLOTS_MAX);
    static constexpr bool WRING = FIT_RESIDENT < CHUNKS && FIT_STREAMED > FIT_RESIDENT && FIT_STREAMED >= 5;
    static constexpr int FIT = WRING ? FIT_STREAMED : FIT_RESIDENT;
    static constexpr bool RING = FIT < CHUNKS;
    static constexpr int SLOTS = RING ? FIT : CHUNKS;
    static constexpr int INITIAL = RING ? SLOTS - 1 : CHUNKS;    // chunks issued before the loop
    static constexpr int WT_BYTES = WRING ? SLOTS * W_CHUNK_BYTES : W_BYTES;
    static constexpr int AT_BYTES = WRING ? SLOTS * CHUNK_BYTES : A_AREA;
    // LDS slot of weight chunk c.
    static constexpr int wslot(int c) { return WRING ? c % SLOTS : c; }
    static_assert(SLOTS >= 2 && ROWS % 32 == 0, "chunk ring");
    static_assert(WT_BYTES + AT_BYTES <= LDS_BYTES && CHUNK_BYTES <= AT_BYTES, "LDS budget");
    static_assert(AT_BYTES >= A_AREA, "the row table and the staged page table fit in the rows' area");
};

// Weight chunks put in flight at kernel start; the later ones go out one per
// row chunk, after it.  Gathering, the rows' addresses are known only after
// the index round trip: enough weight to keep HBM busy over it goes first
// (more for many rows, whose product takes longer to catch up).  Reading
// k_latent_buffer, the rows can go out at once, in K order with the weight.
// With the weight streamed through the ring, only chunks with a free slot
// can go early.
template <int MB, bool GATHER>
constexpr int w_early()
{
    return cmin(GATHER ? (MB <= 3 ? 3 : 5) : 1, SmallCfg<MB>::WRING ? SmallCfg<MB>::INITIAL : CHUNKS);
}
static_assert(PT_STAGE_MAX * 4 <= ROW_TABLE, "the staged page table and the row table do not overlap");
static_assert(W_PIECES % COMPUTE_WAVES == 0 && COMPUTE_WAVES == LOADER_WAVES, "weight loads split evenly");

// Loader wave (each issues, per chunk c, MB row loads and then its share of
// weight chunk c + E; with the weight streamed, of weight chunk c itself when
// c >= E): chunk q's row loads and (q >= E) weight loads must have landed.
// Resident weight with E >= 1: the weight loads of chunk q went out before
// its row loads, so the loads still allowed in flight are the ones issued
// after chunk q's row loads.  Streamed weight, or E = 0: the ones issued
// after chunk q's weight loads.
template <int MB, int E>
constexpr int loads_after(int q)
{
    using C = SmallCfg<MB>;
    const int issued = C::RING ? (C::INITIAL + q < CHUNKS ? C::INITIAL + q : CHUNKS) : CHUNKS;
    if (C::WRING || E == 0) {
        int n = 0;
        for (int c = q + 1; c < issued; ++c)
            n += MB + (c >= E ? W_PER_WAVE : 0);
        return n;
    }
    int n = q + E < CHUNKS ? W_PER_WAVE : 0;
    for (int c = q + 1; c < issued; ++c)
        n += MB + (c + E < CHUNKS ? W_PER_WAVE : 0);
    return n;
}
template <int MB, int E, int Q>
__device__ inline void wait_loads()
{
    vm_wait<loads_after<MB, E>(Q)>();
}

// Compute wave (issued W_PER_WAVE weight loads per chunk of the first E
// chunks, in K order, at kernel start): its share of weight chunk q has
// landed (chunks from E on are the loader waves').
template <int E, int Q>
__device__ inline void wait_weight()
{
    vm_wait<(Q < E ? W_PER_WAVE * (E - 1 - Q) : 0)>();
}

// Waves 0..3: the product, chunk by chunk as the pieces land, then the
// outputs staged in LDS.  A wave owns NBW 32-row blocks of the weight tile
// starting at block nb0 and the 32-row blocks MB0, MB0 + MSTEP, ... of the M
// rows; every weight fragment it reads serves all its M blocks and every row
// fragment all its weight blocks.
template <int MB, int E, int MB0, int MSTEP, int NBW>
__device__ inline void compute_waves(const char* wt, char* at, int nb0, int lane)
{
    using C = SmallCfg<MB>;
    constexpr int SLOTS = C::SLOTS;
    constexpr int NBLK = MB > MB0 ? (MB - MB0 + MSTEP - 1) / MSTEP : 0;   // M blocks of this wave
    // One accumulator per output block.  A wave with a single block runs its
    // MFMAs as one dependent chain: each chunk's four arrive faster than the
    // chunks do, and the chain ends with no partial sums to add (four
    // independent chains summed at the end measured 1-2 % slower).
    const int frow = lane & 31, half = lane >> 5;
    const int rsw = (frow >> 1) & 7;          // granule swizzle of every row this lane reads
    f32x16 acc[NBW][NBLK > 0 ? NBLK : 1];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
            acc[j][i] = f32x16{};
#pragma unroll
    for (int q = 0; q < CHUNKS; ++q) {
        switch (q) {
        case 0: wait_weight<E, 0>(); break;
        case 1: wait_weight<E, 1>(); break;
        case 2: wait_weight<E, 2>(); break;
        case 3: wait_weight<E, 3>(); break;
        case 4: wait_weight<E, 4>(); break;
        case 5: wait_weight<E, 5>(); break;
        case 6: wait_weight<E, 6>(); break;
        default: wait_weight<E, 7>(); break;
        }
        lds_barrier();
        const char* ws = wt + C::wslot(q) * W_CHUNK_BYTES + (nb0 * 32 + frow) * CROWB;
        const char* as = at + (q % SLOTS) * C::CHUNK_BYTES + frow * CROWB;
        // Fragments of k step kk + 1 are read before step kk's MFMAs go out,
        // so the LDS latency is exposed once per chunk (after its barrier),
        // not once per k step.
        bf16x8 wf[2][NBW], af[2][NBLK > 0 ? NBLK : 1];
        auto read_step = [&](int kk, int b) __attribute__((always_inline)) {
            const int g = (2 * kk + half) ^ rsw;
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                wf[b][j] = as_bf16x8(lds_ld16(ws + j * 32 * CROWB + g * 16));
#pragma unroll
            for (int i = 0; i < NBLK; ++i)
                af[b][i] = as_bf16x8(lds_ld16(as + (MB0 + MSTEP * i) * 32 * CROWB + g * 16));
        };
        read_step(0, 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int b = kk & 1;
            if (kk < 3)
                read_step(kk + 1, b ^ 1);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int i = 0; i < NBLK; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b][j], af[b][i], acc[j][i], 0, 0, 0);
        }
        // Keep that order (the scheduler would otherwise put each read right
        // before the MFMA that needs it).
        constexpr int NRD = NBW + (NBLK > 0 ? NBLK : 0), NMF = NBW * NBLK;
        if constexpr (NMF > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
            for (int kk = 0; kk < 3; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
        }
    }
    // Every wave is past its last LDS read of the chunks: stage the outputs.
    // Lane holds rows 32 mb + frow, columns 32 nb + 8 q + 4 half + 0..3 (q < 4).
    lds_barrier();
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
            const int m = (MB0 + MSTEP * i) * 32 + frow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int g = (nb0 + j) * 4 + q;
                const u32x2 v = {pack_bf16x2(acc[j][i][4 * q], acc[j][i][4 * q + 1]),
                                 pack_bf16x2(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3])};
                lds_st8(at + m * CROWB + ((g ^ (m & 7)) * 16) + half * 8, v);
            }
        }
}

template <int MB, bool GATHER>
__global__ void __launch_bounds__(SNT, 1) decompress_small_bf16(DecompressArgs a)
{
    using C = SmallCfg<MB>;
    constexpr bool gather = GATHER;
    constexpr int E = w_early<MB, GATHER>();
    constexpr int SLOTS = C::SLOTS;
    __shared__ __attribute__((aligned(1024))) char wt[C::WT_BYTES];
    __shared__ __attribute__((aligned(1024))) char at[C::AT_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * SBN;
    const int M = a.M;
    const int grid = gridDim.x;
    const uint32_t wt_lds = lds_addr(wt), at_lds = lds_addr(at);
    const int gpr = a.D * 2 / 16;                // 16-byte granules per cache row
    const bool early_copy = gather && gpr <= EARLY_COPY_GRANULES;
    const int lrow = lane >> 3, lpos = lane & 7;
    // The row table (first columns of row r at rowaddr[r]; rows M .. ROWS-1
    // repeat row M-1, loaded and never stored) lives at the end of the row
    // chunks' area until every loader wave has read its rows' addresses.
    char* tbl = at + ROW_TABLE;
    uint64_t* rowaddr = reinterpret_cast<uint64_t*>(tbl);

    // Weight load (c, p): chunk c, tile rows 8 p .. 8 p + 7, one 128-byte row
    // piece per 8 lanes; lane l fills granule position l % 8 of row
    // 8 p + l / 8 with logical granule (l % 8) ^ ((row / 2) % 8).
    const i32x4 wr = make_srd(a.W, (uint32_t)((int64_t)a.N * SK * 2));
    auto issue_w = [&](int c, int p) __attribute__((always_inline)) {
        const int row = 8 * p + lrow;
        const uint32_t voff = (uint32_t)(row * SK * 2 + ((lpos ^ ((row >> 1) & 7)) * 16));
        asm_ld16_lds(wr, wt_lds + C::wslot(c) * W_CHUNK_BYTES + p * 1024, voff, (uint32_t)(n0 * SK * 2 + c * CROWB));
    };

    // 1. Wave 4 resolves the rows' cache addresses into a table in LDS: one
    //    lane per request reads its offsets and writes each of its rows'
    //    request and token position into LDS; then one lane per row (on
    //    waves 4..7) looks up the page-table entry of its row.  A page table of at most
    //    PT_STAGE_MAX entries is copied whole into LDS (the row chunks' area,
    //    unused until the table is built) in the same round of loads as the
    //    offsets, so the lookups are LDS reads: one round of memory latency
    //    instead of two.  Rows no request covers (buffer_row_offsets ending
    //    short of M) read the pool's first row.  The compute waves put the
    //    whole weight tile in flight, chunk after chunk (wave v: pieces
    //    W_PER_WAVE v .. of every chunk), only once the first round of index
    //    loads has been issued: a CU serves its waves' vector loads in issue
    //    order, and the index loads must not wait behind 64 KB of weight.
    uint32_t* row_req = reinterpret_cast<uint32_t*>(tbl + SMAX_M * 8);
    uint32_t* row_pos = row_req + SMAX_M;
    const uint32_t pt_entries = a.L.batch * a.L.max_pages;
    const bool pt_staged = pt_entries <= (uint32_t)PT_STAGE_MAX;
    // Lane b of a round reads buffer_row_offsets[b] and cache_offsets[b]; a
    // request's end is its neighbour lane's start (the last lane's comes from
    // one more, wave-uniform, load).  Every load of a round is issued before
    // any of them is used (indices clamped into the arrays instead of
    // branching around the loads; batch >= 1), so each round costs one memory
    // latency.
    uint32_t lo = 0, c0 = 0, last = 0;
    auto load_round = [&](uint32_t b0) __attribute__((always_inline)) {
        const uint32_t b = b0 + lane;
        const uint32_t bc = b < a.L.batch ? b : a.L.batch - 1;
        const uint32_t bend = b0 + 64 < a.L.batch ? b0 + 64 : a.L.batch;
        lo = a.bro[bc];
        c0 = a.co[bc];
        last = a.bro[bend];
    };
    // The barrier (with no wait before it) only orders the issue of the
    // loads; each side has its own copy so that the compiler's wait pass sees
    // the index loads pending on wave 4's path alone.
    if (wave != 4) {
        asm volatile("s_barrier" ::: "memory");
        if (wave < COMPUTE_WAVES) {
#pragma unroll
            for (int c = 0; c < E; ++c)
#pragma unroll
                for (int j = 0; j < W_PER_WAVE; ++j)
                    issue_w(c, W_PER_WAVE * wave + j);
        }
    } else {
        if (gather) {
            if (pt_staged) {
                const i32x4 ptr = make_srd(a.L.page_table, pt_entries * 4);
                for (uint32_t c = 0; c < (pt_entries * 4 + 1023) / 1024; ++c)
                    asm_ld16_lds(ptr, at_lds + c * 1024, (uint32_t)lane * 16, c * 1024);
            }
            load_round(0);
        }
        asm volatile("s_barrier" ::: "memory");
        if (gather) {
            for (int r = lane; r < C::ROWS; r += 64)
                row_req[r] = ~0u;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            for (uint32_t b0 = 0;;) {
                // One use of all three here keeps the compiler from sinking a
                // load into the branch that needs it (a second round trip).
                asm volatile("" : "+v"(lo), "+v"(c0), "+v"(last));
                const uint32_t b = b0 + lane;
                const uint32_t next = (uint32_t)__shfl_down((int)lo, 1);
                const uint32_t hi0 = lane == 63 || b + 1 >= a.L.batch ? last : next;
                const uint32_t hi = b >= a.L.batch ? lo : hi0 < (uint32_t)M ? hi0 : (uint32_t)M;
                for (uint32_t r = lo; r < hi; ++r) {
                    row_req[r] = b;
                    row_pos[r] = c0 + (r - lo);
                }
                b0 += 64;
                if (b0 >= a.L.batch)
                    break;
                load_round(b0);
            }
        } else {
            for (int r = lane; r < M; r += 64)
                rowaddr[r] = (uint64_t)(static_cast<const char*>(a.lat) + (int64_t)r * a.D * 2);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            for (int r = M + lane; r < C::ROWS; r += 64)
                rowaddr[r] = rowaddr[M - 1];
        }
        // The compiler's own wait (vmcnt(0), known to its wait pass): no load
        // of this branch is left pending where the wave roles' code joins,
        // so no conservative wait lands on the weight waves, whose loads into
        // LDS it cannot see and would wait for too.  Gathering, the page
        // table's copy (loads older than the offsets' ones) has then landed.
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    if (gather) {
        // Every row's request and position, and the page table's copy, are in
        // LDS.  Waves 4..7 look the rows up, one per lane (row 64 (wave - 4) +
        // lane; rows M .. ROWS-1 take row M-1's address), so the division and
        // 64-bit address arithmetic of 256 rows run as one step on four waves
        // instead of four steps on one.
        lds_barrier();
        if (wave >= 4) {
            const int r = 64 * (wave - 4) + lane;
            if (r < C::ROWS) {
                const PagedLayer& L = a.L;
                const int re = r < M ? r : M - 1;
                const uint32_t b = row_req[re];
                const bool valid = b != ~0u;
                const uint32_t pos = valid ? row_pos[re] : 0u, bb = valid ? b : 0u;
                uint32_t lp = pos / L.page_size;
                const uint32_t slot = pos - lp * L.page_size;
                lp = lp < L.max_pages ? lp : L.max_pages - 1;
                const size_t e = (size_t)bb * L.max_pages + lp;
                const uint32_t pgv = pt_staged ? reinterpret_cast<const uint32_t*>(at)[e] : L.page_table[e];
                const uint32_t pg = pgv < L.num_pages ? pgv : L.num_pages - 1;
                const int64_t off = valid ? (int64_t)pg * L.stride_page + (int64_t)slot * L.stride_token : 0;
                rowaddr[r] = (uint64_t)(L.base + off);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    }
    lds_barrier();              // row table written

    // 2. Loader waves 4..7 (w = wave - 4) take the row loads i = w, w + 4, ...
    //    of every chunk (lane l: row 8 i + l / 8, granule position l % 8 with
    //    logical granule (l % 8) ^ ((row / 2) % 8)).
    const int w = wave - 4;
    const char* src_row[MB];
    u32x4 cp[EARLY_COPY_ROWS][2];
    if (wave >= 4) {
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int r = 8 * (w + 4 * k) + lrow;
            src_row[k] = reinterpret_cast<const char*>(rowaddr[r]) + (lpos ^ ((r >> 1) & 7)) * 16;
        }
        // This block's first k_latent_buffer rows (r = block, block + grid):
        // whole cache rows, granules lane and lane + 64, in flight now and
        // stored at the end.
        if (w == 0 && early_copy) {
#pragma unroll
            for (int j = 0; j < EARLY_COPY_ROWS; ++j) {
                const int r = blockIdx.x + j * grid;
                const char* base = reinterpret_cast<const char*>(rowaddr[r < M ? r : M - 1]);
                cp[j][0] = lane < gpr ? gld16(base + lane * 16) : u32x4{};
                cp[j][1] = lane + 64 < gpr ? gld16(base + (lane + 64) * 16) : u32x4{};
            }
        }
    }
    lds_barrier();              // row table read: row chunks may land on it

    if (wave >= 4) {
        // Chunk c: this wave's row loads, then its share of weight chunk
        // c + E (streamed weight: of chunk c, in the same slot), so rows and
        // the rest of the weight arrive in K order.
        auto issue_chunk = [&](int c) __attribute__((always_inline)) {
            const int slot = c % SLOTS;
#pragma unroll
            for (int k = 0; k < MB; ++k)
                asm_gld16_lds(src_row[k] + c * CROWB, at_lds + slot * C::CHUNK_BYTES + (w + 4 * k) * 1024);
            const int cw = C::WRING ? c : c + E;
            if (cw >= E && cw < CHUNKS)
#pragma unroll
                for (int j = 0; j < W_PER_WAVE; ++j)
                    issue_w(cw, W_PER_WAVE * w + j);
        };
#pragma unroll
        for (int c = 0; c < C::INITIAL; ++c)
            issue_chunk(c);
#pragma unroll
        for (int q = 0; q < CHUNKS; ++q) {
            switch (q) {
            case 0: wait_loads<MB, E, 0>(); break;
            case 1: wait_loads<MB, E, 1>(); break;
            case 2: wait_loads<MB, E, 2>(); break;
            case 3: wait_loads<MB, E, 3>(); break;
            case 4: wait_loads<MB, E, 4>(); break;
            case 5: wait_loads<MB, E, 5>(); break;
            case 6: wait_loads<MB, E, 6>(); break;
            default: wait_loads<MB, E, 7>(); break;
            }
            lds_barrier();
            // Every wave is done with chunk q-1: refill its slot.
            if (C::RING && q + SLOTS - 1 < CHUNKS)
                issue_chunk(q + SLOTS - 1);
        }

        // k_latent_buffer: the rows copied through registers, then (few weight
        // tiles, or rows wider than 2 KB) the rest of this block's rows r with
        // r % grid == block, by the 8 lanes that hold r's address.
        if (gather) {
            char* lat = static_cast<char*>(a.lat);
            if (w == 0 && early_copy) {
#pragma unroll
                for (int j = 0; j < EARLY_COPY_ROWS; ++j) {
                    const int r = blockIdx.x + j * grid;
                    if (r < M) {
                        char* dst = lat + (int64_t)r * a.D * 2;
                        if (lane < gpr)
                            gst16(dst + lane * 16, cp[j][0]);
                        if (lane + 64 < gpr)
                            gst16(dst + (lane + 64) * 16, cp[j][1]);
                    }
                }
            }
            const int first = early_copy ? (int)blockIdx.x + EARLY_COPY_ROWS * grid : (int)blockIdx.x;
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const int r = 8 * (w + 4 * k) + lrow;
                if (r < M && r >= first && r % grid == (int)blockIdx.x) {
                    const char* base = src_row[k] - (lpos ^ ((r >> 1) & 7)) * 16;
                    char* dst = lat + (int64_t)r * a.D * 2;
                    for (int g = lpos; g < gpr; g += 8)
                        gst16(dst + g * 16, gld16(base + g * 16));
                }
            }
        }
        lds_barrier();          // matches the compute waves' barrier before staging
    } else if constexpr (MB >= 6) {
        // 3. The product.  Many rows: wave v owns both weight blocks and M
        //    blocks v, v + 4 (one LDS fragment read per MFMA).
        switch (wave) {
        case 0: compute_waves<MB, E, 0, 4, 2>(wt, at, 0, lane); break;
        case 1: compute_waves<MB, E, 1, 4, 2>(wt, at, 0, lane); break;
        case 2: compute_waves<MB, E, 2, 4, 2>(wt, at, 0, lane); break;
        default: compute_waves<MB, E, 3, 4, 2>(wt, at, 0, lane); break;
        }
    } else if (wave < 2) {
        // Few rows: wave v owns weight block v % 2 and M blocks v / 2, v / 2 + 2, ...
        compute_waves<MB, E, 0, 2, 1>(wt, at, wave & 1, lane);
    } else {
        compute_waves<MB, E, 1, 2, 1>(wt, at, wave & 1, lane);
    }
    lds_barrier();              // outputs staged

    // 4. Outputs: each store writes 8 whole 128-byte row segments (lane l: row
    //    8 s + l / 8, granule l % 8).
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int sg = lane & 7;
    for (int s = wave; s * 8 < M; s += SNT / 64) {
        const int m = 8 * s + lrow;
        if (m < M) {
            const u32x4 v = lds_ld16(at + m * CROWB + ((sg ^ (m & 7)) * 16));
            gst16(out + (int64_t)m * a.N + n0 + 8 * sg, v);
        }
    }
}

template <bool GATHER>
void launch_small(const DecompressArgs& a, hipStream_t s)
{
    const dim3 grid(a.N / SBN), block(SNT);
    log_launch(GATHER ? "decompress_small_bf16<gather>" : "decompress_small_bf16<rows>", grid.x, block.x,
               "M=%d N=%d K=%d row_blocks=%d", a.M, a.N, a.K, (a.M + 31) / 32);
    switch ((a.M + 31) / 32) {
    case 1: hipLaunchKernelGGL((decompress_small_bf16<1, GATHER>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decompress_small_bf16<2, GATHER>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decompress_small_bf16<3, GATHER>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decompress_small_bf16<4, GATHER>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((decompress_small_bf16<5, GATHER>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decompress_small_bf16<6, GATHER>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((decompress_small_bf16<7, GATHER>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decompress_small_bf16<8, GATHER>), grid, block, 0, s, a); break;
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
    if (gather)
        launch_small<true>(a, s);
    else
        launch_small<false>(a, s);
    return hipGetLastError();
}

}  // namespace mla
