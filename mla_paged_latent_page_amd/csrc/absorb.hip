// Query absorption (page "mla_prefill_decode_graph_fp8", Args q [tot_seq_len,
// num_heads, qk_nope_head_dim + qk_rope_head_dim] and w_uk [num_heads,
// kv_latent_dim, qk_nope_head_dim], the weight that takes the non-rope part of
// each query head into the KV latent space):
//   out[t][h][c] = bf16( sum_{d < 128} q[t][h][d] * w_uk[h][c][d] ),  c < kv_latent_dim
// in fp32, and, when asked, the rope part q[t][h][128:] copied right after it, so
// that an absorbed query head has the layout of a cache row (latent, then rope).
//
// Bound by HBM: at decode sizes the weight (num_heads * 512 * 128 bf16, 16 MiB)
// and the output dominate.  One block of 4 waves per head and two 128-column
// tiles of the latent columns (one when kv_latent_dim / 128 is odd); the
// blocks of one head are dispatched to the same XCD, next to each other, so
// they read that head's query rows from HBM once and share them in the XCD's
// L2.  Query rows come in chunks of 128 (32 KB) and each weight tile
// (128 x 128, 32 KB) once, all into LDS by loads issued from inline assembly
// with explicit waits, in the order query chunk, tile 0, tile 1: tile 0 is
// computed and stored while tile 1 is still arriving.  v_mfma_f32_32x32x16_bf16
// with the weight as the row operand: wave w owns a tile's latent columns
// 32 w .. 32 w + 31 for all 128 rows of a chunk; the results go through LDS so
// that each store writes whole 256-byte row segments.
#include "launch.hpp"

namespace mla {
namespace {

constexpr int AB_N = 128;            // latent columns per tile
constexpr int AB_K = 128;            // qk_nope_head_dim
constexpr int AB_M = 128;            // query rows per chunk
constexpr int AB_NT = 256;
constexpr int AB_ROWB = AB_K * 2;    // 256-byte tile rows: 16 granules, XOR-swizzled by row % 16
constexpr int AB_ROPE_REGS = 4;      // rope granules per thread held in registers (rope <= 64 columns)

template <int N>
__device__ inline void ab_vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same with a wave-uniform count known at run time (0..8).
__device__ inline void ab_vm_wait_upto8(int n)
{
    switch (n) {
    case 0: ab_vm_wait<0>(); break;
    case 1: ab_vm_wait<1>(); break;
    case 2: ab_vm_wait<2>(); break;
    case 3: ab_vm_wait<3>(); break;
    case 4: ab_vm_wait<4>(); break;
    case 5: ab_vm_wait<5>(); break;
    case 6: ab_vm_wait<6>(); break;
    case 7: ab_vm_wait<7>(); break;
    default: ab_vm_wait<8>(); break;
    }
}

// TPB column tiles of one head per block (2 when the head's tile count is
// even).  Block b runs on XCD b % 8; there its j-th block (j = b / 8) takes
// tiles TPB (j % bph) .. of head (j / bph) * 8 + b % 8, bph = tiles / TPB.
// Per chunk of 128 query rows, each wave's loads go out in the order: rope
// granules (into registers), query chunk, then (first chunk only) weight tile
// 0 and weight tile 1; tile 0 is computed and stored while tile 1's weight is
// still arriving.  Outputs go through LDS so that each store writes whole
// 256-byte row segments.
template <int TPB>
__global__ void __launch_bounds__(AB_NT, 1) absorb_bf16(AbsorbArgs a)
{
    __shared__ __attribute__((aligned(1024))) char wt[TPB][AB_N * AB_ROWB];
    __shared__ __attribute__((aligned(1024))) char at[AB_M * AB_ROWB];
    __shared__ __attribute__((aligned(1024))) char st[AB_M * AB_ROWB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bph = a.NL / AB_N / TPB;
    const int j = (int)(blockIdx.x >> 3);
    const int u = j % bph, h = (j / bph) * 8 + (int)(blockIdx.x & 7);
    if (h >= a.H)
        return;
    const uint32_t at_lds = lds_addr(at);

    // One load moves 4 tile rows: lane l fills physical granule l % 16 of row
    // 4 i + l / 16, which holds logical granule (l % 16) ^ (row % 16).
    const int lr = lane >> 4, lg = lane & 15;
    // Query rows t0 .. t0 + 127 of head h (rows past T read as zeros: their
    // offsets are past the end of the resource).
    const i32x4 qr = make_srd(a.q, (uint32_t)((int64_t)a.T * a.H * a.Dq * 2));
    auto load_chunk = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < AB_M / 16; ++k) {
            const int i = wave + 4 * k, row = 4 * i + lr;
            const uint32_t off = (uint32_t)(((int64_t)(t0 + row) * a.H + h) * a.Dq * 2);
            asm_ld16_lds(qr, at_lds + i * 1024, off + (uint32_t)((lg ^ (row & 15)) * 16), 0u);
        }
    };
    // The rope part (the block with the head's first tiles copies it): R * 2
    // bytes per row, granule idx of the chunk = row idx / gpr, granule idx % gpr.
    const bool rope = a.R > 0 && u == 0;
    const int gpr = a.R > 0 ? a.R / 8 : 1;   // granules per rope row (1 when there is none: a safe divisor)
    u32x4 rp[AB_ROPE_REGS];
    auto load_rope = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < AB_ROPE_REGS; ++k) {
            const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
            if (rope && idx < AB_M * gpr && t0 + r < a.T)
                rp[k] = ld16(a.q + ((int64_t)(t0 + r) * a.H + h) * a.Dq + AB_K + g * 8);
        }
    };

    load_rope(0);
    load_chunk(0);
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
        const i32x4 wr = make_srd(a.w + ((int64_t)h * a.NL + (u * TPB + tt) * AB_N) * AB_K, (uint32_t)(AB_N * AB_ROWB));
        const uint32_t wt_lds = lds_addr(wt[tt]);
#pragma unroll
        for (int k = 0; k < AB_N / 16; ++k) {
            const int i = wave + 4 * k, row = 4 * i + lr;
            asm_ld16_lds(wr, wt_lds + i * 1024, (uint32_t)(row * AB_ROWB + ((lg ^ (row & 15)) * 16)), 0u);
        }
    }

    const int frow = lane & 31, half = lane >> 5;
    uint16_t* out = a.out;
    for (int t0 = 0; t0 < a.T; t0 += AB_M) {
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
            // This wave's loads of the chunk and of weight tile tt have landed;
            // the barrier makes everyone's visible.  vmcnt counts stores too:
            // a wait allows for the vector memory operations issued after the
            // loads it waits for, counting only stores certain to have been
            // issued (one that no lane takes may be skipped), which only
            // makes the wait stronger.
            //  * chunk 0, tile 0: weight tile 1's loads (8) may stay in flight;
            //  * chunk 0, tile 1: tile 0's output stores may, one per k with
            //    row 4 (wave + 4 k) < T;
            //  * later chunks, tile 0: the previous chunk's last 8 output
            //    stores (all its rows exist) went out after the query loads;
            //  * later chunks, tile 1: nothing new to wait for.
            if (tt == 0) {
                if (t0 == 0 && TPB == 2)
                    ab_vm_wait<AB_N / 16>();
                else if (t0 == 0)
                    ab_vm_wait<0>();
                else
                    ab_vm_wait<AB_M / 16>();
            } else if (t0 == 0) {
                int issued = 0;
#pragma unroll
                for (int k = 0; k < AB_M / 16; ++k)
                    issued += 4 * (wave + 4 * k) < a.T;
                ab_vm_wait_upto8(issued);
            }
            lds_barrier();
            const char* wrow = wt[tt] + (wave * 32 + frow) * AB_ROWB;   // latent column 32 wave + frow of the tile
            f32x16 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = f32x16{};
            // The fragments of k step kk + 1 are read before step kk's MFMAs
            // go out (order pinned below), so the LDS latency is exposed once
            // per tile, not once per MFMA.
            bf16x8 wf[2], af[2][4];
            auto read_step = [&](int kk, int b) __attribute__((always_inline)) {
                const int g = 2 * kk + half;   // lane's 8 k values: granule g of the row
                wf[b] = as_bf16x8(lds_ld16(wrow + ((g ^ (frow & 15)) * 16)));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 32 * i + frow;
                    af[b][i] = as_bf16x8(lds_ld16(at + r * AB_ROWB + ((g ^ (r & 15)) * 16)));
                }
            };
            read_step(0, 0);
#pragma unroll
            for (int kk = 0; kk < AB_K / 16; ++kk) {
                const int b = kk & 1;
                if (kk + 1 < AB_K / 16)
                    read_step(kk + 1, b ^ 1);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b], af[b][i], acc[i], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
            for (int kk = 0; kk + 1 < AB_K / 16; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            // Stage: lane holds rows 32 i + frow, tile columns 32 wave + 8 q + 4 half + 0..3.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * i + frow;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int g = 4 * wave + q;
                    const u32x2 v = {pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]),
                                     pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3])};
                    lds_st8(st + r * AB_ROWB + ((g ^ (r & 15)) * 16) + half * 8, v);
                }
            }
            lds_barrier();
            // Every wave is done with the chunk after the last tile: the next
            // one (and its rope granules) may land while this tile is stored.
            if (tt == TPB - 1 && t0 + AB_M < a.T) {
                if (rope) {
                    // the stores below need this chunk's rope registers first
#pragma unroll
                    for (int k = 0; k < AB_ROPE_REGS; ++k) {
                        const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
                        if (idx < AB_M * gpr && t0 + r < a.T)
                            st16(out + ((int64_t)(t0 + r) * a.H + h) * a.Do + a.NL + g * 8, rp[k]);
                    }
                }
                load_rope(t0 + AB_M);
                load_chunk(t0 + AB_M);
            }
            // Each store: 4 rows of 256 bytes (lane l: row 4 s + l / 16, granule l % 16).
            const int n0 = (u * TPB + tt) * AB_N;
#pragma unroll
            for (int k = 0; k < AB_M / 16; ++k) {
                const int row = 4 * (wave + 4 * k) + lr;
                const int t = t0 + row;
                if (t < a.T) {
                    const u32x4 v = lds_ld16(st + row * AB_ROWB + ((lg ^ (row & 15)) * 16));
                    st16(out + ((int64_t)t * a.H + h) * a.Do + n0 + 8 * lg, v);
                }
            }
            if (tt == TPB - 1 && t0 + AB_M >= a.T && rope) {
#pragma unroll
                for (int k = 0; k < AB_ROPE_REGS; ++k) {
                    const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
                    if (idx < AB_M * gpr && t0 + r < a.T)
                        st16(out + ((int64_t)(t0 + r) * a.H + h) * a.Do + a.NL + g * 8, rp[k]);
                }
            }
            // Rope wider than the registers hold: the rest, loaded here.
            if (tt == TPB - 1 && rope && gpr * AB_M > AB_NT * AB_ROPE_REGS) {
                for (int idx = tid + AB_NT * AB_ROPE_REGS; idx < AB_M * gpr; idx += AB_NT) {
                    const int r = idx / gpr, g = idx - r * gpr;
                    const int t = t0 + r;
                    if (t < a.T) {
                        const int64_t th = (int64_t)t * a.H + h;
                        st16(out + th * a.Do + a.NL + g * 8, ld16(a.q + th * a.Dq + AB_K + g * 8));
                    }
                }
            }
            // The staging tile is read into registers before the next tile's
            // (or chunk's) outputs are written over it.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
}

// The fp8 form (w_uk in e4m3 with fp32 scales per 128 x 128 block of each
// head; the query's non-rope part quantised per 1 x 128 block like the
// decompress activations: s_q = amax / 448, codes = e4m3(x * (448 / amax))):
//   out[t][h][c] = bf16( s_q[t][h] * w_uk_scale[h][c / 128][0]
//                        * sum_{d < 128} codes_q[t][h][d] * w_uk[h][c][d] )
// Same blocks as the bf16 form.  Each block quantises its query chunk in LDS
// (16 lanes per row, amax by a 16-lane butterfly), then runs
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales: the 128 columns are
// one scale block, so the epilogue applies s_q * s_w once.  fp8 tile rows are
// 128 bytes, 8 granules XOR-swizzled by (row / 2) % 8.
constexpr int AF_ROWB = AB_K;

__device__ inline int f8_granule(int row, int g) { return (g ^ ((row >> 1) & 7)) * 16; }

__device__ inline i32x8 join16(u32x4 lo, u32x4 hi)
{
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int TPB>
__global__ void __launch_bounds__(AB_NT, 1) absorb_fp8(AbsorbArgs a)
{
    __shared__ __attribute__((aligned(1024))) char wt[TPB][AB_N * AF_ROWB];   // weight codes
    __shared__ __attribute__((aligned(1024))) char at[AB_M * AB_ROWB];        // bf16 query rows
    __shared__ __attribute__((aligned(1024))) char qt[AB_M * AF_ROWB];        // query codes
    __shared__ __attribute__((aligned(1024))) char st[AB_M * AB_ROWB];        // output staging
    __shared__ float qsc[AB_M];                                               // query scales

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tpn = a.NL / AB_N, bph = tpn / TPB;
    const int j = (int)(blockIdx.x >> 3);
    const int u = j % bph, h = (j / bph) * 8 + (int)(blockIdx.x & 7);
    if (h >= a.H)
        return;
    const uint32_t at_lds = lds_addr(at);

    const int lr = lane >> 4, lg = lane & 15;
    const i32x4 qr = make_srd(a.q, (uint32_t)((int64_t)a.T * a.H * a.Dq * 2));
    auto load_chunk = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < AB_M / 16; ++k) {
            const int i = wave + 4 * k, row = 4 * i + lr;
            const uint32_t off = (uint32_t)(((int64_t)(t0 + row) * a.H + h) * a.Dq * 2);
            asm_ld16_lds(qr, at_lds + i * 1024, off + (uint32_t)((lg ^ (row & 15)) * 16), 0u);
        }
    };
    const bool rope = a.R > 0 && u == 0;
    const int gpr = a.R > 0 ? a.R / 8 : 1;   // granules per rope row (1 when there is none: a safe divisor)
    u32x4 rp[AB_ROPE_REGS];
    auto load_rope = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < AB_ROPE_REGS; ++k) {
            const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
            if (rope && idx < AB_M * gpr && t0 + r < a.T)
                rp[k] = ld16(a.q + ((int64_t)(t0 + r) * a.H + h) * a.Dq + AB_K + g * 8);
        }
    };

    load_rope(0);
    load_chunk(0);
    // Weight codes of tile tt: rows of head h (16 KB).  One load = 8 rows:
    // lane l fills physical granule l % 8 of row 8 i + l / 8.
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
        const i32x4 wr = make_srd(a.wq + ((int64_t)h * a.NL + (u * TPB + tt) * AB_N) * AB_K, (uint32_t)(AB_N * AF_ROWB));
        const uint32_t wt_lds = lds_addr(wt[tt]);
        const int fr = lane >> 3, fg = lane & 7;
#pragma unroll
        for (int k = 0; k < AB_N / 32; ++k) {
            const int i = wave + 4 * k, row = 8 * i + fr;
            asm_ld16_lds(wr, wt_lds + i * 1024, (uint32_t)(row * AF_ROWB + ((fg ^ ((row >> 1) & 7)) * 16)), 0u);
        }
    }

    const int frow = lane & 31, half = lane >> 5;
    const int wrow = wave * 32 + frow;
    uint16_t* out = a.out;
    for (int t0 = 0; t0 < a.T; t0 += AB_M) {
        // The chunk (and on the first chunk weight tile 0) has landed; the
        // waits count stores too, as in the bf16 form: on the first chunk
        // weight tile 1's 4 loads may stay in flight, on later ones the
        // previous chunk's last 8 output stores.
        if (t0 == 0 && TPB == 2)
            ab_vm_wait<AB_N / 32>();
        else if (t0 == 0)
            ab_vm_wait<0>();
        else
            ab_vm_wait<AB_M / 16>();
        lds_barrier();
        // Quantise the chunk: lanes 16 k .. 16 k + 15 hold row 16 p + 4 wave + k,
        // 8 values each (one granule of the bf16 row).  All of the lane's
        // granules are read before the first is used (one LDS round trip, not
        // one per row).
        u32x4 qv[AB_M / 16];
#pragma unroll
        for (int p = 0; p < AB_M / 16; ++p) {
            const int r = 16 * p + 4 * wave + lr;
            qv[p] = lds_ld16(at + r * AB_ROWB + ((lg ^ (r & 15)) * 16));
        }
        __builtin_amdgcn_sched_barrier(0);
        // Row maxima first (the lane group's 8 rows), then one pair of
        // divisions per lane for row lg % 8 of its group, whose results each
        // row's lanes take from lane p of their 16-lane row (a DPP row
        // broadcast): two divisions per lane instead of sixteen.
        float amx[AB_M / 16];
#pragma unroll
        for (int p = 0; p < AB_M / 16; ++p) {
            const u32x4 v = qv[p];
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                am = fmaxf(am, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
            amx[p] = max16(am);
        }
        float my_am = amx[0];
#pragma unroll
        for (int p = 1; p < AB_M / 16; ++p)
            my_am = (lg & 7) == p ? amx[p] : my_am;
        float my_sq = 1.0f, my_inv = 1.0f;
        if (my_am > 0.0f) {
            my_sq = my_am / 448.0f;
            my_inv = 448.0f / my_am;
        }
#pragma unroll
        for (int p = 0; p < AB_M / 16; ++p) {
            const int r = 16 * p + 4 * wave + lr;
            const u32x4 v = qv[p];
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_lo(v[i]);
                x[2 * i + 1] = bf16_hi(v[i]);
            }
            const float inv = row16_lane(my_inv, p);
            const u32x2 codes = {pack_e4m3x2(x[0] * inv, x[1] * inv) | (pack_e4m3x2(x[2] * inv, x[3] * inv) << 16),
                                 pack_e4m3x2(x[4] * inv, x[5] * inv) | (pack_e4m3x2(x[6] * inv, x[7] * inv) << 16)};
            lds_st8(qt + r * AF_ROWB + f8_granule(r, lg >> 1) + (lg & 1) * 8, codes);
            const float sq = row16_lane(my_sq, p);
            if (lg == 0)
                qsc[r] = sq;
        }
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
            // Weight tile 1 on the first chunk: its loads, with tile 0's output
            // stores (those certain to have been issued) allowed in flight.
            if (tt == 1 && t0 == 0) {
                int issued = 0;
#pragma unroll
                for (int k = 0; k < AB_M / 16; ++k)
                    issued += 4 * (wave + 4 * k) < a.T;
                ab_vm_wait_upto8(issued);
            }
            lds_barrier();
            f32x16 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = f32x16{};
            // Both k steps' fragments are read before the first MFMA goes out
            // (order pinned below), so the second step's reads run under the
            // first step's MFMAs.
            i32x8 wf[2], af[2][4];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int g0 = 4 * kk + 2 * half;   // lane's 32 codes: granules g0, g0 + 1
                wf[kk] = join16(lds_ld16(wt[tt] + wrow * AF_ROWB + f8_granule(wrow, g0)),
                                lds_ld16(wt[tt] + wrow * AF_ROWB + f8_granule(wrow, g0 + 1)));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 32 * i + frow;
                    af[kk][i] = join16(lds_ld16(qt + r * AF_ROWB + f8_granule(r, g0)),
                                       lds_ld16(qt + r * AF_ROWB + f8_granule(r, g0 + 1)));
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[kk], af[kk][i], acc[i], 0, 0, 0, 127,
                                                                             0, 127);
            __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            const float sw = a.wscale[(int64_t)h * tpn + u * TPB + tt];
            // Stage: lane holds rows 32 i + frow, tile columns 32 wave + 8 q + 4 half + 0..3.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * i + frow;
                const float rs = qsc[r] * sw;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int g = 4 * wave + q;
                    const u32x2 v = {pack_bf16x2(acc[i][4 * q] * rs, acc[i][4 * q + 1] * rs),
                                     pack_bf16x2(acc[i][4 * q + 2] * rs, acc[i][4 * q + 3] * rs)};
                    lds_st8(st + r * AB_ROWB + ((g ^ (r & 15)) * 16) + half * 8, v);
                }
            }
            lds_barrier();
            if (tt == TPB - 1 && t0 + AB_M < a.T) {
                if (rope) {
#pragma unroll
                    for (int k = 0; k < AB_ROPE_REGS; ++k) {
                        const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
                        if (idx < AB_M * gpr && t0 + r < a.T)
                            st16(out + ((int64_t)(t0 + r) * a.H + h) * a.Do + a.NL + g * 8, rp[k]);
                    }
                }
                load_rope(t0 + AB_M);
                load_chunk(t0 + AB_M);
            }
            const int n0 = (u * TPB + tt) * AB_N;
#pragma unroll
            for (int k = 0; k < AB_M / 16; ++k) {
                const int row = 4 * (wave + 4 * k) + lr;
                const int t = t0 + row;
                if (t < a.T) {
                    const u32x4 v = lds_ld16(st + row * AB_ROWB + ((lg ^ (row & 15)) * 16));
                    st16(out + ((int64_t)t * a.H + h) * a.Do + n0 + 8 * lg, v);
                }
            }
            if (tt == TPB - 1 && t0 + AB_M >= a.T && rope) {
#pragma unroll
                for (int k = 0; k < AB_ROPE_REGS; ++k) {
                    const int idx = tid + AB_NT * k, r = idx / gpr, g = idx - r * gpr;
                    if (idx < AB_M * gpr && t0 + r < a.T)
                        st16(out + ((int64_t)(t0 + r) * a.H + h) * a.Do + a.NL + g * 8, rp[k]);
                }
            }
            if (tt == TPB - 1 && rope && gpr * AB_M > AB_NT * AB_ROPE_REGS) {
                for (int idx = tid + AB_NT * AB_ROPE_REGS; idx < AB_M * gpr; idx += AB_NT) {
                    const int r = idx / gpr, g = idx - r * gpr;
                    const int t = t0 + r;
                    if (t < a.T) {
                        const int64_t th = (int64_t)t * a.H + h;
                        st16(out + th * a.Do + a.NL + g * 8, ld16(a.q + th * a.Dq + AB_K + g * 8));
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
}

}  // namespace

hipError_t launch_absorb_fp8(const AbsorbArgs& a, hipStream_t s)
{
    const int heads8 = (a.H + 7) / 8 * 8, tiles = a.NL / AB_N;
    if (tiles % 2 == 0) {
        log_launch("absorb_fp8<2>", heads8 * (tiles / 2), AB_NT, "T=%d H=%d latent=%d", a.T, a.H, a.NL);
        hipLaunchKernelGGL(absorb_fp8<2>, dim3(heads8 * (tiles / 2)), dim3(AB_NT), 0, s, a);
    } else {
        log_launch("absorb_fp8<1>", heads8 * tiles, AB_NT, "T=%d H=%d latent=%d", a.T, a.H, a.NL);
        hipLaunchKernelGGL(absorb_fp8<1>, dim3(heads8 * tiles), dim3(AB_NT), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_absorb_bf16(const AbsorbArgs& a, hipStream_t s)
{
    const int heads8 = (a.H + 7) / 8 * 8, tiles = a.NL / AB_N;
    if (tiles % 2 == 0) {
        log_launch("absorb_bf16<2>", heads8 * (tiles / 2), AB_NT, "T=%d H=%d latent=%d", a.T, a.H, a.NL);
        hipLaunchKernelGGL(absorb_bf16<2>, dim3(heads8 * (tiles / 2)), dim3(AB_NT), 0, s, a);
    } else {
        log_launch("absorb_bf16<1>", heads8 * tiles, AB_NT, "T=%d H=%d latent=%d", a.T, a.H, a.NL);
        hipLaunchKernelGGL(absorb_bf16<1>, dim3(heads8 * tiles), dim3(AB_NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mla
