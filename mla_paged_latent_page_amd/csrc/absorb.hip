// Query absorption (page "mla_prefill_decode_graph_fp8", Args q [tot_seq_len,
// num_heads, qk_nope_head_dim + qk_rope_head_dim] and w_uk [num_heads,
// kv_latent_dim, qk_nope_head_dim], the weight that takes the non-rope part of
// each query head into the KV latent space):
//   out[t][h][c] = bf16( sum_{d < 128} q[t][h][d] * w_uk[h][c][d] ),  c < kv_latent_dim
// in fp32, and, when asked, the rope part q[t][h][128:] copied right after it, so
// that an absorbed query head has the layout of a cache row (latent, then rope).
//
// Bound by HBM: at decode sizes the weight (num_heads * 512 * 128 bf16, 16 MiB)
// and the output dominate.  One block of 4 waves per head and 128 latent
// columns; the kv_latent_dim / 128 blocks of one head are dispatched to the
// same XCD, next to each other, so they read that head's query rows from HBM
// once and share them in the XCD's L2.  The weight tile (128 x 128, 32 KB) is
// put into LDS once; query rows follow in chunks of 128 (32 KB), both by LDS
// DMA from inline assembly with explicit waits.  v_mfma_f32_32x32x16_bf16 with
// the weight as the row operand: wave w owns the tile's latent columns
// 32 w .. 32 w + 31 for all 128 rows of a chunk and stores 4 consecutive
// columns per lane.
#include "launch.hpp"

namespace mla {
namespace {

constexpr int AB_N = 128;            // latent columns per block
constexpr int AB_K = 128;            // qk_nope_head_dim
constexpr int AB_M = 128;            // query rows per chunk
constexpr int AB_NT = 256;
constexpr int AB_ROWB = AB_K * 2;    // 256-byte tile rows: 16 granules, XOR-swizzled by row % 16

__global__ void __launch_bounds__(AB_NT, 2) absorb_bf16(AbsorbArgs a)
{
    __shared__ __attribute__((aligned(1024))) char wt[AB_N * AB_ROWB];
    __shared__ __attribute__((aligned(1024))) char at[AB_M * AB_ROWB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Block b runs on XCD b % 8; there its j-th block (j = b / 8) is column
    // tile j % tpn of head (j / tpn) * 8 + b % 8.
    const int tpn = a.NL / AB_N;
    const int j = (int)(blockIdx.x >> 3);
    const int nt = j % tpn, h = (j / tpn) * 8 + (int)(blockIdx.x & 7);
    if (h >= a.H)
        return;
    const int n0 = nt * AB_N;
    const uint32_t wt_lds = lds_addr(wt), at_lds = lds_addr(at);

    // One load moves 4 tile rows: lane l fills physical granule l % 16 of row
    // 4 i + l / 16, which holds logical granule (l % 16) ^ (row % 16).
    const int lr = lane >> 4, lg = lane & 15;
    const i32x4 wr = make_srd(a.w + ((int64_t)h * a.NL + n0) * AB_K, (uint32_t)(AB_N * AB_ROWB));
    for (int i = wave; i < AB_N / 4; i += 4) {
        const int row = 4 * i + lr;
        asm_ld16_lds(wr, wt_lds + i * 1024, (uint32_t)(row * AB_ROWB + ((lg ^ (row & 15)) * 16)), 0u);
    }
    // Query rows t0 .. t0 + 127 of head h (rows past T read as zeros: their
    // offsets are past the end of the resource).
    const i32x4 qr = make_srd(a.q, (uint32_t)((int64_t)a.T * a.H * a.Dq * 2));
    auto load_chunk = [&](int t0) __attribute__((always_inline)) {
        for (int i = wave; i < AB_M / 4; i += 4) {
            const int row = 4 * i + lr;
            const uint32_t off = (uint32_t)(((int64_t)(t0 + row) * a.H + h) * a.Dq * 2);
            asm_ld16_lds(qr, at_lds + i * 1024, off + (uint32_t)((lg ^ (row & 15)) * 16), 0u);
        }
    };
    load_chunk(0);

    const int frow = lane & 31, half = lane >> 5;
    const char* wrow = wt + (wave * 32 + frow) * AB_ROWB;   // latent column n0 + 32 wave + frow
    uint16_t* out = a.out;
    for (int t0 = 0; t0 < a.T; t0 += AB_M) {
        // This wave's loads (the chunk, and at first the weight tile) have
        // landed; the barrier makes everyone's visible.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < AB_K / 16; ++kk) {
            const int g = 2 * kk + half;   // lane's 8 k values: granule g of the row
            const bf16x8 wf = as_bf16x8(lds_ld16(wrow + ((g ^ (frow & 15)) * 16)));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * i + frow;
                const bf16x8 af = as_bf16x8(lds_ld16(at + r * AB_ROWB + ((g ^ (r & 15)) * 16)));
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc[i], 0, 0, 0);
            }
        }
        // Every wave is done with the chunk: the next one may land in its place
        // while this one's outputs are stored.
        lds_barrier();
        if (t0 + AB_M < a.T)
            load_chunk(t0 + AB_M);
        // Lane holds rows t0 + 32 i + frow, columns n0 + 32 wave + 8 q + 4 half + 0..3.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 32 * i + frow;
            if (t < a.T) {
                uint16_t* orow = out + ((int64_t)t * a.H + h) * a.Do + n0 + 32 * wave + 4 * half;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 v = {pack_bf16x2(acc[i][4 * q], acc[i][4 * q + 1]),
                                     pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3])};
                    *reinterpret_cast<u32x2*>(orow + 8 * q) = v;
                }
            }
        }
        // The rope part (column tile 0 of each head copies it): R * 2 bytes per row.
        if (a.R > 0 && nt == 0) {
            const int gpr = a.R / 8;
            for (int idx = tid; idx < AB_M * gpr; idx += AB_NT) {
                const int r = idx / gpr, g = idx - r * gpr;
                const int t = t0 + r;
                if (t < a.T) {
                    const int64_t th = (int64_t)t * a.H + h;
                    st16(out + th * a.Do + a.NL + g * 8, ld16(a.q + th * a.Dq + AB_K + g * 8));
                }
            }
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

__global__ void __launch_bounds__(AB_NT, 2) absorb_fp8(AbsorbArgs a)
{
    __shared__ __attribute__((aligned(1024))) char wt[AB_N * AF_ROWB];   // weight codes
    __shared__ __attribute__((aligned(1024))) char at[AB_M * AB_ROWB];   // bf16 query rows
    __shared__ __attribute__((aligned(1024))) char qt[AB_M * AF_ROWB];   // query codes
    __shared__ float qsc[AB_M];                                          // query scales

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tpn = a.NL / AB_N;
    const int j = (int)(blockIdx.x >> 3);
    const int nt = j % tpn, h = (j / tpn) * 8 + (int)(blockIdx.x & 7);
    if (h >= a.H)
        return;
    const int n0 = nt * AB_N;
    const uint32_t wt_lds = lds_addr(wt), at_lds = lds_addr(at);

    // Weight codes: rows n0 .. n0 + 127 of head h (16 KB).  One load = 8 rows:
    // lane l fills physical granule l % 8 of row 8 i + l / 8.
    const i32x4 wr = make_srd(a.wq + ((int64_t)h * a.NL + n0) * AB_K, (uint32_t)(AB_N * AF_ROWB));
    {
        const int fr = lane >> 3, fg = lane & 7;
        for (int i = wave; i < AB_N / 8; i += 4) {
            const int row = 8 * i + fr;
            asm_ld16_lds(wr, wt_lds + i * 1024, (uint32_t)(row * AF_ROWB + ((fg ^ ((row >> 1) & 7)) * 16)), 0u);
        }
    }
    const float sw = a.wscale[(int64_t)h * tpn + nt];
    const int lr = lane >> 4, lg = lane & 15;
    const i32x4 qr = make_srd(a.q, (uint32_t)((int64_t)a.T * a.H * a.Dq * 2));
    auto load_chunk = [&](int t0) __attribute__((always_inline)) {
        for (int i = wave; i < AB_M / 4; i += 4) {
            const int row = 4 * i + lr;
            const uint32_t off = (uint32_t)(((int64_t)(t0 + row) * a.H + h) * a.Dq * 2);
            asm_ld16_lds(qr, at_lds + i * 1024, off + (uint32_t)((lg ^ (row & 15)) * 16), 0u);
        }
    };
    load_chunk(0);

    const int frow = lane & 31, half = lane >> 5;
    const int wrow = wave * 32 + frow;
    uint16_t* out = a.out;
    for (int t0 = 0; t0 < a.T; t0 += AB_M) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        // Quantise the chunk: lanes 16 k .. 16 k + 15 hold row 16 p + 4 wave + k,
        // 8 values each (one granule of the bf16 row).
#pragma unroll
        for (int p = 0; p < AB_M / 16; ++p) {
            const int r = 16 * p + 4 * wave + lr;
            const u32x4 v = lds_ld16(at + r * AB_ROWB + ((lg ^ (r & 15)) * 16));
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = bf16_lo(v[i]);
                x[2 * i + 1] = bf16_hi(v[i]);
            }
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                am = fmaxf(am, fabsf(x[i]));
            am = fmaxf(am, __shfl_xor(am, 1));
            am = fmaxf(am, __shfl_xor(am, 2));
            am = fmaxf(am, __shfl_xor(am, 4));
            am = fmaxf(am, __shfl_xor(am, 8));
            float sq = 1.0f, inv = 1.0f;
            if (am > 0.0f) {
                sq = am / 448.0f;
                inv = 448.0f / am;
            }
            const u32x2 codes = {pack_e4m3x2(x[0] * inv, x[1] * inv) | (pack_e4m3x2(x[2] * inv, x[3] * inv) << 16),
                                 pack_e4m3x2(x[4] * inv, x[5] * inv) | (pack_e4m3x2(x[6] * inv, x[7] * inv) << 16)};
            lds_st8(qt + r * AF_ROWB + f8_granule(r, lg >> 1) + (lg & 1) * 8, codes);
            if (lg == 0)
                qsc[r] = sq;
        }
        lds_barrier();
        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int g0 = 4 * kk + 2 * half;   // lane's 32 codes: granules g0, g0 + 1
            const i32x8 wf = join16(lds_ld16(wt + wrow * AF_ROWB + f8_granule(wrow, g0)),
                                    lds_ld16(wt + wrow * AF_ROWB + f8_granule(wrow, g0 + 1)));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * i + frow;
                const i32x8 af = join16(lds_ld16(qt + r * AF_ROWB + f8_granule(r, g0)),
                                        lds_ld16(qt + r * AF_ROWB + f8_granule(r, g0 + 1)));
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, af, acc[i], 0, 0, 0, 127, 0, 127);
            }
        }
        float rs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rs[i] = qsc[32 * i + frow] * sw;
        lds_barrier();
        if (t0 + AB_M < a.T)
            load_chunk(t0 + AB_M);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 32 * i + frow;
            if (t < a.T) {
                uint16_t* orow = out + ((int64_t)t * a.H + h) * a.Do + n0 + 32 * wave + 4 * half;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 v = {pack_bf16x2(acc[i][4 * q] * rs[i], acc[i][4 * q + 1] * rs[i]),
                                     pack_bf16x2(acc[i][4 * q + 2] * rs[i], acc[i][4 * q + 3] * rs[i])};
                    *reinterpret_cast<u32x2*>(orow + 8 * q) = v;
                }
            }
        }
        if (a.R > 0 && nt == 0) {
            const int gpr = a.R / 8;
            for (int idx = tid; idx < AB_M * gpr; idx += AB_NT) {
                const int r = idx / gpr, g = idx - r * gpr;
                const int t = t0 + r;
                if (t < a.T) {
                    const int64_t th = (int64_t)t * a.H + h;
                    st16(out + th * a.Do + a.NL + g * 8, ld16(a.q + th * a.Dq + AB_K + g * 8));
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_absorb_fp8(const AbsorbArgs& a, hipStream_t s)
{
    const int heads8 = (a.H + 7) / 8 * 8;
    hipLaunchKernelGGL(absorb_fp8, dim3(heads8 * (a.NL / AB_N)), dim3(AB_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_absorb_bf16(const AbsorbArgs& a, hipStream_t s)
{
    const int heads8 = (a.H + 7) / 8 * 8;
    hipLaunchKernelGGL(absorb_bf16, dim3(heads8 * (a.NL / AB_N)), dim3(AB_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
