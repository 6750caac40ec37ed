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

    // 2. The product.  Wave w: weight block wb = w % 2, row blocks j0, j0 + 2, ...
    const int wb = wave & 1, j0 = wave >> 1;
    constexpr int NTM = (MB + 1) / 2;        // row blocks of wave 0 / 1 (waves 2 / 3 may have one fewer)
    const int nt = (MB - j0 + 1) / 2;
    const int frow = lane & 31;
    int fr_off[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            fr_off[kk][h] = frow * FS_ROWB + (((4 * kk + 2 * (lane >> 5) + h) ^ ((frow >> 1) & 7)) * 16);

    f32x16 acc[NTM];
    float ref[NTM];
#pragma unroll
    for (int t = 0; t < NTM; ++t) {
        acc[t] = f32x16{};
        ref[t] = 0.0f;
    }
#pragma unroll
    for (int kb = 0; kb < FS_KB; ++kb) {
        switch (kb) {
        case 0: fs_vm_wait<3 * C::LOADS>(); break;
        case 1: fs_vm_wait<2 * C::LOADS>(); break;
        case 2: fs_vm_wait<1 * C::LOADS>(); break;
        default: fs_vm_wait<0>(); break;
        }
        lds_barrier();
        const float sw = swc[kb][0][lane];
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

    // 3. Outputs through LDS (the first scale block's row codes, read by now
    //    by every wave): lane l holds row 32 j + l % 32, columns
    //    32 wb + 8 q + 4 (l / 32) .. +3 (q < 4) of the block's 64.
    lds_barrier();
    char* stg = aq[0];
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

}  // namespace mla
