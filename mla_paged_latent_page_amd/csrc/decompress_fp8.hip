// Paged gather + fp8 block-scaled up-projection for gfx950 (page
// "mla_prefill_decode_graph_fp8": Parameters fp8_dtype, fp8_scale_dtype,
// m/n/k_scale_granularity; Args w_k [num_heads*qk_nope_head_dim, kv_latent_dim],
// w_k_scale; granularities 1 x 128 for activations, 128 x 128 for the weight).
//
// Pass 1 (gather_quant_fp8_kernel), QROWS rows per wave: copy the cache row into
// k_latent, and quantise its first K columns per block of 128: amax by a
// 16-lane reduction, s = amax/448, codes = e4m3(x * (448/amax)) with the
// hardware round-to-nearest-even conversion.  Codes and scales go to the
// workspace.  Quantising once here, instead of inside every N-tile of the
// product, costs one extra write+read of M*K bytes but saves re-quantising
// each activation element N/BN times.
//
// Pass 2 is the block-scaled product of decompress_fp8_ring.hip over those
// codes and scales (gemm_fp8_ring).
#include "launch.hpp"

namespace mla {
namespace {

constexpr int QROWS = 4;   // rows per wave

__global__ void __launch_bounds__(256) gather_quant_fp8_kernel(DecompressArgs a)
{
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * QROWS;
    if (r0 >= a.M)
        return;
    // Lane i < QROWS resolves row r0 + i (rows past M get offset 0 and are
    // neither loaded nor stored); the offsets are broadcast with readlane, so
    // the wave pays one chain of dependent index loads for QROWS rows.
    int64_t my_off = 0;
    const int my_row = r0 + lane;
    if (lane < QROWS && my_row < a.M) {
        const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)my_row);
        const uint32_t p = a.co[b] + ((uint32_t)my_row - a.bro[b]);
        my_off = token_offset(a.L, b, p);
    }
    const uint32_t off_lo = (uint32_t)my_off, off_hi = (uint32_t)(my_off >> 32);
    const char* src[QROWS];
#pragma unroll
    for (int i = 0; i < QROWS; ++i)
        src[i] = a.L.base + (((uint64_t)__builtin_amdgcn_readlane(off_hi, i) << 32) | __builtin_amdgcn_readlane(off_lo, i));
    const int nrows = min(QROWS, a.M - r0);
    const int nkb = a.K / 128;

    for (int c0 = 0; c0 < a.K; c0 += 512) {
        const int c = c0 + lane * 8;
        const bool in = c < a.K;  // K % 128 == 0: whole 16-lane groups are in or out
        // Every row's 16 bytes in flight before the first is used.
        u32x4 v[QROWS];
#pragma unroll
        for (int i = 0; i < QROWS; ++i)
            v[i] = in && i < nrows ? ld16(src[i] + (int64_t)c * 2) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < QROWS; ++i) {
            if (i >= nrows)
                break;
            const int r = r0 + i;
            uint16_t* lat = static_cast<uint16_t*>(a.lat) + (int64_t)r * a.D;
            uint8_t* q = static_cast<uint8_t*>(a.q) + (int64_t)r * a.K;
            float* qs = a.q_scale + (int64_t)r * nkb;
            if (in)
                st16(lat + c, v[i]);
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf16_lo(v[i][j]);
                x[2 * j + 1] = bf16_hi(v[i][j]);
            }
            float am = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                am = fmaxf(am, fabsf(x[j]));
            am = max16(am);
            float s = 1.0f, inv = 1.0f;
            if (am > 0.0f) {
                s = am / 448.0f;
                inv = 448.0f / am;
            }
            u32x2 codes;
            codes[0] = pack_e4m3x2(x[0] * inv, x[1] * inv) | (pack_e4m3x2(x[2] * inv, x[3] * inv) << 16);
            codes[1] = pack_e4m3x2(x[4] * inv, x[5] * inv) | (pack_e4m3x2(x[6] * inv, x[7] * inv) << 16);
            if (in) {
                *reinterpret_cast<u32x2*>(q + c) = codes;
                if ((lane & 15) == 0)
                    qs[c / 128] = s;
            }
        }
    }
    // The columns past K (the rope part) are copied as they are.
    const int rg = (a.D - a.K) / 8;
    for (int g = lane; g < rg; g += 64) {
        u32x4 v[QROWS];
#pragma unroll
        for (int i = 0; i < QROWS; ++i)
            if (i < nrows)
                v[i] = ld16(src[i] + (int64_t)(a.K + g * 8) * 2);
#pragma unroll
        for (int i = 0; i < QROWS; ++i)
            if (i < nrows)
                st16(static_cast<uint16_t*>(a.lat) + (int64_t)(r0 + i) * a.D + a.K + g * 8, v[i]);
    }
}

// Blocks of 4 waves, QROWS rows per wave.
inline int quant_blocks(int M) { return (M + 4 * QROWS - 1) / (4 * QROWS); }

}  // namespace

hipError_t launch_decompress_fp8(const DecompressArgs& a, hipStream_t s)
{
    if (small_fp8_gq_fits(first_projection(a)))
        return launch_small_fp8_gq(first_projection(a), s);
    log_launch("gather_quant_fp8_kernel", quant_blocks(a.M), 256, "M=%d K=%d D=%d", a.M, a.K, a.D);
    hipLaunchKernelGGL(gather_quant_fp8_kernel, dim3(quant_blocks(a.M)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const DecompressArgs p = first_projection(a);
    return small_fp8_fits(p) ? launch_small_fp8(p, s) : launch_product_fp8_ring(p, num_cus(), s);
}

// fp8 cache: the gather copies each row's codes and scales bit for bit into
// k_latent_buffer and k_latent_scales, and the product reads them from there
// (row strides D bytes and nblk floats): the cache is already quantised, so
// there is no quantisation pass.
hipError_t launch_decompress_fp8_cache(const DecompressArgs& a, hipStream_t s)
{
    if (small_fp8_gc_fits(a))
        return launch_small_fp8_gc(a, s);
    const hipError_t e = launch_gather_rows(a, 1, s);
    if (e != hipSuccess)
        return e;
    DecompressArgs p = a;   // both projections when a second one is present
    p.q = a.lat;
    p.q_scale = a.lat_scale;
    p.q_ld = a.D;
    p.qs_ld = a.nblk;
    return small_fp8_fits(p) ? launch_small_fp8(p, s) : launch_product_fp8_ring(p, num_cus(), s);
}

// Fused K and V (fp8): one gather and quantisation pass, then one product
// launch over both projections' N-tiles.
hipError_t launch_decompress_kv_fp8(const DecompressArgs& a, hipStream_t s)
{
    log_launch("gather_quant_fp8_kernel", quant_blocks(a.M), 256, "M=%d K=%d D=%d", a.M, a.K, a.D);
    hipLaunchKernelGGL(gather_quant_fp8_kernel, dim3(quant_blocks(a.M)), dim3(256), 0, s, first_projection(a));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_product_fp8_ring(a, num_cus(), s);
}

}  // namespace mla
