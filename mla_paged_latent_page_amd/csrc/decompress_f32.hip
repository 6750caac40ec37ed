// Paged gather + fp32 up-projection (the binary32 form of the operation of page
// "generic_flare_mla_decompress_k_cache_ragged_paged"; its `dtype` parameter is the
// element type of weight, k_latent_buffer and k_buffer alike).
//
// fp32 has no dense MFMA advantage worth a tiled kernel at the small sizes this
// type is used for, so the path is two plain kernels: the paged row gather of
// gather.hip and an LDS-tiled FMA product reading the gathered rows.
#include "launch.hpp"

namespace mla {
namespace {

// out[m][n] = sum_k lat[m][k] * W[n][k]; 16x16 threads, each one output, 16-wide k tiles.
__global__ void __launch_bounds__(256) matmul_f32_kernel(DecompressArgs a, int tiles_n)
{
    __shared__ float As[16][17];
    __shared__ float Ws[16][17];
    const float* lat = static_cast<const float*>(a.lat);
    const float* W = static_cast<const float*>(a.W);
    float* out = static_cast<float*>(a.out);
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int bx = blockIdx.x % tiles_n, by = blockIdx.x / tiles_n;
    const int m = by * 16 + ty, n = bx * 16 + tx;
    const int wn = bx * 16 + ty;  // weight row this thread stages
    float acc = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += 16) {
        const int k = k0 + tx;
        As[ty][tx] = (m < a.M && k < a.K) ? lat[(int64_t)m * a.D + k] : 0.0f;
        Ws[ty][tx] = (wn < a.N && k < a.K) ? W[(int64_t)wn * a.K + k] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            acc = fmaf(As[ty][kk], Ws[tx][kk], acc);
        __syncthreads();
    }
    if (m < a.M && n < a.N)
        out[(int64_t)m * a.N + n] = acc;
}

}  // namespace

hipError_t launch_product_f32(const DecompressArgs& a, hipStream_t s)
{
    const int tiles_n = (a.N + 15) / 16, tiles_m = (a.M + 15) / 16;
    log_launch("matmul_f32_kernel", tiles_n * tiles_m, 256, "M=%d N=%d K=%d", a.M, a.N, a.K);
    hipLaunchKernelGGL(matmul_f32_kernel, dim3(tiles_n * tiles_m), dim3(256), 0, s, a, tiles_n);
    return hipGetLastError();
}

hipError_t launch_decompress_f32(const DecompressArgs& a, hipStream_t s)
{
    hipError_t e = launch_gather_rows(a, 4, s);
    if (e != hipSuccess)
        return e;
    return launch_product_f32(a, s);
}

// Fused K and V (f32): one gather, then the two products.
hipError_t launch_decompress_kv_f32(const DecompressArgs& a, hipStream_t s)
{
    hipError_t e = launch_gather_rows(a, 4, s);
    if (e != hipSuccess)
        return e;
    e = launch_product_f32(first_projection(a), s);
    return e != hipSuccess ? e : launch_product_f32(second_projection(a), s);
}

}  // namespace mla
