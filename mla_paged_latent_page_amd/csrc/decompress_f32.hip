// Paged gather + fp32 up-projection (the binary32 form of the operation of page
// "generic_flare_mla_decompress_k_cache_ragged_paged"; its `dtype` parameter is the
// element type of weight, k_latent_buffer and k_buffer alike).
//
// fp32 has no dense MFMA advantage worth a tiled kernel at the small sizes this
// type is used for, so the path is two plain kernels: a row gather (one 16-byte
// granule per thread, the request found by binary search over the ragged offsets)
// and an LDS-tiled FMA product reading the gathered rows.
#include "launch.hpp"

namespace mla {
namespace {

__global__ void __launch_bounds__(256) gather_rows_kernel(DecompressArgs a, int granules_per_row)
{
    const int64_t total = (int64_t)a.M * granules_per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(idx / granules_per_row);
        const int g = (int)(idx - (int64_t)r * granules_per_row);
        const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)r);
        const uint32_t p = a.co[b] + ((uint32_t)r - a.bro[b]);
        const int64_t off = token_offset(a.L, b, p);
        st16(static_cast<char*>(a.lat) + idx * 16, ld16(a.L.base + off + (int64_t)g * 16));
    }
}

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

hipError_t launch_decompress_f32(const DecompressArgs& a, hipStream_t s)
{
    const int gpr = a.D * 4 / 16;
    const int64_t total = (int64_t)a.M * gpr;
    const int64_t blocks = (total + 255) / 256;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, s, a, gpr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int tiles_n = (a.N + 15) / 16, tiles_m = (a.M + 15) / 16;
    hipLaunchKernelGGL(matmul_f32_kernel, dim3(tiles_n * tiles_m), dim3(256), 0, s, a, tiles_n);
    return hipGetLastError();
}

}  // namespace mla
