// Measured ceilings for the roofline report (used by bench.py only; not part
// of the path or of include/mla_paged.h): what this MI355X sustains for the
// resources the path's kernels are bound by.
//
//  * mfma_bf16_loop: every CU runs 8 waves (two per SIMD) of back-to-back
//    v_mfma_f32_32x32x16_bf16 on operands read from LDS each k step (random
//    bf16 data, as in the product kernels), 8 independent accumulators per
//    wave: the matrix-pipe ceiling at the clock the chip holds under this load.
//  * read_stream: every lane reads 16-byte pieces of its block's share of a
//    buffer (non-temporal loads), folds them into one word per thread: the
//    HBM read ceiling (large buffers) or a short read's floor (16 MiB).
//  * write_stream: every lane writes 16-byte pieces with non-temporal stores,
//    the way the product epilogues write their outputs.
//  * empty: a launch that does no work (its time in a graph replay is the
//    launch overhead every short kernel pays).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(512, 1) mfma_bf16_loop(const u32x4* __restrict__ src, float* sink, int steps)
{
    __shared__ __attribute__((aligned(1024))) u32x4 lds[4096];   // 64 KB of operands
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 4096; i += 512)
        lds[i] = src[i];
    __syncthreads();
    // Fragment reads: 6 per k step per wave (2 of one operand, 4 of the other),
    // each a 1 KB piece; wave w reads pieces 6w .. 6w+5 of 64 (all inside lds).
    const int base = wave * 6 * 64 + lane;
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x16{};
    for (int s = 0; s < steps; ++s) {
        const int o = (s & 7) * 64;   // rotate which piece feeds which operand
        bf16x8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = __builtin_bit_cast(bf16x8, lds[(base + i * 64 + o) & 4095]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = __builtin_bit_cast(bf16x8, lds[(base + (2 + j) * 64 + o) & 4095]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float f = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f += acc[i][j][lane & 15];
    sink[blockIdx.x * 512 + tid] = f;
}

template <int U>
__global__ void __launch_bounds__(256) read_stream(const u32x4* __restrict__ in, uint32_t* __restrict__ out,
                                                   int64_t per_block)
{
    const u32x4* p = in + (int64_t)blockIdx.x * per_block;
    uint32_t s = 0;
    for (int64_t i = threadIdx.x; i < per_block; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u)
            s += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) write_stream(u32x4* __restrict__ out, int64_t per_block)
{
    u32x4* p = out + (int64_t)blockIdx.x * per_block;
    const u32x4 v = {threadIdx.x, blockIdx.x, 0x3F800000u, 0u};
    for (int64_t i = threadIdx.x; i < per_block; i += 256)
        __builtin_nontemporal_store(v, p + i);
}

__global__ void empty() {}

}  // namespace

#define PEAKS_API extern "C" __attribute__((visibility("default")))

// src: >= 64 KB of bf16 data; sink: grid * 512 floats.
PEAKS_API int peaks_mfma_bf16(const void* src, void* sink, int grid, int steps, void* stream)
{
    hipLaunchKernelGGL(mfma_bf16_loop, dim3(grid), dim3(512), 0, (hipStream_t)stream, (const u32x4*)src,
                       (float*)sink, steps);
    return (int)hipGetLastError();
}

// bytes: a multiple of grid * 256 * 16 * 4; out: grid * 256 words.
PEAKS_API int peaks_read(const void* in, void* out, int64_t bytes, int grid, void* stream)
{
    const int64_t per_block = bytes / 16 / grid;
    if (per_block % (256 * 4))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_stream<4>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)in,
                       (uint32_t*)out, per_block);
    return (int)hipGetLastError();
}

// bytes: a multiple of grid * 256 * 16.
PEAKS_API int peaks_write(void* out, int64_t bytes, int grid, void* stream)
{
    const int64_t per_block = bytes / 16 / grid;
    if (per_block % 256)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(write_stream, dim3(grid), dim3(256), 0, (hipStream_t)stream, (u32x4*)out, per_block);
    return (int)hipGetLastError();
}

PEAKS_API int peaks_empty(void* stream)
{
    hipLaunchKernelGGL(empty, dim3(256), dim3(64), 0, (hipStream_t)stream);
    return (int)hipGetLastError();
}
