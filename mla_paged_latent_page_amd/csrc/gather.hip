// Paged gather of latent rows (page "generic_flare_mla_decompress_k_cache_ragged_paged",
// summary and Args buffer_row_offsets_1d, cache_offsets_1d, k_latent_buffer):
//   k_latent[r][0:D] = cache row of request b at position cache_offsets[b] + (r - row_offsets[b])
// as a bit copy.  The copy is HBM-bound: it reads and writes D * elem bytes per row.
// With an fp8 cache the row's fp32 scales (one per 128 columns, the collection's
// scale_dtype_ and quantization_granularity_) are copied the same way from the
// scale pool into k_latent_scales[r][0:nblk].
//
// Each wave copies ROWS consecutive rows.  Lanes 0..ROWS-1 resolve one row each
// (request by binary search, then page and slot), the offsets are broadcast
// with readlane, and then the wave copies the rows as one flat run of 16-byte
// granules (the destination rows are consecutive): every lane issues ROWS
// loads before its first store, and every instruction but the last has all
// 64 lanes busy (a row of 72 granules per lane pass would leave 56 idle).
#include "launch.hpp"

namespace mla {
namespace {

constexpr int ROWS = 8;  // rows per wave

__global__ void __launch_bounds__(256) gather_rows_kernel(DecompressArgs a, int granules_per_row)
{
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * ROWS;
    if (r0 >= a.M)
        return;

    // Lane i < ROWS resolves row r0 + i (rows past M get a harmless offset 0).
    int64_t my_off = 0, my_soff = 0;
    const int my_row = r0 + lane;
    if (lane < ROWS && my_row < a.M) {
        const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)my_row);
        const uint32_t p = a.co[b] + ((uint32_t)my_row - a.bro[b]);
        my_off = token_offset(a.L, b, p);
        if (a.lat_scale)
            my_soff = token_offset(a.Ls, b, p);
    }
    const uint32_t off_lo = (uint32_t)my_off, off_hi = (uint32_t)(my_off >> 32);
    const char* src[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const uint64_t o = ((uint64_t)__builtin_amdgcn_readlane(off_hi, i) << 32) | __builtin_amdgcn_readlane(off_lo, i);
        src[i] = a.L.base + o;
    }
    const int nrows = min(ROWS, a.M - r0);
    if (a.lat_scale) {
        // Scales: element idx = i * nblk + j of the wave's ROWS x nblk block is
        // scale j of row r0 + i, whose offset lane i resolved.
        const uint32_t s_lo = (uint32_t)my_soff, s_hi = (uint32_t)(my_soff >> 32);
        for (int base = 0; base < ROWS * a.nblk; base += 64) {
            const int idx = base + lane;
            const int i = min(idx / a.nblk, ROWS - 1);
            const uint64_t o = ((uint64_t)(uint32_t)__shfl((int)s_hi, i, 64) << 32) | (uint32_t)__shfl((int)s_lo, i, 64);
            if (idx < nrows * a.nblk) {
                const int j = idx - i * a.nblk;
                a.lat_scale[(int64_t)r0 * a.nblk + idx] = *reinterpret_cast<const float*>(a.Ls.base + o + j * 4);
            }
        }
    }
    const int64_t row_bytes = (int64_t)granules_per_row * 16;
    char* dst = static_cast<char*>(a.lat) + (int64_t)r0 * row_bytes;
    // The wave's rows are consecutive in k_latent_buffer: granule f of the
    // flat run is granule f % gpr of row f / gpr, and its destination is
    // dst + 16 f.  Every lane has a granule in every step but the last.
    const int total = nrows * granules_per_row;
    for (int f0 = 0; f0 < total; f0 += 64 * ROWS) {
        u32x4 v[ROWS];
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int f = f0 + u * 64 + lane;
            const int i = f / granules_per_row, g = f - i * granules_per_row;
            const char* sp = src[0];
#pragma unroll
            for (int k = 1; k < ROWS; ++k)
                sp = i == k ? src[k] : sp;
            v[u] = f < total ? ld16(sp + g * 16) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int f = f0 + u * 64 + lane;
            if (f < total)
                st16(dst + (int64_t)f * 16, v[u]);
        }
    }
}

}  // namespace

hipError_t launch_gather_rows(const DecompressArgs& a, int elem_bytes, hipStream_t s)
{
    const int gpr = a.D * elem_bytes / 16;
    const int waves = (a.M + ROWS - 1) / ROWS;
    log_launch("gather_rows_kernel", (waves + 3) / 4, 256, "M=%d row_bytes=%d", a.M, gpr * 16);
    hipLaunchKernelGGL(gather_rows_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a, gpr);
    return hipGetLastError();
}

}  // namespace mla
