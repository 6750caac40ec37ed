// Paged gather of latent rows (page "generic_flare_mla_decompress_k_cache_ragged_paged",
// summary and Args buffer_row_offsets_1d, cache_offsets_1d, k_latent_buffer):
//   k_latent[r][0:D] = cache row of request b at position cache_offsets[b] + (r - row_offsets[b])
// as a bit copy.  One wave per row: the row's request and page are resolved with
// wave-uniform (scalar) loads, then the lanes copy the row in 16-byte pieces.
// The copy is HBM-bound (it reads and writes D * elem bytes per row).
#include "launch.hpp"

namespace mla {
namespace {

__global__ void __launch_bounds__(256) gather_rows_kernel(DecompressArgs a, int granules_per_row)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.M)
        return;
    const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)r);
    const uint32_t p = a.co[b] + ((uint32_t)r - a.bro[b]);
    const char* src = a.L.base + token_offset(a.L, b, p);
    char* dst = static_cast<char*>(a.lat) + (int64_t)r * granules_per_row * 16;
    for (int g = lane; g < granules_per_row; g += 64)
        st16(dst + g * 16, ld16(src + g * 16));
}

}  // namespace

hipError_t launch_gather_rows(const DecompressArgs& a, int elem_bytes, hipStream_t s)
{
    const int gpr = a.D * elem_bytes / 16;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, a, gpr);
    return hipGetLastError();
}

}  // namespace mla
