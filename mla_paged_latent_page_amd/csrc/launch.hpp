// Host-side launchers of the gfx950 kernels.  The C ABI in api.hip validates
// arguments and then calls exactly one of these; they only size the grid and
// enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mla {

struct DecompressArgs {
    const uint32_t* bro;   // buffer_row_offsets [batch+1]
    const uint32_t* co;    // cache_offsets [>= batch]
    PagedLayer L;          // layer view of the latent pool (kv half 0)
    const void* W;         // [N][K] weight (bf16 / f32 / e4m3 codes)
    const float* W_scale;  // fp8 only: [N/128][K/128]
    void* lat;             // k_latent_buffer [M][D]
    void* out;             // k_buffer [M][N]
    void* q;               // fp8 only: activation codes [M][K]
    float* q_scale;        // fp8 only: activation scales [M][K/128]
    int M, N, K, D;        // D = elements per cache token row = row stride of lat
};

struct KvMatmulArgs {
    const uint16_t* H;         // hidden_state bf16 [T][Kd]
    const uint32_t* iro;       // input_row_offsets [batch+1]
    const uint16_t* W;         // weight bf16 [Kd][N]
    const uint32_t* cache_len; // [batch]
    PagedLayer L;              // layer view of the K/V pool
    int T, Kd, N, HD;          // N = 2*HD
};

hipError_t launch_gather_rows(const DecompressArgs& a, int elem_bytes, hipStream_t s);
hipError_t launch_product_bf16(const DecompressArgs& a, hipStream_t s);
hipError_t launch_product_f32(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_bf16(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_f32(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_fp8(const DecompressArgs& a, hipStream_t s);
hipError_t launch_kv_matmul(const KvMatmulArgs& a, hipStream_t s);
hipError_t launch_product_fp8_ring(const DecompressArgs& a, int cus, hipStream_t s);
hipError_t launch_kv_matmul_ring(const KvMatmulArgs& a, int cus, hipStream_t s);
int num_cus();
bool small_bf16_fits(const DecompressArgs& a);
hipError_t launch_small_bf16(const DecompressArgs& a, int gather, hipStream_t s);

}  // namespace mla
