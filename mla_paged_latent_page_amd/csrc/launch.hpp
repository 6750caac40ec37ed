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
    // Optional second projection of the same rows (the fused K and V form):
    // out2[M][N2] = rows x W2^T, with W2 [N2][K] (and W2_scale for fp8).  N2 == 0: none.
    const void* W2;
    const float* W2_scale;
    void* out2;
    int N2;
    // fp8 cache: the scale pool's layer view (one fp32 per 128 columns of a
    // token row, nblk per row), where the gather copies each row's scales
    // (lat_scale [M][nblk]; null: no scales), and the row strides the fp8
    // product reads its activation codes and scales with (q_ld bytes, qs_ld
    // floats; 0 means K and K/128).
    PagedLayer Ls;
    float* lat_scale;
    int nblk;
    int q_ld, qs_ld;
};

struct KvMatmulArgs {
    const uint16_t* H;         // hidden_state bf16 [T][Kd]
    const uint32_t* iro;       // input_row_offsets [batch+1]
    const uint16_t* W;         // weight bf16 [Kd][N]
    const uint32_t* cache_len; // [batch]
    PagedLayer L;              // layer view of the K/V pool
    int T, Kd, N, HD;          // N = 2*HD
};

struct LatentWriteArgs {
    const uint16_t* X;         // new tokens' rows, bf16 [T][D] (latent K, then rope R)
    const uint32_t* iro;       // input_row_offsets [batch+1]
    const uint32_t* cache_len; // [batch] positions already cached
    const float* gamma;        // RMSNorm weights [K]
    const float* freqs;        // [max_seq][R]: (cos, sin) pairs per position
    float eps;
    PagedLayer L;              // layer view of the latent pool
    int T, K, R, D, max_seq;
    // e4m3 cache only: the scale pool's layer view (one fp32 per 128 columns
    // of a token row, byte strides).
    PagedLayer Ls;
};

struct AbsorbArgs {
    const uint16_t* q;         // bf16 [T][H][Dq]: 128 nope columns, then rope
    const uint16_t* w;         // w_uk bf16 [H][NL][128]
    const uint8_t* wq;         // fp8 form: w_uk e4m3 codes [H][NL][128]
    const float* wscale;       // fp8 form: [H][NL / 128] (one 128 x 128 block per latent tile)
    uint16_t* out;             // bf16 [T][H][Do]: NL latent columns, then R rope columns
    int T, H, NL, Dq, Do, R;   // R: rope columns copied (0: none)
};

hipError_t launch_gather_rows(const DecompressArgs& a, int elem_bytes, hipStream_t s);
hipError_t launch_absorb_bf16(const AbsorbArgs& a, hipStream_t s);
hipError_t launch_absorb_fp8(const AbsorbArgs& a, hipStream_t s);
hipError_t launch_latent_write(const LatentWriteArgs& a, hipStream_t s);
hipError_t launch_latent_write_fp8(const LatentWriteArgs& a, hipStream_t s);
hipError_t launch_product_bf16(const DecompressArgs& a, hipStream_t s);
hipError_t launch_product_f32(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_bf16(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_f32(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_fp8(const DecompressArgs& a, hipStream_t s);
// Fused K and V forms: one gather (and quantisation), both projections.
hipError_t launch_decompress_kv_bf16(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_kv_f32(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_kv_fp8(const DecompressArgs& a, hipStream_t s);
hipError_t launch_decompress_fp8_cache(const DecompressArgs& a, hipStream_t s);
// The same arguments with the second projection moved into the first slot.
inline DecompressArgs second_projection(const DecompressArgs& a)
{
    DecompressArgs b = a;
    b.W = a.W2;
    b.W_scale = a.W2_scale;
    b.out = a.out2;
    b.N = a.N2;
    b.W2 = nullptr;
    b.W2_scale = nullptr;
    b.out2 = nullptr;
    b.N2 = 0;
    return b;
}
inline DecompressArgs first_projection(const DecompressArgs& a)
{
    DecompressArgs b = a;
    b.W2 = nullptr;
    b.W2_scale = nullptr;
    b.out2 = nullptr;
    b.N2 = 0;
    return b;
}
hipError_t launch_kv_matmul(const KvMatmulArgs& a, hipStream_t s);
hipError_t launch_product_fp8_ring(const DecompressArgs& a, int cus, hipStream_t s);
hipError_t launch_kv_matmul_ring(const KvMatmulArgs& a, int cus, hipStream_t s);
constexpr int kRingTileN = 256;   // N-tile width of the bf16 ring kernel
int num_cus();
bool small_bf16_fits(const DecompressArgs& a);

// With MLA_PAGED_LOG set in the environment (to anything but "0", read once),
// every kernel launch prints one line to stderr: the kernel, its grid and
// block sizes and its shape parameters (printf-style).  Otherwise nothing.
void log_launch(const char* kernel, unsigned grid, unsigned block, const char* fmt, ...)
    __attribute__((format(printf, 4, 5)));
hipError_t launch_small_bf16(const DecompressArgs& a, int gather, hipStream_t s);
// Few-rows fp8 product (at most 192 rows, K = 512, one projection) from the
// activation codes and scales in a.q / a.q_scale.
bool small_fp8_fits(const DecompressArgs& a);
hipError_t launch_small_fp8(const DecompressArgs& a, hipStream_t s);
// At most 64 rows from a bf16 cache gathered, quantised and multiplied in one
// launch (K = 512, one projection); the workspace codes and scales are written too.
bool small_fp8_gq_fits(const DecompressArgs& a);
hipError_t launch_small_fp8_gq(const DecompressArgs& a, hipStream_t s);
// The same for at most 64 rows of an e4m3 cache (codes and scales gathered, no
// quantisation).
bool small_fp8_gc_fits(const DecompressArgs& a);
hipError_t launch_small_fp8_gc(const DecompressArgs& a, hipStream_t s);

}  // namespace mla
