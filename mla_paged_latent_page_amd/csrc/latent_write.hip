// Latent write path: the rows the decompress path gathers, produced from new
// tokens (page "mla_prefill_decode_graph_fp8", Args kv_input_fn (the latent
// values, [tot_seq_len, cache_head_dim], cache_head_dim = kv_lora_rank +
// qk_rope_head_dim), kv_norm_gamma [kv_lora_rank], epsilon, freqs_cis
// [max_seq_len, qk_rope_head_dim], input_row_offsets, kv_collection).
//
// Token t of request b (input_row_offsets[b] <= t < input_row_offsets[b+1])
// goes to position p = cache_lengths[b] + (t - input_row_offsets[b]):
//   latent part  y[k] = gamma[k] * x[k] / sqrt(mean_k x[k]^2 + epsilon)     (k < K)
//   rope part    (y[K+2j], y[K+2j+1]) = (x0 c - x1 s, x0 s + x1 c),
//                x0 = x[K+2j], x1 = x[K+2j+1], (c, s) = freqs_cis[p][2j], [2j+1]
// computed in fp32 and stored, rounded to bf16, as the cache row of position p.
//
// HBM-bound: per token one 1152-byte row in, 256 bytes of freqs_cis, one row
// out.  One wave per token: lane l holds latent values 8l .. 8l+7 (one
// 16-byte load), the wave's sum of squares is a butterfly over the 64 lanes,
// and lanes 0 .. R/8-1 hold the rope part (4 pairs each) with their 4 (cos,
// sin) pairs of the position's freqs_cis row.
#include "launch.hpp"

namespace mla {
namespace {

constexpr int WRITE_WAVES = 4;

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__global__ void __launch_bounds__(64 * WRITE_WAVES) latent_write_kernel(LatentWriteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * WRITE_WAVES + (threadIdx.x >> 6);
    if (t >= a.T)
        return;
    const uint32_t b = find_request(a.iro, a.L.batch, (uint32_t)t);
    const uint32_t p = a.cache_len[b] + ((uint32_t)t - a.iro[b]);
    const uint32_t pf = p < (uint32_t)a.max_seq ? p : (uint32_t)a.max_seq - 1;   // freqs row, clamped
    char* dst = const_cast<char*>(a.L.base) + token_offset(a.L, b, p);
    const char* src = reinterpret_cast<const char*>(a.X) + (int64_t)t * a.D * 2;

    // Latent part: K / 8 lanes hold 8 values each (K <= 512).
    const bool lat = lane * 8 < a.K;
    u32x4 xv = lat ? ld16(src + lane * 16) : u32x4{0u, 0u, 0u, 0u};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(xv[i]);
        x[2 * i + 1] = bf16_hi(xv[i]);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        ss += x[i] * x[i];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    if (lat) {
        const float* g = a.gamma + lane * 8;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(g), g1 = *reinterpret_cast<const f32x4*>(g + 4);
        const float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        u32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            y[i] = pack_bf16x2(gg[2 * i] * (x[2 * i] * inv), gg[2 * i + 1] * (x[2 * i + 1] * inv));
        st16(dst + lane * 16, y);
    }

    // Rope part: R / 8 lanes hold 4 pairs each, with the 4 (cos, sin) pairs of
    // freqs_cis row p.
    if (lane * 8 < a.R) {
        const u32x4 rv = ld16(src + a.K * 2 + lane * 16);
        const float* f = a.freqs + (int64_t)pf * a.R + lane * 8;
        const f32x4 f0 = *reinterpret_cast<const f32x4*>(f), f1 = *reinterpret_cast<const f32x4*>(f + 4);
        const float cs[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
        u32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = bf16_lo(rv[i]), x1 = bf16_hi(rv[i]);
            const float c = cs[2 * i], s = cs[2 * i + 1];
            y[i] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
        }
        st16(dst + a.K * 2 + lane * 16, y);
    }
}

}  // namespace

hipError_t launch_latent_write(const LatentWriteArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(latent_write_kernel, dim3((a.T + WRITE_WAVES - 1) / WRITE_WAVES), dim3(64 * WRITE_WAVES), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace mla
