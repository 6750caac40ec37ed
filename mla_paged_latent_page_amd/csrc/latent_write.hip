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
// out.  A wave owns 2 consecutive tokens: it puts both input rows in flight
// first (lane l holds latent values 8l .. 8l+7 of each, one 16-byte load; lanes
// 0 .. R/8-1 also hold 4 rope pairs), then finds the tokens' requests with one
// round of loads: lane j reads input_row_offsets[j], [j + 64], [j + 128] and
// [j + 192] (256 entries per pass), and the request of token t is the number
// of entries <= t, minus one, counted by ballots.  Then come the dependent
// loads of both tokens (cache length, page table, freqs_cis row), and only
// after them the stores.
//
// e4m3 cache (the collection's scale_dtype_ fp32 and quantization_granularity_
// 128 of page "generic_flare_mla_decompress_k_cache_ragged_paged"): the same
// fp32 values, quantised per 128-column block of the row (K % 128 == 0, so the
// rope columns start a block): amax over the block by DPP exchanges within
// 16 lanes (8 columns per lane), s = amax / 448 (1 for an all-zero block),
// codes e4m3fn(y * (448 / amax)) rounded to nearest even; each lane stores
// its 8 codes, the first lane of a block stores s into the scale pool.
#include "launch.hpp"

namespace mla {
namespace {

constexpr int WRITE_WAVES = 4;
constexpr int TOKENS_PER_WAVE = 2;

// Sum over the 64 lanes: within each 16-lane row by DPP (the exchanges of
// max16), then the four row sums read out of lanes 0, 16, 32 and 48.  Every
// lane gets the same total.
__device__ inline float wave_sum(float v)
{
    v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);   // row_half_mirror
    v += dpp_f32<0x140>(v);   // row_mirror
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}


// Amax of one 128-column block: 8 values per lane, 16 lanes per block.
__device__ inline float block_amax(const float (&y)[8])
{
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        am = fmaxf(am, fabsf(y[i]));
    return max16(am);
}

// Eight fp32 values of a block as e4m3 codes (packed little-endian) with the
// block's 448 / amax.
__device__ inline u32x2 codes8(const float (&y)[8], float to_codes)
{
    return {pack_e4m3x2(y[0] * to_codes, y[1] * to_codes) | (pack_e4m3x2(y[2] * to_codes, y[3] * to_codes) << 16),
            pack_e4m3x2(y[4] * to_codes, y[5] * to_codes) | (pack_e4m3x2(y[6] * to_codes, y[7] * to_codes) << 16)};
}

template <bool FP8>
__global__ void __launch_bounds__(64 * WRITE_WAVES) latent_write_kernel(LatentWriteArgs a)
{
    constexpr int TW = TOKENS_PER_WAVE;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = (blockIdx.x * WRITE_WAVES + wave) * TW;
    if (t0 >= a.T)
        return;
    const bool lat = lane * 8 < a.K;   // K <= 512: at most 64 lanes
    const bool rot = lane * 8 < a.R;   // R <= 512

    // Input rows of the wave's tokens (a tail wave re-reads its last token).
    u32x4 xv[TW], rv[TW];
#pragma unroll
    for (int k = 0; k < TW; ++k) {
        const int t = min(t0 + k, a.T - 1);
        const char* src = reinterpret_cast<const char*>(a.X) + (int64_t)t * a.D * 2;
        xv[k] = lat ? ld16(src + lane * 16) : u32x4{0u, 0u, 0u, 0u};
        rv[k] = rot ? ld16(src + a.K * 2 + lane * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    // Request of each token: entries b < batch with input_row_offsets[b] <= t
    // form a prefix (the offsets do not decrease); its last index is the
    // request (empty requests are skipped by taking the last).
    uint32_t cnt[TW];
#pragma unroll
    for (int k = 0; k < TW; ++k)
        cnt[k] = 0;
    for (uint32_t c = 0; c < a.L.batch; c += 256) {
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t j = c + u * 64 + lane;
            v[u] = j < a.L.batch ? a.iro[j] : 0xFFFFFFFFu;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < TW; ++k)
                cnt[k] += (uint32_t)__popcll(__ballot(v[u] <= (uint32_t)(t0 + k)));
    }

    // Per token: request, position, destination and its freqs_cis row, all
    // loaded before the first store.
    int64_t off[TW], soff[TW];
    f32x4 fr0[TW], fr1[TW];
#pragma unroll
    for (int k = 0; k < TW; ++k) {
        const uint32_t t = (uint32_t)min(t0 + k, a.T - 1);
        const uint32_t b = cnt[k] == 0 ? 0u : min(cnt[k], a.L.batch) - 1;
        const uint32_t p = a.cache_len[b] + (t - a.iro[b]);
        const uint32_t pf = p < (uint32_t)a.max_seq ? p : (uint32_t)a.max_seq - 1;   // freqs row, clamped
        off[k] = store_offset(a.L, b, p);   // -1: no slot for this position, nothing is stored
        soff[k] = FP8 ? store_offset(a.Ls, b, p) : 0;
        const float* f = a.freqs + (int64_t)pf * a.R + lane * 8;
        fr0[k] = rot ? *reinterpret_cast<const f32x4*>(f) : f32x4{0.f, 0.f, 0.f, 0.f};
        fr1[k] = rot ? *reinterpret_cast<const f32x4*>(f + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4 g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
    if (lat) {
        g0 = *reinterpret_cast<const f32x4*>(a.gamma + lane * 8);
        g1 = *reinterpret_cast<const f32x4*>(a.gamma + lane * 8 + 4);
    }
    const float gg[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};

#pragma unroll
    for (int k = 0; k < TW; ++k) {
        if (t0 + k >= a.T)
            break;
        if (off[k] < 0)
            continue;
        char* dst = const_cast<char*>(a.L.base) + off[k];

        // Latent part: RMS over the K latent values, scaled by gamma.
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(xv[k][i]);
            x[2 * i + 1] = bf16_hi(xv[k][i]);
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ss += x[i] * x[i];
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        float yl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            yl[i] = lat ? gg[i] * (x[i] * inv) : 0.0f;

        // Rope part: 4 pairs per lane with the 4 (cos, sin) pairs of freqs_cis row p.
        float yr[8];
        {
            const float cs[8] = {fr0[k][0], fr0[k][1], fr0[k][2], fr0[k][3], fr1[k][0], fr1[k][1], fr1[k][2], fr1[k][3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = bf16_lo(rv[k][i]), x1 = bf16_hi(rv[k][i]);
                const float c = cs[2 * i], s = cs[2 * i + 1];
                yr[2 * i] = rot ? x0 * c - x1 * s : 0.0f;
                yr[2 * i + 1] = rot ? x0 * s + x1 * c : 0.0f;
            }
        }

        if constexpr (!FP8) {
            if (lat) {
                u32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = pack_bf16x2(yl[2 * i], yl[2 * i + 1]);
                st16(dst + lane * 16, y);
            }
            if (rot) {
                u32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = pack_bf16x2(yr[2 * i], yr[2 * i + 1]);
                st16(dst + a.K * 2 + lane * 16, y);
            }
        } else {
            // Codes at byte 8 lane (latent) and K + 8 lane (rope); block j of
            // the row is lanes 16 j .. 16 j + 15 of the latent part, and block
            // K / 128 + j lanes 16 j .. of the rope part.  Lanes past the row
            // hold zeros, which leave every amax unchanged.
            float* sdst = reinterpret_cast<float*>(const_cast<char*>(a.Ls.base) + soff[k]);
            // Scale s = amax / 448 (1 for an all-zero block) and 448 / amax of
            // the lane's latent and rope blocks: even lanes divide for the
            // latent block, odd lanes for the rope block, and every lane takes
            // both results from lanes 0 and 1 of its 16-lane row (one pair of
            // IEEE divisions per lane instead of two).
            const float aml = block_amax(yl), amr = block_amax(yr);
            const float am = (lane & 1) ? amr : aml;
            float sc = 1.0f, to = 1.0f;
            if (am > 0.0f) {
                sc = am / 448.0f;
                to = 448.0f / am;
            }
            const float sl = row16_lane(sc, 0), sr = row16_lane(sc, 1);
            const u32x2 cl = codes8(yl, row16_lane(to, 0)), cr = codes8(yr, row16_lane(to, 1));
            if (lat) {
                *reinterpret_cast<u32x2*>(dst + lane * 8) = cl;
                if ((lane & 15) == 0)
                    sdst[lane >> 4] = sl;
            }
            if (rot) {
                *reinterpret_cast<u32x2*>(dst + a.K + lane * 8) = cr;
                if ((lane & 15) == 0)
                    sdst[a.K / 128 + (lane >> 4)] = sr;
            }
        }
    }
}

}  // namespace

hipError_t launch_latent_write(const LatentWriteArgs& a, hipStream_t s)
{
    constexpr int per_block = WRITE_WAVES * TOKENS_PER_WAVE;
    log_launch("latent_write_kernel<bf16>", (a.T + per_block - 1) / per_block, 64 * WRITE_WAVES, "T=%d K=%d R=%d", a.T, a.K, a.R);
    hipLaunchKernelGGL(latent_write_kernel<false>, dim3((a.T + per_block - 1) / per_block), dim3(64 * WRITE_WAVES), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_latent_write_fp8(const LatentWriteArgs& a, hipStream_t s)
{
    constexpr int per_block = WRITE_WAVES * TOKENS_PER_WAVE;
    log_launch("latent_write_kernel<e4m3>", (a.T + per_block - 1) / per_block, 64 * WRITE_WAVES, "T=%d K=%d R=%d", a.T, a.K, a.R);
    hipLaunchKernelGGL(latent_write_kernel<true>, dim3((a.T + per_block - 1) / per_block), dim3(64 * WRITE_WAVES), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace mla
