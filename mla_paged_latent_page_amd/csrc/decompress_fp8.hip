// Paged gather + fp8 block-scaled up-projection for gfx950 (page
// "mla_prefill_decode_graph_fp8": Parameters fp8_dtype, fp8_scale_dtype,
// m/n/k_scale_granularity; Args w_k [num_heads*qk_nope_head_dim, kv_latent_dim],
// w_k_scale; granularities 1 x 128 for activations, 128 x 128 for the weight).
//
// Pass 1 (gather_quant_fp8_kernel), one wave per row: copy the cache row into
// k_latent, and quantise its first K columns per block of 128: amax by a
// 16-lane reduction, s = amax/448, codes = e4m3(x * (448/amax)) with the
// hardware round-to-nearest-even conversion.  Codes and scales go to the
// workspace.  Quantising once here, instead of inside every N-tile of the
// product, costs one extra write+read of M*K bytes but saves re-quantising
// each activation element N/BN times.
//
// Pass 2 (gemm_fp8_kernel): one v_mfma_scale_f32_16x16x128_f8f6f4 covers
// exactly one 128-wide K block, so each MFMA result is the block's partial sum;
// it is folded into the fp32 accumulator with one FMA by s_a[row][kb] *
// s_w[n/128][kb] (the fp32 scales are not powers of two, so the MFMA's own E8M0
// scale inputs stay at 1).  A wave's N range lies inside one 128-column weight
// block, so s_w is uniform per wave and K block.  Same LDS swizzle, epilogue and
// XCD-aware tile order as the bf16 kernel.
#include "launch.hpp"

namespace mla {
namespace {

__global__ void __launch_bounds__(256) gather_quant_fp8_kernel(DecompressArgs a)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.M)
        return;
    const uint32_t b = find_request(a.bro, a.L.batch, (uint32_t)r);
    const uint32_t p = a.co[b] + ((uint32_t)r - a.bro[b]);
    const char* src = a.L.base + token_offset(a.L, b, p);
    uint16_t* lat = static_cast<uint16_t*>(a.lat) + (int64_t)r * a.D;
    uint8_t* q = static_cast<uint8_t*>(a.q) + (int64_t)r * a.K;
    const int nkb = a.K / 128;
    float* qs = a.q_scale + (int64_t)r * nkb;

    for (int c0 = 0; c0 < a.K; c0 += 512) {
        const int c = c0 + lane * 8;
        const bool in = c < a.K;  // K % 128 == 0: whole 16-lane groups are in or out
        u32x4 v = in ? ld16(src + (int64_t)c * 2) : u32x4{0, 0, 0, 0};
        if (in)
            st16(lat + c, v);
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(v[i]);
            x[2 * i + 1] = bf16_hi(v[i]);
        }
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            am = fmaxf(am, fabsf(x[i]));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        am = fmaxf(am, __shfl_xor(am, 4));
        am = fmaxf(am, __shfl_xor(am, 8));
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
    for (int g = lane; g < (a.D - a.K) / 8; g += 64)
        st16(lat + a.K + g * 8, ld16(src + (int64_t)(a.K + g * 8) * 2));
}

template <int BM, int BN, int WM, int WN>
struct Fp8Tile {
    static constexpr int BK = 128;            // bytes == elements == one scale block
    static constexpr int GPR = BK / 16;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int RP = NT / GPR;
    static constexpr int AR = BM / RP;
    static constexpr int BR = BN / RP;
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int FM = TM / 16;
    static constexpr int FN = TN / 16;
    static constexpr int A_STAGE = BM * BK;   // bytes
    static constexpr int B_STAGE = BN * BK;
    static constexpr int MAIN_LDS = 2 * (A_STAGE + B_STAGE);
    static constexpr int EPI_LDS = BM * BN * 2;
    static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
    static constexpr int CG = BN / 8;
    static_assert(NT % GPR == 0 && BM % RP == 0 && BN % RP == 0, "loader shape");
    static_assert(128 % TN == 0, "a wave's columns must sit inside one 128-wide weight scale block");
    static_assert((CG & (CG - 1)) == 0, "output tile width");
};

struct Fp8Params {
    DecompressArgs a;
    int tiles_m, tiles_n;
    int xcd_map;
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_fp8_kernel(Fp8Params P)
{
    using T = Fp8Tile<BM, BN, WM, WN>;
    constexpr int BK = T::BK, GPR = T::GPR, NT = T::NT, RP = T::RP;
    __shared__ __attribute__((aligned(16))) char smem[T::LDS];
    char* As = smem;
    char* Bs = smem + 2 * T::A_STAGE;

    const DecompressArgs& a = P.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of_block(blockIdx.x, P.tiles_m, P.tiles_n, P.xcd_map, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nkb = a.K / 128;
    const char* qa = static_cast<const char*>(a.q);
    const char* qw = static_cast<const char*>(a.W);

    const int gcol = tid % GPR, rsub = tid / GPR;
    int64_t aoff[T::AR];
    uint32_t boff[T::BR];
#pragma unroll
    for (int j = 0; j < T::AR; ++j) {
        int m = m0 + rsub + j * RP;
        m = m < a.M ? m : a.M - 1;
        aoff[j] = (int64_t)m * a.K + gcol * 16;
    }
#pragma unroll
    for (int j = 0; j < T::BR; ++j) {
        int n = n0 + rsub + j * RP;
        n = n < a.N ? n : a.N - 1;
        boff[j] = (uint32_t)((int64_t)n * a.K + gcol * 16);
    }

    u32x4 ra[T::AR], rb[T::BR];
    auto gload = [&](int kt) {
        const int kb = kt * BK;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) ra[j] = ld16(qa + aoff[j] + kb);
#pragma unroll
        for (int j = 0; j < T::BR; ++j) rb[j] = ld16(qw + boff[j] + kb);
    };
    auto lstore = [&](int buf) {
        char* as = As + buf * T::A_STAGE;
        char* bs = Bs + buf * T::B_STAGE;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) {
            const int r = rsub + j * RP;
            lds_st16(as + r * BK + swz(r, gcol, GPR) * 16, ra[j]);
        }
#pragma unroll
        for (int j = 0; j < T::BR; ++j) {
            const int r = rsub + j * RP;
            lds_st16(bs + r * BK + swz(r, gcol, GPR) * 16, rb[j]);
        }
    };

    // rows of this lane's accumulators (clamped for the scale lookups)
    int mrow[T::FM];
#pragma unroll
    for (int j = 0; j < T::FM; ++j) {
        const int m = m0 + wm * T::TM + j * 16 + (lane & 15);
        mrow[j] = m < a.M ? m : a.M - 1;
    }
    int nblk = (n0 + wn * T::TN) / 128;
    const int nblk_max = (a.N - 1) / 128;
    nblk = nblk < nblk_max ? nblk : nblk_max;

    f32x4 acc[T::FN][T::FM];
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
            acc[i][j] = f32x4{};

    const int KT = a.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const float sw = a.W_scale[nblk * nkb + kt];
        float cs[T::FM];
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
            cs[j] = a.q_scale[(int64_t)mrow[j] * nkb + kt] * sw;

        const char* as = As + buf * T::A_STAGE;
        const char* bs = Bs + buf * T::B_STAGE;
        const int g0 = 2 * (lane >> 4);
        i32x8 fb[T::FM];
#pragma unroll
        for (int j = 0; j < T::FM; ++j) {
            const int m = wm * T::TM + j * 16 + (lane & 15);
            const u32x4 lo = lds_ld16(as + m * BK + swz(m, g0, GPR) * 16);
            const u32x4 hi = lds_ld16(as + m * BK + swz(m, g0 + 1, GPR) * 16);
            fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int i = 0; i < T::FN; ++i) {
            const int n = wn * T::TN + i * 16 + (lane & 15);
            const u32x4 lo = lds_ld16(bs + n * BK + swz(n, g0, GPR) * 16);
            const u32x4 hi = lds_ld16(bs + n * BK + swz(n, g0 + 1, GPR) * 16);
            const i32x8 fa = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
            for (int j = 0; j < T::FM; ++j) {
                const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fa, fb[j], f32x4{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] = fmaf(part[e], cs[j], acc[i][j][e]);
            }
        }
        if (kt + 1 < KT) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds D[n][m] for n = 4*(lane>>4) + e, m = lane & 15 in each 16x16 block.
    uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);
    constexpr int CG = T::CG;
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j) {
            const int m = wm * T::TM + j * 16 + (lane & 15);
            const int n = wn * T::TN + i * 16 + 4 * (lane >> 4);
            u32x2 v;
            v[0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            v[1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            lds_st8(Cs + m * BN + swz(m, n >> 3, CG) * 8 + (n & 7), v);
        }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(a.out);
    for (int idx = tid; idx < BM * CG; idx += NT) {
        const int r = idx / CG, g = idx - r * CG;
        const int m = m0 + r, n = n0 + g * 8;
        const u32x4 v = lds_ld16(Cs + r * BN + swz(r, g, CG) * 8);
        if (m < a.M && n < a.N)
            st16_nt(out + (int64_t)m * a.N + n, v);
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm(const DecompressArgs& a, hipStream_t s)
{
    Fp8Params P;
    P.a = a;
    P.tiles_m = (a.M + BM - 1) / BM;
    P.tiles_n = (a.N + BN - 1) / BN;
    P.xcd_map = (P.tiles_n % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((gemm_fp8_kernel<BM, BN, WM, WN>), dim3(P.tiles_m * P.tiles_n), dim3(64 * WM * WN), 0, s, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decompress_fp8(const DecompressArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(gather_quant_fp8_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    static const int cfg = [] {
        const char* v = getenv("MLA_PAGED_FP8_TILE");
        return v ? atoi(v) : 0;
    }();
    switch (cfg) {
    case 1: return launch_gemm<256, 128, 4, 2>(a, s);
    case 2: return launch_gemm<128, 256, 2, 4>(a, s);
    case 3: return launch_gemm<128, 128, 2, 2>(a, s);
    default:
        return launch_product_fp8_ring(first_projection(a), num_cus(), s);
    }
}

// fp8 cache: the gather copies each row's codes and scales bit for bit into
// k_latent_buffer and k_latent_scales, and the product reads them from there
// (row strides D bytes and nblk floats): the cache is already quantised, so
// there is no quantisation pass.
hipError_t launch_decompress_fp8_cache(const DecompressArgs& a, hipStream_t s)
{
    const hipError_t e = launch_gather_rows(a, 1, s);
    if (e != hipSuccess)
        return e;
    DecompressArgs p = a;   // both projections when a second one is present
    p.q = a.lat;
    p.q_scale = a.lat_scale;
    p.q_ld = a.D;
    p.qs_ld = a.nblk;
    return launch_product_fp8_ring(p, num_cus(), s);
}

// Fused K and V (fp8): one gather and quantisation pass, then one product
// launch over both projections' N-tiles.
hipError_t launch_decompress_kv_fp8(const DecompressArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(gather_quant_fp8_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, first_projection(a));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_product_fp8_ring(a, num_cus(), s);
}

}  // namespace mla
