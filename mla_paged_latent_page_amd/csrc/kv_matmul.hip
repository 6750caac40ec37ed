// Projection of hidden states into the paged K/V cache for gfx950 (page
// "kv_matmul_ragged_paged", summary and Args hidden_state (sum(seq_lens),
// num_heads*head_size), input_row_offsets, weight (num_heads*head_size,
// num_kv_heads*head_size), kv_collection, layer_idx).
//
//   out[t][n] = sum_k H[t][k] * W[k][n]   (fp32 accumulate, bf16 RNE into the cache)
//   token t of request b goes to position cache_lengths[b] + (t - row_offsets[b]);
//   columns [0, HD) form its K row, [HD, 2HD) its V row.
//
// Same MFMA core as the decompress kernel (bf16 32x32x16, weight as the row
// operand, swizzled double-buffered LDS, LDS-staged epilogue).  The weight is
// [K][N] with N contiguous while the MFMA wants 8 consecutive k per lane, so
// each thread loads a KR x 8 block (KR rows of 16 bytes) and transposes it in
// registers into 8 column pieces of KR k-values before writing LDS [n][k].
// The epilogue resolves each tile row to its cache slot once (request search,
// then page table) and writes 16-byte pieces of the K and V rows straight into
// the pages; a 256-wide column tile maps to 512 contiguous bytes of one row.
#include "launch.hpp"

namespace mla {
namespace {

template <int BM, int BN, int WM, int WN>
struct KvTile {
    static constexpr int BK = 64;
    static constexpr int GPR = BK / 8;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int RP = NT / GPR;
    static constexpr int AR = BM / RP;
    static constexpr int KR = (BK / 8) * (BN / 8) >= NT ? 8 : 4;   // k rows per weight piece
    static constexpr int PIECES = (BK / KR) * (BN / 8);
    static constexpr int PT = PIECES / NT;                        // pieces per thread
    static constexpr int TM = BM / WM;
    static constexpr int TN = BN / WN;
    static constexpr int FM = TM / 32;
    static constexpr int FN = TN / 32;
    static constexpr int A_STAGE = BM * BK;
    static constexpr int B_STAGE = BN * BK;
    static constexpr int MAIN_LDS = 2 * (A_STAGE + B_STAGE) * 2;
    static constexpr int EPI_LDS = BM * BN * 2;
    static constexpr int LDS = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
    static constexpr int CG = BN / 8;
    static_assert(NT % GPR == 0 && BM % RP == 0, "loader shape");
    static_assert(PIECES % NT == 0 && PT >= 1, "weight loader shape");
    static_assert((CG & (CG - 1)) == 0, "output tile width");
};

struct KvParams {
    KvMatmulArgs a;
    int tiles_m, tiles_n;
    int xcd_map;
};

// Column c (0..7) of a KR x 8 block of bf16 held as KR rows of 4 dwords:
// dword d of the result packs rows 2d and 2d+1 of that column.
template <int KR>
__device__ inline void transpose_piece(const u32x4 (&in)[KR], uint32_t (&outw)[8][KR / 2])
{
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int d = 0; d < KR / 2; ++d) {
            const uint32_t lo = in[2 * d][c >> 1], hi = in[2 * d + 1][c >> 1];
            outw[c][d] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
kv_matmul_kernel(KvParams P)
{
    using T = KvTile<BM, BN, WM, WN>;
    constexpr int BK = T::BK, GPR = T::GPR, NT = T::NT, RP = T::RP, KR = T::KR;
    __shared__ __attribute__((aligned(16))) char smem[T::LDS + BM * 8];
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);
    uint16_t* Bs = As + 2 * T::A_STAGE;
    int64_t* rowoff = reinterpret_cast<int64_t*>(smem + T::LDS);

    const KvMatmulArgs& a = P.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of_block(blockIdx.x, P.tiles_m, P.tiles_n, P.xcd_map, tm, tn);
    const int t0 = tm * BM, n0 = tn * BN;

    // Cache slot (K half) of every token of the tile; -1 past the last token.
    for (int r = tid; r < BM; r += NT) {
        const int t = t0 + r;
        int64_t off = -1;
        if (t < a.T) {
            const uint32_t b = find_request(a.iro, a.L.batch, (uint32_t)t);
            const uint32_t p = a.cache_len[b] + ((uint32_t)t - a.iro[b]);
            off = store_offset(a.L, b, p);
        }
        rowoff[r] = off;
    }

    const int gcol = tid % GPR, rsub = tid / GPR;
    const char* hrow[T::AR];
#pragma unroll
    for (int j = 0; j < T::AR; ++j) {
        int t = t0 + rsub + j * RP;
        t = t < a.T ? t : a.T - 1;
        hrow[j] = reinterpret_cast<const char*>(a.H) + ((int64_t)t * a.Kd + gcol * 8) * 2;
    }
    // weight pieces: piece p -> k rows (p % (BK/KR))*KR .. +KR, columns (p / (BK/KR))*8 .. +8
    constexpr int KQ = BK / KR;
    uint32_t woff[T::PT];
    int pk[T::PT], pn[T::PT];
#pragma unroll
    for (int q = 0; q < T::PT; ++q) {
        const int piece = tid + q * NT;
        pk[q] = piece % KQ;
        pn[q] = piece / KQ;
        int n = n0 + pn[q] * 8;
        n = n < a.N ? n : a.N - 8;
        woff[q] = (uint32_t)(((int64_t)pk[q] * KR * a.N + n) * 2);
    }
    const char* wbase = reinterpret_cast<const char*>(a.W);
    const int64_t wstage = (int64_t)BK * a.N * 2;  // bytes between k stages

    u32x4 ra[T::AR];
    u32x4 rw[T::PT][KR];
    auto gload = [&](int kt) {
        const int kb = kt * BK * 2;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) ra[j] = ld16(hrow[j] + kb);
#pragma unroll
        for (int q = 0; q < T::PT; ++q)
#pragma unroll
            for (int i = 0; i < KR; ++i)
                rw[q][i] = ld16(wbase + kt * wstage + woff[q] + (int64_t)i * a.N * 2);
    };
    auto lstore = [&](int buf) {
        uint16_t* as = As + buf * T::A_STAGE;
        uint16_t* bs = Bs + buf * T::B_STAGE;
#pragma unroll
        for (int j = 0; j < T::AR; ++j) {
            const int r = rsub + j * RP;
            lds_st16(as + r * BK + swz(r, gcol, GPR) * 8, ra[j]);
        }
#pragma unroll
        for (int q = 0; q < T::PT; ++q) {
            uint32_t tw[8][KR / 2];
            transpose_piece<KR>(rw[q], tw);
            const int kg = (pk[q] * KR) / 8, half = (pk[q] * KR) % 8;  // granule, element offset
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int n = pn[q] * 8 + c;
                uint16_t* dst = bs + n * BK + swz(n, kg, GPR) * 8 + half;
                if constexpr (KR == 8)
                    lds_st16(dst, u32x4{tw[c][0], tw[c][1], tw[c][2], tw[c][3]});
                else
                    lds_st8(dst, u32x2{tw[c][0], tw[c][1]});
            }
        }
    };

    f32x16 acc[T::FN][T::FM];
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
            acc[i][j] = f32x16{};

    const int KT = a.Kd / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint16_t* as = As + buf * T::A_STAGE;
        const uint16_t* bs = Bs + buf * T::B_STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int g = 2 * ks + (lane >> 5);
            bf16x8 fa[T::FN], fb[T::FM];
#pragma unroll
            for (int i = 0; i < T::FN; ++i) {
                const int n = wn * T::TN + i * 32 + (lane & 31);
                fa[i] = as_bf16x8(lds_ld16(bs + n * BK + swz(n, g, GPR) * 8));
            }
#pragma unroll
            for (int j = 0; j < T::FM; ++j) {
                const int m = wm * T::TM + j * 32 + (lane & 31);
                fb[j] = as_bf16x8(lds_ld16(as + m * BK + swz(m, g, GPR) * 8));
            }
#pragma unroll
            for (int i = 0; i < T::FN; ++i)
#pragma unroll
                for (int j = 0; j < T::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) lstore(buf ^ 1);
        __syncthreads();
    }

    uint16_t* Cs = reinterpret_cast<uint16_t*>(smem);
    constexpr int CG = T::CG;
#pragma unroll
    for (int i = 0; i < T::FN; ++i)
#pragma unroll
        for (int j = 0; j < T::FM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wm * T::TM + j * 32 + (lane & 31);
                const int n = wn * T::TN + i * 32 + 8 * q + 4 * (lane >> 5);
                u32x2 v;
                v[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                v[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                lds_st8(Cs + m * BN + swz(m, n >> 3, CG) * 8 + (n & 7), v);
            }
    __syncthreads();
    char* pool = const_cast<char*>(a.L.base);
    for (int idx = tid; idx < BM * CG; idx += NT) {
        const int r = idx / CG, g = idx - r * CG;
        const int n = n0 + g * 8;
        const int64_t off = rowoff[r];
        if (off < 0 || n >= a.N)
            continue;
        const int kv = n >= a.HD ? 1 : 0;
        const int c = n - kv * a.HD;
        const u32x4 v = lds_ld16(Cs + r * BN + swz(r, g, CG) * 8);
        st16_nt(pool + off + kv * a.L.stride_kv + (int64_t)c * 2, v);
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const KvMatmulArgs& a, hipStream_t s)
{
    KvParams P;
    P.a = a;
    P.tiles_m = (a.T + BM - 1) / BM;
    P.tiles_n = (a.N + BN - 1) / BN;
    P.xcd_map = (P.tiles_n % 8 == 0) ? 1 : 0;
    log_launch("kv_matmul_kernel", P.tiles_m * P.tiles_n, 64 * WM * WN, "tiles=%dx%d tile=%dx%d", P.tiles_m, P.tiles_n, BM,
               BN);
    hipLaunchKernelGGL((kv_matmul_kernel<BM, BN, WM, WN>), dim3(P.tiles_m * P.tiles_n), dim3(64 * WM * WN), 0, s, P);
    return hipGetLastError();
}

}  // namespace

// The LDS-ring kernel when the shapes fit its tiling (hidden_dim % 128 == 0,
// HD % 256 == 0); the general tiled kernel above otherwise.
hipError_t launch_kv_matmul(const KvMatmulArgs& a, hipStream_t s)
{
    if (a.Kd % 128 == 0 && a.HD % 256 == 0)
        return launch_kv_matmul_ring(a, num_cus(), s);
    return launch_cfg<256, 256, 2, 4>(a, s);
}

}  // namespace mla
