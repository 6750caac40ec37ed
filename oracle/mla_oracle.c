/*
 * mla_oracle.c -- CPU oracle for the paged MLA latent-K path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP library; both sides only take
 * their inputs from the same seeded generators.
 *
 * It is deliberately plain and slow: scalar loops in the order the operations
 * are defined, products summed in binary64 in k order, OpenMP only over
 * independent output rows.  Build with gcc -O2 -ffp-contract=off, no fast-math.
 *
 * Sources (MAX kernel API pages):
 *  - "generic_flare_mla_decompress_k_cache_ragged_paged", summary and Args:
 *    latent K rows are gathered per request from the paged cache into
 *    k_latent_buffer (buffer_row_offsets give where each request's rows go,
 *    cache_offsets the cache position the copy starts at), then multiplied by
 *    the weight to give k_buffer.
 *  - "mla_prefill_decode_graph_fp8", Parameters m/n/k_scale_granularity and Args
 *    w_k [num_heads*qk_nope_head_dim, kv_latent_dim], w_k_scale: the fp8
 *    block-scaled form of the same up-projection.
 *  - "kv_matmul_ragged_paged", summary and Args: hidden_state times weight,
 *    written into the paged K/V cache of the layer.
 *
 * Parity pins: every function here is checked in tests/test_oracle_*.py
 * against something other than itself (library routines, closed forms,
 * special cases, invariants); see the docstrings of those tests.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * Number formats.
 * ---------------------------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE-754 binary32: decode by placing the
 * 16 bits above 16 zero bits. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP OFP8 E4M3 ("fn": finite only): sign, 4 exponent bits with bias 7,
 * 3 mantissa bits.  Exponent field 0 is subnormal (2^-6 * m/8); the single
 * NaN per sign is exponent 15 with mantissa 7; there is no infinity, so the
 * largest finite magnitude is 2^8 * 1.75 = 448. */
static double e4m3_to_double(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* float -> e4m3fn: the representable value nearest to x, ties to the code with
 * an even mantissa; magnitudes past 448 saturate to 448; NaN gives 0x7F.  The
 * non-negative finite codes 0x00..0x7E are increasing in value, so the nearest
 * one is found by bisection over the codes themselves. */
static uint8_t float_to_e4m3(float x)
{
    if (isnan(x))
        return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_to_double((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - e4m3_to_double((uint8_t)lo);
    double dhi = e4m3_to_double((uint8_t)hi) - a;
    int code;
    if (dlo < dhi)
        code = lo;
    else if (dhi < dlo)
        code = hi;
    else
        code = (lo & 1) ? hi : lo;
    return sign | (uint8_t)code;
}

/* element of a buffer of the given type as a double */
enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

static double elem(const void* base, int dtype, int64_t i)
{
    switch (dtype) {
    case OR_F32: return (double)f32_from_bits(((const uint32_t*)base)[i]);
    case OR_BF16: return (double)bf16_to_float(((const uint16_t*)base)[i]);
    default: return e4m3_to_double(((const uint8_t*)base)[i]);
    }
}

/* exported codecs, so the tests can pin them against torch's casts */
void or_bf16_decode(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_to_float(in[i]);
}

void or_e4m3_decode(const uint8_t* in, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_to_double(in[i]);
}

void or_e4m3_encode(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = float_to_e4m3(in[i]);
}

/* ------------------------------------------------------------------------
 * Paged cache addressing.
 *
 * The pool is indexed [page][layer][kv][slot][...row...] through element
 * strides; a request's logical token position p lives in physical page
 * page_table[b][p / page_size] at slot p % page_size.
 * ---------------------------------------------------------------------- */
typedef struct {
    int64_t stride_page, stride_layer, stride_kv, stride_token; /* elements */
    uint32_t num_pages, num_layers, page_size;
    const uint32_t* page_table; /* [batch][max_pages] */
    uint32_t max_pages;
} or_pool_t;

/* element offset of token position p of request b (kv half kv), or -1 when the
 * position has no page or the page id is out of range */
static int64_t token_offset(const or_pool_t* P, uint32_t b, int64_t p, uint32_t layer, uint32_t kv)
{
    int64_t lp = p / P->page_size;
    if (p < 0 || lp >= P->max_pages)
        return -1;
    uint32_t pg = P->page_table[(int64_t)b * P->max_pages + lp];
    if (pg >= P->num_pages)
        return -1;
    return (int64_t)pg * P->stride_page + (int64_t)layer * P->stride_layer +
           (int64_t)kv * P->stride_kv + (p % P->page_size) * P->stride_token;
}

/* ------------------------------------------------------------------------
 * Gather ("...decompress_k_cache_ragged_paged", summary; Args
 * buffer_row_offsets_1d, cache_offsets_1d, buffer_length, k_latent_buffer).
 *
 * For request b and i < rows_b = buffer_row_offsets[b+1] - buffer_row_offsets[b]:
 * the cache row at position cache_offsets[b] + i is copied bit for bit to
 * k_latent_buffer row buffer_row_offsets[b] + i (row_elems elements).
 *
 * Returns 0, or -1 offsets not starting at 0 / decreasing, -2 the last offset
 * differs from buffer_length, -3 a read past a request's cached length,
 * -4 a missing or out-of-range page, -5 bad layer.
 * ---------------------------------------------------------------------- */
int or_gather(const uint8_t* pool, int elem_bytes,
              int64_t stride_page, int64_t stride_layer, int64_t stride_token,
              uint32_t num_pages, uint32_t num_layers, uint32_t page_size,
              const uint32_t* page_table, uint32_t max_pages, uint32_t batch,
              const uint32_t* cache_lengths,
              const uint32_t* buffer_row_offsets, const uint32_t* cache_offsets,
              int64_t buffer_length, uint32_t layer, int64_t row_elems,
              uint8_t* k_latent)
{
    or_pool_t P = {stride_page, stride_layer, 0, stride_token, num_pages, num_layers,
                   page_size, page_table, max_pages};
    if (layer >= num_layers)
        return -5;
    if (buffer_row_offsets[0] != 0)
        return -1;
    for (uint32_t b = 0; b < batch; ++b)
        if (buffer_row_offsets[b + 1] < buffer_row_offsets[b])
            return -1;
    if ((int64_t)buffer_row_offsets[batch] != buffer_length)
        return -2;
    for (uint32_t b = 0; b < batch; ++b) {
        int64_t rows = (int64_t)buffer_row_offsets[b + 1] - buffer_row_offsets[b];
        if (cache_lengths && (int64_t)cache_offsets[b] + rows > (int64_t)cache_lengths[b])
            return -3;
        for (int64_t i = 0; i < rows; ++i) {
            int64_t src = token_offset(&P, b, (int64_t)cache_offsets[b] + i, layer, 0);
            if (src < 0)
                return -4;
            int64_t dst = ((int64_t)buffer_row_offsets[b] + i) * row_elems;
            memcpy(k_latent + dst * elem_bytes, pool + src * elem_bytes,
                   (size_t)(row_elems * elem_bytes));
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Up-projection (same page, summary; "mla_prefill_decode_graph_fp8", Args w_k:
 * shape [num_heads*qk_nope_head_dim, kv_latent_dim]).
 *
 * out[j][n] = sum_{k<K} A[rows[j]][k] * W[n][k]   (y = A W^T over the first K
 * columns of each gathered row), summed in binary64 in k order.
 * ---------------------------------------------------------------------- */
void or_matmul_nt(const void* A, int a_dtype, int64_t lda,
                  const void* W, int w_dtype, int64_t ldw,
                  int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows[j];
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += elem(A, a_dtype, r * lda + k) * elem(W, w_dtype, n * ldw + k);
            out[j * N + n] = s;
        }
    }
}

/* ------------------------------------------------------------------------
 * fp8 block-scaled up-projection ("mla_prefill_decode_graph_fp8", Parameters
 * fp8_dtype, fp8_scale_dtype, m/n/k_scale_granularity; Args w_k, w_k_scale).
 *
 * Activation quantisation, per row and per block of k_gran columns (m
 * granularity 1): amax = max |x| in binary32; the scale is s = amax / 448 and
 * the codes are e4m3fn(x * (448 / amax)), both quotients rounded to binary32;
 * an all-zero block takes s = 1 and codes 0.  448 is the largest e4m3fn value,
 * so the largest magnitude of the block maps onto it.
 * ---------------------------------------------------------------------- */
void or_quantize_e4m3_rows(const uint16_t* A_bf16, int64_t lda, int64_t M, int64_t K,
                           int64_t k_gran, uint8_t* q, float* s)
{
    int64_t nkb = (K + k_gran - 1) / k_gran;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t k0 = kb * k_gran, k1 = k0 + k_gran < K ? k0 + k_gran : K;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(bf16_to_float(A_bf16[r * lda + k]));
                if (a > amax)
                    amax = a;
            }
            float scale = 1.0f, inv = 1.0f;
            if (amax > 0.0f) {
                scale = amax / 448.0f;
                inv = 448.0f / amax;
            }
            s[r * nkb + kb] = scale;
            for (int64_t k = k0; k < k1; ++k) {
                float x = bf16_to_float(A_bf16[r * lda + k]);
                float y = x * inv;
                q[r * K + k] = float_to_e4m3(y);
            }
        }
    }
}

/* ------------------------------------------------------------------------
 * Quantisation of binary32 rows into an e4m3fn paged cache (the collection's
 * scale_dtype_ fp32 and quantization_granularity_ of page
 * "generic_flare_mla_decompress_k_cache_ragged_paged"): the same rule as the
 * activation quantisation above, per row and per block of gran columns (the
 * last block may be shorter): amax = max |y| over the block, s = amax / 448,
 * codes e4m3fn(y * (448 / amax)), quotients rounded to binary32; an all-zero
 * block takes s = 1 and codes 0.
 * ---------------------------------------------------------------------- */
void or_quantize_f32_rows(const float* Y, int64_t T, int64_t D, int64_t gran, uint8_t* q, float* s)
{
    int64_t nb = (D + gran - 1) / gran;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < T; ++r) {
        for (int64_t kb = 0; kb < nb; ++kb) {
            int64_t k0 = kb * gran, k1 = k0 + gran < D ? k0 + gran : D;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(Y[r * D + k]);
                if (a > amax)
                    amax = a;
            }
            float block_scale = 1.0f, to_codes = 1.0f;
            if (amax > 0.0f) {
                block_scale = amax / 448.0f;
                to_codes = 448.0f / amax;
            }
            s[r * nb + kb] = block_scale;
            for (int64_t k = k0; k < k1; ++k)
                q[r * D + k] = float_to_e4m3(Y[r * D + k] * to_codes);
        }
    }
}

/* out[j][n] = sum_kb s_a[r][kb] * s_w[n/n_gran][kb] * sum_{k in block kb} qa[r][k] qw[n][k]
 * with the codes decoded exactly and everything summed in binary64. */
void or_fp8_matmul_nt(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                      int64_t N, int64_t K, int64_t n_gran, int64_t k_gran,
                      const int64_t* rows, int64_t nrows, double* out)
{
    int64_t nkb = (K + k_gran - 1) / k_gran;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows[j];
        for (int64_t n = 0; n < N; ++n) {
            double total = 0.0;
            for (int64_t kb = 0; kb < nkb; ++kb) {
                int64_t k0 = kb * k_gran, k1 = k0 + k_gran < K ? k0 + k_gran : K;
                double part = 0.0;
                for (int64_t k = k0; k < k1; ++k)
                    part += e4m3_to_double(qa[r * K + k]) * e4m3_to_double(qw[n * K + k]);
                total += (double)sa[r * nkb + kb] * (double)sw[(n / n_gran) * nkb + kb] * part;
            }
            out[j * N + n] = total;
        }
    }
}

/* ------------------------------------------------------------------------
 * Write path ("kv_matmul_ragged_paged", summary and Args hidden_state
 * (sum(seq_lens), num_heads*head_size), input_row_offsets, weight
 * (num_heads*head_size, num_kv_heads*head_size), kv_collection).
 *
 * out[j][n] = sum_k hidden[rows[j]][k] * W[k][n]   (y = hidden W), binary64.
 * ---------------------------------------------------------------------- */
void or_matmul_nn(const uint16_t* H, int64_t ldh, const uint16_t* W, int64_t ldw,
                  int64_t N, int64_t K, const int64_t* rows, int64_t nrows, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t r = rows[j];
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += (double)bf16_to_float(H[r * ldh + k]) * (double)bf16_to_float(W[k * ldw + n]);
            out[j * N + n] = s;
        }
    }
}

/* Where the write path puts each token.  Token t of request b (t in
 * [input_row_offsets[b], input_row_offsets[b+1])) is appended after the
 * request's cached tokens: position p = cache_lengths[b] + (t - offsets[b]).
 * Its K row (output columns [0, N/2)) goes to kv half 0 and its V row (columns
 * [N/2, N)) to kv half 1 of that slot.  dst[t][kv] = element offset of the row.
 * Returns 0 or -4 for a position without a valid page. */
int or_kv_destinations(int64_t stride_page, int64_t stride_layer, int64_t stride_kv,
                       int64_t stride_token, uint32_t num_pages, uint32_t num_layers,
                       uint32_t page_size, const uint32_t* page_table, uint32_t max_pages,
                       uint32_t batch, const uint32_t* cache_lengths,
                       const uint32_t* input_row_offsets, uint32_t layer, int64_t* dst)
{
    or_pool_t P = {stride_page, stride_layer, stride_kv, stride_token, num_pages, num_layers,
                   page_size, page_table, max_pages};
    if (layer >= num_layers)
        return -5;
    for (uint32_t b = 0; b < batch; ++b) {
        for (int64_t t = input_row_offsets[b]; t < (int64_t)input_row_offsets[b + 1]; ++t) {
            int64_t p = (int64_t)cache_lengths[b] + (t - (int64_t)input_row_offsets[b]);
            for (uint32_t kv = 0; kv < 2; ++kv) {
                int64_t o = token_offset(&P, b, p, layer, kv);
                if (o < 0)
                    return -4;
                dst[t * 2 + kv] = o;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Latent write path ("mla_prefill_decode_graph_fp8", Args kv_input_fn,
 * kv_norm_gamma, epsilon, freqs_cis).
 *
 * Row t of X (bf16, K latent then R rope columns) for position pos[t]:
 *   out[t][k]      = gamma[k] * x[k] / sqrt(sum_{k<K} x[k]^2 / K + eps)     k < K
 *   out[t][K+2j]   = x[K+2j] * c - x[K+2j+1] * s
 *   out[t][K+2j+1] = x[K+2j] * s + x[K+2j+1] * c,  c = freqs[pos][2j], s = freqs[pos][2j+1]
 * in binary64 (the caller rounds).  Returns 0, or -6 for a position at or past
 * max_seq.
 * ---------------------------------------------------------------------- */
int or_latent_rows(const uint16_t* X, int64_t T, int64_t K, int64_t R, const float* gamma, double eps,
                   const float* freqs, int64_t max_seq, const int64_t* pos, double* out)
{
    const int64_t D = K + R;
    for (int64_t t = 0; t < T; ++t)
        if (R > 0 && (pos[t] < 0 || pos[t] >= max_seq))
            return -6;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* x = X + t * D;
        double* y = out + t * D;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = bf16_to_float(x[k]);
            ss += v * v;
        }
        double rms = sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            y[k] = (double)gamma[k] * (double)bf16_to_float(x[k]) / rms;
        for (int64_t j = 0; 2 * j < R; ++j) {
            double x0 = bf16_to_float(x[K + 2 * j]), x1 = bf16_to_float(x[K + 2 * j + 1]);
            double c = freqs[pos[t] * R + 2 * j], s = freqs[pos[t] * R + 2 * j + 1];
            y[K + 2 * j] = x0 * c - x1 * s;
            y[K + 2 * j + 1] = x0 * s + x1 * c;
        }
    }
    return 0;
}
