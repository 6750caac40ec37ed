/*
 * mla_paged.h -- C ABI of the MI355X (gfx950) paged MLA latent-K library.
 *
 * Three operations, after the MAX kernel API pages (and the two steps of the
 * first one as calls of their own: mla_gather_latent_paged, mla_latent_matmul):
 *
 *   mla_decompress_k_paged      page "generic_flare_mla_decompress_k_cache_ragged_paged"
 *                               (summary; Args buffer_row_offsets_1d, cache_offsets_1d,
 *                               buffer_length, weight, kv_collection, layer_idx,
 *                               k_latent_buffer, k_buffer, context)
 *   mla_decompress_k_paged_fp8  the same operation with the fp8 block-scaled weight of
 *                               page "mla_prefill_decode_graph_fp8" (Parameters fp8_dtype,
 *                               fp8_scale_dtype, m/n/k_scale_granularity; Args w_k, w_k_scale)
 *   kv_matmul_paged             page "kv_matmul_ragged_paged" (summary; Args hidden_state,
 *                               input_row_offsets, weight, kv_collection, layer_idx, ctx)
 *
 * Conventions for every call:
 *   - Pointers marked [device] are HIP device pointers; [host] pointers are read
 *     during the call only.  The caller allocates and frees every buffer and keeps
 *     it valid until the work queued on `stream` has finished.
 *   - Matrices are row-major with the innermost dimension contiguous.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work:
 *     they never synchronise, never allocate device memory and keep no state
 *     between calls.  They are safe to call from several host threads.
 *   - Errors are returned synchronously, before anything is enqueued, in this
 *     order: host pointers and shapes (MLA_ERR_NULL_POINTER, MLA_ERR_INVALID_SHAPE,
 *     MLA_ERR_INVALID_DTYPE, MLA_ERR_MISALIGNED, MLA_ERR_OUT_OF_RANGE,
 *     MLA_ERR_WORKSPACE), then the current device (MLA_ERR_UNSUPPORTED_DEVICE unless
 *     it is a gfx950), then the launch (MLA_ERR_HIP; mla_last_hip_error() gives the
 *     hipError_t).  A call with no rows to process returns MLA_OK after the host
 *     checks and enqueues nothing.
 *   - With MLA_PAGED_LOG set in the environment (to anything but "0"; read once
 *     per process) every kernel launch prints one line to stderr naming the
 *     kernel, its grid and block sizes and its shapes.
 *   - Index contents in device memory (offsets, page ids) are the caller's
 *     contract and are not validated on the host.  Read paths clamp every page
 *     id, page index and row to the buffers they were given, so a bad index
 *     yields unspecified values in the output rows it affects but never an
 *     access outside the pool, the weight or the outputs.  Write paths
 *     (kv_matmul_paged, mla_write_latent_paged(_fp8)) store nothing for a token
 *     whose position lies past its request's page table or whose page id lies
 *     past the pool; every other byte of the pool keeps its value.
 *   - Shapes whose 256-row tiles would need byte offsets of 2^31 or more (a
 *     row of 2^22 bf16 elements in an output, a weight or the cache) return
 *     MLA_ERR_INVALID_SHAPE.
 */
#ifndef MLA_PAGED_H
#define MLA_PAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PAGED_ABI_VERSION 1

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL_POINTER = 1,
    MLA_ERR_INVALID_SHAPE = 2,
    MLA_ERR_INVALID_DTYPE = 3,
    MLA_ERR_MISALIGNED = 4,
    MLA_ERR_OUT_OF_RANGE = 5,
    MLA_ERR_WORKSPACE = 6,
    MLA_ERR_UNSUPPORTED_DEVICE = 7,
    MLA_ERR_HIP = 8
} mla_status_t;

typedef enum {
    MLA_DTYPE_F32 = 0,       /* IEEE binary32 */
    MLA_DTYPE_BF16 = 1,      /* bfloat16 */
    MLA_DTYPE_F8E4M3FN = 2   /* OCP OFP8 E4M3 (finite, max 448) */
} mla_dtype_t;

/*
 * A paged KV cache collection (the `kv_collection` + `layer_idx` of the pages):
 * one pool holds every layer.  Element (page, layer, kv, slot, i) of the pool is at
 *   blocks + page*stride_page + layer*stride_layer + kv*stride_kv + slot*stride_token + i
 * (strides in elements), where i < num_heads*head_dim indexes one token's row.
 * Token position p of request b lives in physical page page_table[b][p / page_size]
 * at slot p % page_size.
 */
typedef struct {
    void* blocks;                   /* [device] pool base; 16-byte aligned */
    int32_t dtype;                  /* mla_dtype_t of the pool: F32 or BF16 (F8E4M3FN with
                                       scales, mla_decompress_k_paged_fp8_cache only) */
    uint32_t num_layers;
    uint32_t num_pages;
    uint32_t page_size;             /* tokens per page, >= 1 */
    uint32_t num_kv;                /* 1 = MLA latent cache, 2 = K then V */
    uint32_t num_heads;             /* heads per token row */
    uint32_t head_dim;              /* elements per head */
    int64_t stride_page;            /* elements */
    int64_t stride_layer;
    int64_t stride_kv;
    int64_t stride_token;           /* token rows are contiguous: row = num_heads*head_dim */
    const uint32_t* page_table;     /* [device] [batch_size][max_pages_per_seq] page ids */
    uint32_t batch_size;            /* requests in the batch */
    uint32_t max_pages_per_seq;
    const uint32_t* cache_lengths;  /* [device] [batch_size] tokens already cached
                                       (read by kv_matmul_paged: where appends start;
                                       may be NULL for the decompress calls) */
} mla_paged_cache_t;

/* [host] Fill the four strides for a contiguous pool laid out
 * [page][layer][kv][slot][head][dim].  Returns MLA_ERR_NULL_POINTER or MLA_OK. */
mla_status_t mla_paged_cache_default_strides(mla_paged_cache_t* cache);

/*
 * The scales of an fp8 (F8E4M3FN) pool (the collection's scale_dtype_ = fp32 and
 * quantization_granularity_ of page "generic_flare_mla_decompress_k_cache_ragged_paged",
 * signature): every token row of num_heads*head_dim codes has
 * nblk = ceil(num_heads*head_dim / granularity) fp32 scales; scale j multiplies the
 * codes of columns [j*granularity, (j+1)*granularity).  The scales of (page, layer,
 * kv, slot) start at
 *   scales + page*stride_page + layer*stride_layer + kv*stride_kv + slot*stride_token
 * (strides in floats) and are contiguous.  The same page table addresses both pools.
 */
typedef struct {
    const float* scales;            /* [device] scale pool; 4-byte aligned */
    uint32_t granularity;           /* columns per scale; supported: 128 */
    int64_t stride_page;            /* floats */
    int64_t stride_layer;
    int64_t stride_kv;
    int64_t stride_token;           /* >= nblk */
} mla_cache_scales_t;

/*
 * Gather each request's latent rows from the paged cache, then up-project them
 * (page "generic_flare_mla_decompress_k_cache_ragged_paged", summary and Args;
 * weight shape from page "mla_prefill_decode_graph_fp8", Args w_k).
 *
 *   For request b < cache->batch_size and i < rows_b = buffer_row_offsets[b+1] -
 *   buffer_row_offsets[b], with r = buffer_row_offsets[b] + i and
 *   p = cache_offsets[b] + i:
 *     k_latent_buffer[r][0:D_c] = cache row of token p of request b in layer layer_idx
 *                                 (a bit copy; D_c = num_heads*head_dim)
 *     k_buffer[r][n]            = sum_{k<K} k_latent_buffer[r][k] * weight[n][k]
 *   accumulated in fp32 and rounded to the cache dtype (round to nearest even).
 *
 * buffer_row_offsets  [device] uint32 [batch_size+1], [0] = 0, nondecreasing
 * cache_offsets       [device] uint32 [>= batch_size]; a [batch_size+1] array is accepted
 *                     (the last entry is not read)
 * buffer_length       [host] M = buffer_row_offsets[batch_size], the rows to produce;
 *                     the grid is sized from it, rows >= M are never written
 * weight              [device] [N][K] in the cache dtype (F32 or BF16), 16-byte aligned
 * N, K                N = num_heads*qk_nope_head_dim, K = kv_lora_rank; 1 <= K <= D_c.
 *                     BF16: K % 64 == 0 and N % 64 == 0.  F32: K % 4 == 0 and N % 4 == 0.
 * cache               [host] num_kv == 1; D_c*elem_size and stride_token*elem_size
 *                     multiples of 16 bytes
 * k_latent_buffer     [device] [>= M][D_c] cache dtype, written
 * k_buffer            [device] [>= M][N] cache dtype, written
 */
mla_status_t mla_decompress_k_paged(const uint32_t* buffer_row_offsets,
                                    const uint32_t* cache_offsets,
                                    int32_t buffer_length,
                                    const void* weight, int32_t N, int32_t K,
                                    const mla_paged_cache_t* cache, uint32_t layer_idx,
                                    void* k_latent_buffer, void* k_buffer,
                                    void* stream);

/*
 * The first step of mla_decompress_k_paged on its own: the paged gather
 * (page "generic_flare_mla_decompress_k_cache_ragged_paged", Args
 * buffer_row_offsets_1d, cache_offsets_1d, k_latent_buffer).
 *
 *   k_latent_buffer[r][0:D_c] = cache row of token cache_offsets[b] + i of request b
 *   (r = buffer_row_offsets[b] + i), a bit copy.
 *
 * Arguments as in mla_decompress_k_paged; the cache dtype is F32 or BF16.
 */
mla_status_t mla_gather_latent_paged(const uint32_t* buffer_row_offsets,
                                     const uint32_t* cache_offsets,
                                     int32_t buffer_length,
                                     const mla_paged_cache_t* cache, uint32_t layer_idx,
                                     void* k_latent_buffer, void* stream);

/*
 * The second step of mla_decompress_k_paged on its own: the up-projection of
 * rows already gathered (page "generic_flare_mla_decompress_k_cache_ragged_paged",
 * Args weight, k_buffer; shape from page "mla_prefill_decode_graph_fp8", Args w_k).
 *
 *   k_buffer[r][n] = sum_{k<K} k_latent_buffer[r * ld_latent + k] * weight[n][k],
 *   fp32 accumulation, rounded to `dtype` (round to nearest even).
 *
 * k_latent_buffer  [device] [buffer_length][ld_latent] in `dtype`; columns >= K are not read
 * ld_latent        row stride in elements, K <= ld_latent <= 2^20, ld_latent*elem % 16 == 0
 * weight           [device] [N][K] in `dtype`
 * dtype            MLA_DTYPE_BF16 (K % 64 == 0, N % 64 == 0) or MLA_DTYPE_F32 (K, N % 4 == 0)
 * k_buffer         [device] [>= buffer_length][N] in `dtype`, written
 * All pointers 16-byte aligned.
 */
mla_status_t mla_latent_matmul(const void* k_latent_buffer, int64_t ld_latent, int32_t buffer_length,
                               const void* weight, int32_t N, int32_t K, int32_t dtype,
                               void* k_buffer, void* stream);

/*
 * Bytes of device workspace mla_decompress_k_paged_fp8 needs for buffer_length rows
 * (the activation codes and scales of the on-the-fly quantisation).  0 on bad
 * arguments.
 */
size_t mla_decompress_k_paged_fp8_workspace_size(int32_t buffer_length, int32_t K, int32_t k_gran);

/*
 * The fp8 block-scaled form of mla_decompress_k_paged (page
 * "mla_prefill_decode_graph_fp8": Parameters fp8_dtype, fp8_scale_dtype,
 * m/n/k_scale_granularity; Args w_k, w_k_scale).
 *
 *   The gather is as in mla_decompress_k_paged (cache dtype BF16).  Each gathered
 *   row is quantised per block of k_gran columns (m_gran = 1): amax = max|x|,
 *   s_a = amax / 448, codes = e4m3fn(x * (448 / amax)) (binary32 quotients, round
 *   to nearest even; an all-zero block takes s_a = 1).  Then
 *     k_buffer[r][n] = bf16( sum_kb s_a[r][kb] * weight_scale[n / n_gran][kb]
 *                                  * sum_{k in block kb} codes[r][k] * weight[n][k] )
 *   with fp32 accumulation.
 *
 * weight_e4m3      [device] [N][K] e4m3fn codes, 16-byte aligned
 * weight_scale     [device] float [N / n_gran][K / k_gran] multipliers (W ~= s * codes)
 * m_gran, n_gran, k_gran  granularities along M, N, K; supported: 1, 128, 128
 * N, K             N % 128 == 0, K % 128 == 0, K <= D_c
 * workspace        [device] >= mla_decompress_k_paged_fp8_workspace_size(M, K, k_gran)
 *                  bytes, 256-byte aligned; its contents on return are the activation
 *                  codes [M][K] followed (at offset align256(M*K)) by the scales
 *                  float [M][K / k_gran]
 * other arguments  as in mla_decompress_k_paged; k_latent_buffer and k_buffer are BF16
 *
 * The workspace argument is an addition to the page's signature: the codes and
 * scales go through device memory between the quantising gather and the product
 * (the product reads codes, half the bytes of the bf16 rows, in a loop bound by
 * its operand loads).  Callers that cannot pass one use
 * mla_decompress_k_paged_fp8_noalloc.
 */
mla_status_t mla_decompress_k_paged_fp8(const uint32_t* buffer_row_offsets,
                                        const uint32_t* cache_offsets,
                                        int32_t buffer_length,
                                        const void* weight_e4m3, const float* weight_scale,
                                        int32_t N, int32_t K,
                                        int32_t m_gran, int32_t n_gran, int32_t k_gran,
                                        const mla_paged_cache_t* cache, uint32_t layer_idx,
                                        void* k_latent_buffer, void* k_buffer,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Fused K and V decompression: one gather, two up-projections of the gathered
 * rows (page "mla_prefill_decode_graph_fp8", Args w_k and w_uv: w_uv projects the
 * latent values to V, shape [num_heads][v_head_dim][kv_latent_dim], i.e. an
 * [N_v][K] matrix with N_v = num_heads*v_head_dim; the gather and the product
 * are those of page "generic_flare_mla_decompress_k_cache_ragged_paged").
 *
 *   k_latent_buffer and k_buffer exactly as mla_decompress_k_paged(..., w_k, N_k, ...)
 *   v_buffer[r][n] = sum_{k<K} k_latent_buffer[r][k] * w_v[n][k]   (n < N_v),
 *   fp32 accumulation, rounded to the cache dtype (round to nearest even).
 *
 * Every element of k_buffer and v_buffer equals, bit for bit, what
 * mla_decompress_k_paged returns with w_k or w_v alone.  Each latent row is read
 * once from the cache; with BF16, K % 128 == 0 and N_k % 256 == 0 both products
 * run in a single launch that reads each tile of gathered rows for both.
 *
 * w_v        [device] [N_v][K] in the cache dtype, 16-byte aligned
 * N_v        BF16: N_v % 64 == 0; F32: N_v % 4 == 0
 * v_buffer   [device] [>= M][N_v] cache dtype, written
 * Other arguments, errors and validation order as in mla_decompress_k_paged
 * (w_k, N_k play the roles of weight, N).
 */
mla_status_t mla_decompress_kv_paged(const uint32_t* buffer_row_offsets,
                                     const uint32_t* cache_offsets,
                                     int32_t buffer_length,
                                     const void* w_k, int32_t N_k,
                                     const void* w_v, int32_t N_v, int32_t K,
                                     const mla_paged_cache_t* cache, uint32_t layer_idx,
                                     void* k_latent_buffer, void* k_buffer, void* v_buffer,
                                     void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_decompress_k_paged_fp8 without the workspace argument.  The activation
 * codes and scales go to a fixed array of MLA_FP8_NOALLOC_SCRATCH_BYTES in
 * device memory that the library holds on each GPU it runs on until the
 * process ends; nothing is allocated per call.
 *
 *   Same arguments, arithmetic and results as mla_decompress_k_paged_fp8 (the
 *   same kernels run).  Calls whose workspace would exceed the array
 *   (mla_decompress_k_paged_fp8_workspace_size(M, K, k_gran) >
 *   MLA_FP8_NOALLOC_SCRATCH_BYTES: more than 65536 rows at K = 512) return
 *   MLA_ERR_WORKSPACE before anything is enqueued.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, other host threads) race on it and must be ordered by
 *   the caller.  Nothing in the array has to start at zero: each call writes
 *   every code and scale it reads.
 *   The first call on a device looks up the array's address there
 *   (MLA_ERR_HIP if that fails).
 */
#define MLA_FP8_NOALLOC_SCRATCH_BYTES (33u << 20)   /* the workspace of 65536 rows at K = 512 */
mla_status_t mla_decompress_k_paged_fp8_noalloc(const uint32_t* buffer_row_offsets,
                                                const uint32_t* cache_offsets, int32_t buffer_length,
                                                const void* weight_e4m3, const float* weight_scale,
                                                int32_t N, int32_t K, int32_t m_gran, int32_t n_gran,
                                                int32_t k_gran, const mla_paged_cache_t* cache,
                                                uint32_t layer_idx, void* k_latent_buffer, void* k_buffer,
                                                void* stream);

/*
 * The fp8 block-scaled form of mla_decompress_kv_paged (page
 * "mla_prefill_decode_graph_fp8": Args w_k, w_k_scale, w_uv, w_uv_scale; the
 * quantisation of the gathered rows as in mla_decompress_k_paged_fp8, done once
 * for both products, which run in a single launch).
 *
 *   v_buffer[r][n] = bf16( sum_kb s_a[r][kb] * w_v_scale[n / n_gran][kb]
 *                                * sum_{k in block kb} codes[r][k] * w_v[n][k] )
 *
 * w_v_e4m3   [device] [N_v][K] e4m3fn codes, 16-byte aligned; N_v % 128 == 0
 * w_v_scale  [device] float [N_v / n_gran][K / k_gran]
 * v_buffer   [device] [>= M][N_v] bf16, written
 * Other arguments (workspace included), errors and validation order as in
 * mla_decompress_k_paged_fp8.
 */
mla_status_t mla_decompress_kv_paged_fp8(const uint32_t* buffer_row_offsets,
                                         const uint32_t* cache_offsets,
                                         int32_t buffer_length,
                                         const void* w_k_e4m3, const float* w_k_scale, int32_t N_k,
                                         const void* w_v_e4m3, const float* w_v_scale, int32_t N_v,
                                         int32_t K, int32_t m_gran, int32_t n_gran, int32_t k_gran,
                                         const mla_paged_cache_t* cache, uint32_t layer_idx,
                                         void* k_latent_buffer, void* k_buffer, void* v_buffer,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * The decompress call on an fp8 paged cache (page
 * "generic_flare_mla_decompress_k_cache_ragged_paged", summary and Args, with a
 * collection whose scale_dtype_ / quantization_granularity_ are fp32 / 128; the
 * weight and its block scales as page "mla_prefill_decode_graph_fp8", Args w_k,
 * w_k_scale, granularities 1 x 128 x 128).
 *
 *   For request b, i < rows_b, r = buffer_row_offsets[b] + i, p = cache_offsets[b] + i:
 *     k_latent_buffer[r][0:D_c]  = e4m3 codes of token p of request b (a bit copy)
 *     k_latent_scales[r][0:nblk] = that token's fp32 scales (a bit copy)
 *     k_buffer[r][n] = bf16( sum_kb k_latent_scales[r][kb] * weight_scale[n/128][kb]
 *                              * sum_{k in block kb} k_latent_buffer[r][k] * weight[n][k] )
 *   over the K/128 blocks of the first K columns, fp32 accumulation, round to
 *   nearest even.  The cache is already quantised: no quantisation step, no workspace.
 *
 * weight_e4m3      [device] [N][K] e4m3fn codes, 16-byte aligned
 * weight_scale     [device] float [N/128][K/128], 4-byte aligned
 * N, K             N % 128 == 0, K % 128 == 0, K <= D_c
 * cache            [host] dtype F8E4M3FN, num_kv == 1, D_c % 16 == 0, byte strides
 *                  multiples of 16
 * cache_scales     [host] granularity 128, stride_token >= nblk = ceil(D_c / 128)
 * k_latent_buffer  [device] uint8 [>= M][D_c], 16-byte aligned, written
 * k_latent_scales  [device] float [>= M][nblk], 4-byte aligned, written
 * k_buffer         [device] bf16 [>= M][N], 16-byte aligned, written
 * M * D_c < 2^31.  Other arguments, errors and validation order as in
 * mla_decompress_k_paged.
 */
mla_status_t mla_decompress_k_paged_fp8_cache(const uint32_t* buffer_row_offsets,
                                              const uint32_t* cache_offsets,
                                              int32_t buffer_length,
                                              const void* weight_e4m3, const float* weight_scale,
                                              int32_t N, int32_t K,
                                              const mla_paged_cache_t* cache,
                                              const mla_cache_scales_t* cache_scales,
                                              uint32_t layer_idx,
                                              void* k_latent_buffer, float* k_latent_scales,
                                              void* k_buffer, void* stream);

/*
 * K and V decompression from an e4m3 cache in one call (the fused form of
 * mla_decompress_kv_paged_fp8 on the cache of mla_decompress_k_paged_fp8_cache;
 * page "mla_prefill_decode_graph_fp8", Args w_k, w_k_scale, w_uv, w_uv_scale):
 * one gather of codes and scales, then
 *   k_buffer[r][n] as mla_decompress_k_paged_fp8_cache with w_k_e4m3 / w_k_scale (N_k columns)
 *   v_buffer[r][n] the same with w_v_e4m3 / w_v_scale (N_v columns)
 * in one product launch over both projections' column tiles.
 *
 * w_v_e4m3         [device] [N_v][K] e4m3fn codes, 16-byte aligned; N_v % 128 == 0
 * w_v_scale        [device] float [N_v/128][K/128], 4-byte aligned
 * v_buffer         [device] bf16 [>= M][N_v], 16-byte aligned, written
 * Other arguments, errors and validation order as in mla_decompress_k_paged_fp8_cache.
 */
mla_status_t mla_decompress_kv_paged_fp8_cache(const uint32_t* buffer_row_offsets,
                                               const uint32_t* cache_offsets, int32_t buffer_length,
                                               const void* w_k_e4m3, const float* w_k_scale, int32_t N_k,
                                               const void* w_v_e4m3, const float* w_v_scale, int32_t N_v,
                                               int32_t K, const mla_paged_cache_t* cache,
                                               const mla_cache_scales_t* cache_scales, uint32_t layer_idx,
                                               void* k_latent_buffer, float* k_latent_scales,
                                               void* k_buffer, void* v_buffer, void* stream);

/*
 * Query absorption for decode (page "mla_prefill_decode_graph_fp8", Args q
 * [tot_seq_len, num_heads, qk_nope_head_dim + qk_rope_head_dim] and w_uk
 * [num_heads, kv_latent_dim, qk_nope_head_dim], the weight that projects the
 * non-rope part of each query head to the KV latent space), bf16:
 *
 *   q_latent[t][h][c] = bf16( sum_{d < d_nope} q[t][h][d] * w_uk[h][c][d] ),  c < kv_latent_dim
 *   q_latent[t][h][kv_latent_dim + i] = q[t][h][d_nope + i],  i < d_rope   (copy_rope = 1 only)
 *
 * fp32 accumulation, round to nearest even.  With copy_rope = 1 an absorbed head
 * has the layout of an MLA cache row (latent, then rope).
 *
 * q             [device] bf16 [total_tokens][num_heads][d_nope + d_rope], 16-byte aligned
 * d_nope        128 (the supported qk_nope_head_dim); d_rope % 8 == 0
 * w_uk          [device] bf16 [num_heads][kv_latent_dim][d_nope], 16-byte aligned
 * kv_latent_dim % 128 == 0
 * copy_rope     0 or 1
 * q_latent      [device] bf16 [total_tokens][num_heads][kv_latent_dim + (copy_rope ? d_rope : 0)],
 *               16-byte aligned, written
 * (total_tokens + 128) * num_heads * (d_nope + d_rope) * 2 < 2^31.
 * Errors and validation order as for the other calls (pointers, shapes,
 * alignment, device).
 */
mla_status_t mla_absorb_q(const void* q, int32_t total_tokens, int32_t num_heads, int32_t d_nope,
                          int32_t d_rope, const void* w_uk, int32_t kv_latent_dim, int32_t copy_rope,
                          void* q_latent, void* stream);

/*
 * The fp8 form of mla_absorb_q (page "mla_prefill_decode_graph_fp8": w_uk in
 * fp8_dtype with w_uk_scale, Parameters m/n/k_scale_granularity).  The non-rope
 * part of each query head is quantised per 1 x 128 block as in
 * mla_decompress_k_paged_fp8 (s_q = amax / 448, codes = e4m3fn(x * (448 / amax)),
 * binary32 quotients, round to nearest even; an all-zero block takes s_q = 1):
 *
 *   q_latent[t][h][c] = bf16( s_q[t][h] * w_uk_scale[h][c / 128][0]
 *                             * sum_{d < 128} codes[t][h][d] * w_uk_e4m3[h][c][d] )
 *
 * with fp32 accumulation; the rope part as in mla_absorb_q.
 *
 * w_uk_e4m3     [device] e4m3fn codes [num_heads][kv_latent_dim][d_nope], 16-byte aligned
 * w_uk_scale    [device] float [num_heads][kv_latent_dim / 128][d_nope / 128], 4-byte aligned
 * m_gran, n_gran, k_gran  supported: 1, 128, 128
 * Other arguments, limits and errors as in mla_absorb_q.
 */
mla_status_t mla_absorb_q_fp8(const void* q, int32_t total_tokens, int32_t num_heads, int32_t d_nope,
                              int32_t d_rope, const void* w_uk_e4m3, const float* w_uk_scale,
                              int32_t kv_latent_dim, int32_t m_gran, int32_t n_gran, int32_t k_gran,
                              int32_t copy_rope, void* q_latent, void* stream);

/*
 * The latent write path: new tokens' latent rows, normalised and rotated, into
 * the MLA cache pages this library's decompress calls read (page
 * "mla_prefill_decode_graph_fp8", Args kv_input_fn (the latent values,
 * [tot_seq_len, cache_head_dim] with cache_head_dim = kv_lora_rank +
 * qk_rope_head_dim), kv_norm_gamma [kv_lora_rank], epsilon, freqs_cis
 * [max_seq_len, qk_rope_head_dim], input_row_offsets, kv_collection, layer_idx).
 *
 *   Token t of request b (input_row_offsets[b] <= t < input_row_offsets[b+1]) is
 *   written at position p = cache_lengths[b] + (t - input_row_offsets[b]):
 *     row[k]       = bf16( gamma[k] * x[k] / sqrt(mean_{k<K} x[k]^2 + epsilon) ),  k < K
 *     row[K+2j]    = bf16( x[K+2j] * c - x[K+2j+1] * s )
 *     row[K+2j+1]  = bf16( x[K+2j] * s + x[K+2j+1] * c ),  (c, s) = freqs_cis[p][2j], [2j+1]
 *   with x = kv_input[t], fp32 arithmetic, round to nearest even; stored as the
 *   cache row of (page_table[b][p / page_size], slot p % page_size) in layer
 *   layer_idx.  Other cache bytes are not touched; cache_lengths is not updated.
 *
 * kv_input         [device] bf16 [total_tokens][D_c], D_c = num_heads*head_dim = K + R
 * input_row_offsets [device] uint32 [batch_size+1], [0] = 0, nondecreasing
 * total_tokens     [host] input_row_offsets[batch_size]
 * kv_norm_gamma    [device] float [K], 16-byte aligned
 * epsilon          >= 0
 * freqs_cis        [device] float [max_seq_len][R], (cos, sin) of each rope pair;
 *                  may be NULL when R == 0; positions must be < max_seq_len
 * K                kv_lora_rank: K % 8 == 0, K <= 512; R = D_c - K: R % 8 == 0, R <= 512
 * cache            [host] num_kv == 1, BF16, cache_lengths set; pages are WRITTEN
 * Errors and validation order as for the other calls (pointers, shapes, dtype,
 * alignment, ranges, device).
 */
mla_status_t mla_write_latent_paged(const void* kv_input, const uint32_t* input_row_offsets,
                                    int32_t total_tokens, const float* kv_norm_gamma, float epsilon,
                                    const float* freqs_cis, int32_t max_seq_len, int32_t K,
                                    const mla_paged_cache_t* cache, uint32_t layer_idx, void* stream);

/*
 * The latent write path into an e4m3 cache (page "mla_prefill_decode_graph_fp8",
 * Args kv_input_fn, kv_norm_gamma, epsilon, freqs_cis, input_row_offsets,
 * kv_collection, layer_idx; the collection's scale_dtype_ fp32 and
 * quantization_granularity_ 128 of page
 * "generic_flare_mla_decompress_k_cache_ragged_paged"): the rows of
 * mla_write_latent_paged, computed the same way in fp32, then quantised per
 * block of 128 columns of the row:
 *   y = the fp32 row values (RMS-normalised latent part, rotated rope part)
 *   amax_j = max |y| over block j, s_j = amax_j / 448 (1 for an all-zero block)
 *   codes = e4m3fn(y * (448 / amax_j)), round to nearest even; s_j into the scale pool
 * at the token's (page, slot) in layer layer_idx, codes into the e4m3 pool.
 * mla_decompress_k_paged_fp8_cache reads what this writes.
 *
 * cache            [host] num_kv == 1, dtype F8E4M3FN, D_c % 16 == 0, cache_lengths set;
 *                  pages are WRITTEN
 * cache_scales     [host] granularity 128, stride_token >= ceil(D_c / 128); WRITTEN
 * K                kv_lora_rank: K % 128 == 0, K <= 512; R = D_c - K: R % 8 == 0, R <= 512
 * Other arguments, errors and validation order as in mla_write_latent_paged.
 */
mla_status_t mla_write_latent_paged_fp8(const void* kv_input, const uint32_t* input_row_offsets,
                                        int32_t total_tokens, const float* kv_norm_gamma, float epsilon,
                                        const float* freqs_cis, int32_t max_seq_len, int32_t K,
                                        const mla_paged_cache_t* cache, const mla_cache_scales_t* cache_scales,
                                        uint32_t layer_idx, void* stream);

/*
 * Project hidden states and write them into the paged K/V cache (page
 * "kv_matmul_ragged_paged", summary and Args).
 *
 *   out[t][n] = sum_k hidden_state[t][k] * weight[k][n], fp32 accumulation.
 *   Token t of request b (input_row_offsets[b] <= t < input_row_offsets[b+1]) is
 *   appended at position p = cache_lengths[b] + (t - input_row_offsets[b]):
 *     K row of (page_table[b][p / page_size], slot p % page_size) = bf16(out[t][0 : HD])
 *     V row of the same slot                                        = bf16(out[t][HD : 2HD])
 *   with HD = num_heads*head_dim.  No other cache element is written, and
 *   cache_lengths is not updated (that bookkeeping is the cache owner's).
 *
 * hidden_state       [device] bf16 [total_tokens][hidden_dim], 16-byte aligned
 * input_row_offsets  [device] uint32 [batch_size+1], [0] = 0, nondecreasing,
 *                    [batch_size] = total_tokens
 * total_tokens       [host] T >= 0
 * hidden_dim         [host] % 64 == 0
 * weight             [device] bf16 [hidden_dim][2*HD], 16-byte aligned
 * cache              [host] BF16, num_kv == 2, HD % 64 == 0, cache_lengths non-NULL;
 *                    pages are written in place
 */
mla_status_t kv_matmul_paged(const void* hidden_state, const uint32_t* input_row_offsets,
                             int32_t total_tokens, int32_t hidden_dim,
                             const void* weight,
                             const mla_paged_cache_t* cache, uint32_t layer_idx,
                             void* stream);

/*
 * Debug check of the index arrays of a call (the preconditions the pages leave to
 * the caller: offsets start at 0 and never decrease, every position a request
 * touches lies inside its page-table row and maps to a page id < num_pages).
 * Copies the arrays to the host and synchronises `stream`; meant for debugging,
 * not for the hot path.
 *
 * row_offsets    [device] uint32 [batch_size+1] (buffer_row_offsets or input_row_offsets)
 * cache_offsets  [device] uint32 [>= batch_size]: positions read start there
 *                (decompress calls), and when cache->cache_lengths is non-NULL they
 *                must also end at or before cache_lengths[b].  NULL: positions
 *                written start at cache_lengths[b] (kv_matmul_paged).
 * rows           [host] must equal row_offsets[batch_size]
 * bad_request    [host] optional; receives the first failing request (-1 if none)
 * Returns MLA_OK, MLA_ERR_INVALID_SHAPE (offsets), MLA_ERR_OUT_OF_RANGE (positions
 * or page ids), MLA_ERR_NULL_POINTER, MLA_ERR_UNSUPPORTED_DEVICE or MLA_ERR_HIP.
 */
mla_status_t mla_check_indices(const uint32_t* row_offsets, const uint32_t* cache_offsets,
                               int32_t rows, const mla_paged_cache_t* cache, int64_t* bad_request,
                               void* stream);

/* Static text for a status code. */
const char* mla_status_string(mla_status_t status);

/* hipError_t of the last MLA_ERR_HIP returned on this host thread (0 if none). */
int32_t mla_last_hip_error(void);

/* MLA_PAGED_ABI_VERSION of the loaded library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_H */
