// C ABI of the paged MLA latent-K library (include/mla_paged.h): host-side
// argument validation, device check, and dispatch to one launcher.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include <cstdarg>
#include <cstdio>

#include "mla_paged.h"
#include "launch.hpp"

namespace mla {

void log_launch(const char* kernel, unsigned grid, unsigned block, const char* fmt, ...)
{
    static const bool on = [] {
        const char* v = std::getenv("MLA_PAGED_LOG");
        return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
    }();
    if (!on)
        return;
    char detail[256];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(detail, sizeof(detail), fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "mla_paged: %s grid %u block %u %s\n", kernel, grid, block, detail);
}

}  // namespace mla

#define MLA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int32_t g_last_hip_error = 0;

mla_status_t hip_failed(hipError_t e)
{
    g_last_hip_error = (int32_t)e;
    return MLA_ERR_HIP;
}

int elem_bytes(int32_t dtype)
{
    switch (dtype) {
    case MLA_DTYPE_F32: return 4;
    case MLA_DTYPE_BF16: return 2;
    case MLA_DTYPE_F8E4M3FN: return 1;
    default: return 0;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The current device must be a gfx950; the answer is cached per device.
mla_status_t check_device()
{
    static std::atomic<int> verdict[64];  // 0 unknown, 1 gfx950, 2 other
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return MLA_ERR_UNSUPPORTED_DEVICE;
    if (dev < 64) {
        const int v = verdict[dev].load(std::memory_order_relaxed);
        if (v == 1)
            return MLA_OK;
        if (v == 2)
            return MLA_ERR_UNSUPPORTED_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return MLA_ERR_UNSUPPORTED_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64)
        verdict[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MLA_OK : MLA_ERR_UNSUPPORTED_DEVICE;
}

// Checks of the cache descriptor shared by every call.  `row_check` holds
// the expected num_kv; `work` says whether device pointers must be present.
mla_status_t check_cache_shape(const mla_paged_cache_t* c, uint32_t num_kv)
{
    if (c->num_layers == 0 || c->num_pages == 0 || c->page_size == 0 || c->num_heads == 0 ||
        c->head_dim == 0 || c->batch_size == 0 || c->max_pages_per_seq == 0 || c->num_kv != num_kv)
        return MLA_ERR_INVALID_SHAPE;
    const int64_t row = (int64_t)c->num_heads * c->head_dim;
    if (c->stride_token < row || c->stride_page <= 0 || c->stride_layer < 0 || c->stride_kv < 0 ||
        (num_kv > 1 && c->stride_kv < row))
        return MLA_ERR_INVALID_SHAPE;
    return MLA_OK;
}

mla_status_t check_cache_alignment(const mla_paged_cache_t* c)
{
    const int eb = elem_bytes(c->dtype);
    if (!aligned16(c->blocks) || (c->stride_token * eb) % 16 || (c->stride_page * eb) % 16 ||
        (c->stride_layer * eb) % 16 || (c->stride_kv * eb) % 16 ||
        ((int64_t)c->num_heads * c->head_dim * eb) % 16)
        return MLA_ERR_MISALIGNED;
    return MLA_OK;
}

mla::PagedLayer layer_view(const mla_paged_cache_t* c, uint32_t layer)
{
    const int eb = elem_bytes(c->dtype);
    mla::PagedLayer L;
    L.base = static_cast<const char*>(c->blocks) + (int64_t)layer * c->stride_layer * eb;
    L.page_table = c->page_table;
    L.stride_page = c->stride_page * eb;
    L.stride_token = c->stride_token * eb;
    L.stride_kv = c->stride_kv * eb;
    L.num_pages = c->num_pages;
    L.page_size = c->page_size;
    L.max_pages = c->max_pages_per_seq;
    L.batch = c->batch_size;
    return L;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The product kernels address one 256-row tile of their operands and outputs
// through 32-bit byte offsets: a row of `width` elements of `eb` bytes times
// 256 rows must stay below 2^31 bytes.
bool tile_fits_32bit(int64_t width, int eb) { return width * eb * 256 < (int64_t(1) << 31); }

}  // namespace

MLA_API mla_status_t mla_paged_cache_default_strides(mla_paged_cache_t* c)
{
    if (!c)
        return MLA_ERR_NULL_POINTER;
    c->stride_token = (int64_t)c->num_heads * c->head_dim;
    c->stride_kv = c->stride_token * c->page_size;
    c->stride_layer = c->stride_kv * c->num_kv;
    c->stride_page = c->stride_layer * c->num_layers;
    return MLA_OK;
}

namespace {

// A second projection of the same rows (the fused K and V form), or none.
struct Second {
    const void* w = nullptr;
    const float* scale = nullptr;   // fp8 only
    int32_t N = 0;
    void* out = nullptr;
    bool present = false;
};

// Validation of the bf16 / f32 decompress calls, in the documented order
// (pointers, shapes, dtype, alignment, ranges); D receives the cache row width.
mla_status_t check_decompress(const uint32_t* bro, const uint32_t* co, int32_t M, const void* weight, int32_t N,
                              int32_t K, const mla_paged_cache_t* cache, uint32_t layer_idx, const void* lat,
                              const void* out, const Second& v, int64_t& D)
{
    if (!cache)
        return MLA_ERR_NULL_POINTER;
    const bool work = M > 0;
    if (work && (!bro || !co || !weight || !lat || !out || !cache->blocks || !cache->page_table))
        return MLA_ERR_NULL_POINTER;
    if (work && v.present && (!v.w || !v.out))
        return MLA_ERR_NULL_POINTER;
    if (M < 0 || N <= 0 || K <= 0 || (v.present && v.N <= 0))
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    D = (int64_t)cache->num_heads * cache->head_dim;
    if (K > D)
        return MLA_ERR_INVALID_SHAPE;
    const int32_t N2 = v.present ? v.N : 64;
    if (cache->dtype == MLA_DTYPE_BF16) {
        if (K % 64 || N % 64 || N2 % 64 || (int64_t)N * K * 2 >= (int64_t(1) << 31) ||
            (int64_t)N2 * K * 2 >= (int64_t(1) << 31) || !tile_fits_32bit(N, 2) || !tile_fits_32bit(N2, 2) ||
            !tile_fits_32bit(D, 2))
            return MLA_ERR_INVALID_SHAPE;
    } else if (cache->dtype == MLA_DTYPE_F32) {
        if (K % 4 || N % 4 || N2 % 4)
            return MLA_ERR_INVALID_SHAPE;
    } else {
        return MLA_ERR_INVALID_DTYPE;
    }
    if (!aligned16(weight) || !aligned16(lat) || !aligned16(out) || !aligned16(v.w) || !aligned16(v.out))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    return MLA_OK;
}

mla::DecompressArgs decompress_args(const uint32_t* bro, const uint32_t* co, int32_t M, const void* weight,
                                    int32_t N, int32_t K, const mla_paged_cache_t* cache, uint32_t layer_idx,
                                    void* lat, void* out, int64_t D, const Second& v)
{
    mla::DecompressArgs a{};
    a.bro = bro;
    a.co = co;
    a.L = layer_view(cache, layer_idx);
    a.W = weight;
    a.lat = lat;
    a.out = out;
    a.M = M;
    a.N = N;
    a.K = K;
    a.D = (int)D;
    if (v.present) {
        a.W2 = v.w;
        a.W2_scale = v.scale;
        a.out2 = v.out;
        a.N2 = v.N;
    }
    return a;
}

}  // namespace

MLA_API mla_status_t mla_decompress_k_paged(const uint32_t* buffer_row_offsets,
                                            const uint32_t* cache_offsets, int32_t buffer_length,
                                            const void* weight, int32_t N, int32_t K,
                                            const mla_paged_cache_t* cache, uint32_t layer_idx,
                                            void* k_latent_buffer, void* k_buffer, void* stream)
{
    int64_t D = 0;
    const Second none;
    if (mla_status_t st = check_decompress(buffer_row_offsets, cache_offsets, buffer_length, weight, N, K, cache,
                                           layer_idx, k_latent_buffer, k_buffer, none, D))
        return st;
    if (buffer_length == 0)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    const mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, buffer_length, weight, N, K,
                                                  cache, layer_idx, k_latent_buffer, k_buffer, D, none);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = cache->dtype == MLA_DTYPE_BF16 ? mla::launch_decompress_bf16(a, s)
                                                        : mla::launch_decompress_f32(a, s);
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_decompress_kv_paged(const uint32_t* buffer_row_offsets,
                                             const uint32_t* cache_offsets, int32_t buffer_length,
                                             const void* w_k, int32_t N_k, const void* w_v, int32_t N_v,
                                             int32_t K, const mla_paged_cache_t* cache, uint32_t layer_idx,
                                             void* k_latent_buffer, void* k_buffer, void* v_buffer,
                                             void* stream)
{
    int64_t D = 0;
    Second v;
    v.w = w_v;
    v.N = N_v;
    v.out = v_buffer;
    v.present = true;
    if (mla_status_t st = check_decompress(buffer_row_offsets, cache_offsets, buffer_length, w_k, N_k, K, cache,
                                           layer_idx, k_latent_buffer, k_buffer, v, D))
        return st;
    if (buffer_length == 0)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    const mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, buffer_length, w_k, N_k, K,
                                                  cache, layer_idx, k_latent_buffer, k_buffer, D, v);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = cache->dtype == MLA_DTYPE_BF16 ? mla::launch_decompress_kv_bf16(a, s)
                                                        : mla::launch_decompress_kv_f32(a, s);
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_gather_latent_paged(const uint32_t* buffer_row_offsets,
                                             const uint32_t* cache_offsets, int32_t buffer_length,
                                             const mla_paged_cache_t* cache, uint32_t layer_idx,
                                             void* k_latent_buffer, void* stream)
{
    if (!cache)
        return MLA_ERR_NULL_POINTER;
    const bool work = buffer_length > 0;
    if (work && (!buffer_row_offsets || !cache_offsets || !k_latent_buffer || !cache->blocks ||
                 !cache->page_table))
        return MLA_ERR_NULL_POINTER;
    if (buffer_length < 0)
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    const int eb = elem_bytes(cache->dtype);
    if (cache->dtype != MLA_DTYPE_BF16 && cache->dtype != MLA_DTYPE_F32)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(k_latent_buffer))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::DecompressArgs a{};
    a.bro = buffer_row_offsets;
    a.co = cache_offsets;
    a.L = layer_view(cache, layer_idx);
    a.lat = k_latent_buffer;
    a.M = buffer_length;
    a.D = (int)((int64_t)cache->num_heads * cache->head_dim);
    const hipError_t e = mla::launch_gather_rows(a, eb, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_latent_matmul(const void* k_latent_buffer, int64_t ld_latent, int32_t buffer_length,
                                       const void* weight, int32_t N, int32_t K, int32_t dtype,
                                       void* k_buffer, void* stream)
{
    const bool work = buffer_length > 0;
    if (work && (!k_latent_buffer || !weight || !k_buffer))
        return MLA_ERR_NULL_POINTER;
    if (buffer_length < 0 || N <= 0 || K <= 0 || ld_latent < K || ld_latent > (int64_t(1) << 20))
        return MLA_ERR_INVALID_SHAPE;
    const int eb = elem_bytes(dtype);
    if (dtype == MLA_DTYPE_BF16) {
        if (K % 64 || N % 64 || (int64_t)N * K * 2 >= (int64_t(1) << 31) || !tile_fits_32bit(N, 2))
            return MLA_ERR_INVALID_SHAPE;
    } else if (dtype == MLA_DTYPE_F32) {
        if (K % 4 || N % 4)
            return MLA_ERR_INVALID_SHAPE;
    } else {
        return MLA_ERR_INVALID_DTYPE;
    }
    if (!aligned16(weight) || !aligned16(k_latent_buffer) || !aligned16(k_buffer) || (ld_latent * eb) % 16)
        return MLA_ERR_MISALIGNED;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::DecompressArgs a{};
    a.W = weight;
    a.lat = const_cast<void*>(k_latent_buffer);
    a.out = k_buffer;
    a.M = buffer_length;
    a.N = N;
    a.K = K;
    a.D = (int)ld_latent;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == MLA_DTYPE_BF16 ? mla::launch_product_bf16(a, s) : mla::launch_product_f32(a, s);
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API size_t mla_decompress_k_paged_fp8_workspace_size(int32_t buffer_length, int32_t K, int32_t k_gran)
{
    if (buffer_length < 0 || K <= 0 || k_gran != 128 || K % k_gran)
        return 0;
    const size_t M = (size_t)buffer_length;
    return align256(M * (size_t)K) + align256(M * (size_t)(K / k_gran) * sizeof(float));
}

namespace {

// Validation of the fp8 decompress calls, in the documented order.
mla_status_t check_decompress_fp8(const uint32_t* bro, const uint32_t* co, int32_t M, const void* w,
                                  const float* w_scale, int32_t N, int32_t K, int32_t m_gran, int32_t n_gran,
                                  int32_t k_gran, const mla_paged_cache_t* cache, uint32_t layer_idx,
                                  const void* lat, const void* out, const void* workspace, size_t workspace_bytes,
                                  const Second& v, int64_t& D)
{
    if (!cache)
        return MLA_ERR_NULL_POINTER;
    const bool work = M > 0;
    if (work && (!bro || !co || !w || !w_scale || !lat || !out || !workspace || !cache->blocks ||
                 !cache->page_table))
        return MLA_ERR_NULL_POINTER;
    if (work && v.present && (!v.w || !v.scale || !v.out))
        return MLA_ERR_NULL_POINTER;
    const int32_t N2 = v.present ? v.N : 128;
    if (M < 0 || N <= 0 || K <= 0 || N2 <= 0 || m_gran != 1 || n_gran != 128 || k_gran != 128 || N % 128 ||
        N2 % 128 || K % 128 || (int64_t)N * K >= (int64_t(1) << 31) || (int64_t)N2 * K >= (int64_t(1) << 31) ||
        !tile_fits_32bit(N, 2) || !tile_fits_32bit(N2, 2) || (int64_t)M * (K / 128) * 4 >= (int64_t(1) << 31))
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    D = (int64_t)cache->num_heads * cache->head_dim;
    if (K > D || !tile_fits_32bit(D, 2))
        return MLA_ERR_INVALID_SHAPE;
    if (cache->dtype != MLA_DTYPE_BF16)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(w) || !aligned16(lat) || !aligned16(out) || !aligned16(v.w) || !aligned16(v.out) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) || (reinterpret_cast<uintptr_t>(w_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(v.scale) & 3u))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (work && workspace_bytes < mla_decompress_k_paged_fp8_workspace_size(M, K, k_gran))
        return MLA_ERR_WORKSPACE;
    return MLA_OK;
}

void set_fp8_workspace(mla::DecompressArgs& a, const float* w_scale, void* workspace)
{
    a.W_scale = w_scale;
    a.q = workspace;
    a.q_scale = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)a.M * (size_t)a.K));
}

}  // namespace

MLA_API mla_status_t mla_decompress_k_paged_fp8(const uint32_t* buffer_row_offsets,
                                                const uint32_t* cache_offsets, int32_t buffer_length,
                                                const void* weight_e4m3, const float* weight_scale,
                                                int32_t N, int32_t K, int32_t m_gran, int32_t n_gran,
                                                int32_t k_gran, const mla_paged_cache_t* cache,
                                                uint32_t layer_idx, void* k_latent_buffer, void* k_buffer,
                                                void* workspace, size_t workspace_bytes, void* stream)
{
    int64_t D = 0;
    const Second none;
    if (mla_status_t st = check_decompress_fp8(buffer_row_offsets, cache_offsets, buffer_length, weight_e4m3,
                                               weight_scale, N, K, m_gran, n_gran, k_gran, cache, layer_idx,
                                               k_latent_buffer, k_buffer, workspace, workspace_bytes, none, D))
        return st;
    if (buffer_length == 0)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, buffer_length, weight_e4m3, N, K,
                                            cache, layer_idx, k_latent_buffer, k_buffer, D, none);
    set_fp8_workspace(a, weight_scale, workspace);
    const hipError_t e = mla::launch_decompress_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

// ---------------------------------------------------------------------------
// The fp8 call without a workspace argument, for callers that cannot allocate.
// Its activation codes and scales go to a fixed array in device memory
// (`scratch`, MLA_FP8_NOALLOC_SCRATCH_BYTES per GPU, held from the library's
// load until the process ends).  Host code never passes the array's name to a
// kernel: the name is a host-side stand-in, not a device address.  The device
// address is looked up once per device, with that device current, and kept.
// ---------------------------------------------------------------------------
namespace {

__device__ __align__(256) unsigned char scratch[MLA_FP8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (null on failure; `e` tells why).
void* scratch_on_current_device(hipError_t& e)
{
    e = hipSuccess;
    int dev = -1;
    if ((e = hipGetDevice(&dev)) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        e = hipErrorInvalidDevice;
        return nullptr;
    }
    if (void* p = g_scratch[dev].load(std::memory_order_acquire))
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (void* p = g_scratch[dev].load(std::memory_order_relaxed))
        return p;
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess || !ptr) {
        if (e == hipSuccess)
            e = hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch[dev].store(ptr, std::memory_order_release);
    return ptr;
}

}  // namespace

MLA_API mla_status_t mla_decompress_k_paged_fp8_noalloc(const uint32_t* buffer_row_offsets,
                                                        const uint32_t* cache_offsets, int32_t buffer_length,
                                                        const void* weight_e4m3, const float* weight_scale,
                                                        int32_t N, int32_t K, int32_t m_gran, int32_t n_gran,
                                                        int32_t k_gran, const mla_paged_cache_t* cache,
                                                        uint32_t layer_idx, void* k_latent_buffer, void* k_buffer,
                                                        void* stream)
{
    int64_t D = 0;
    const Second none;
    // The scratch array stands in for the workspace: the usual checks run with
    // a placeholder that passes the pointer and alignment tests, and a size
    // beyond the array is refused first.
    const size_t need = mla_decompress_k_paged_fp8_workspace_size(buffer_length > 0 ? buffer_length : 0, K, k_gran);
    if (buffer_length > 0 && need > (size_t)MLA_FP8_NOALLOC_SCRATCH_BYTES)
        return MLA_ERR_WORKSPACE;
    void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
    if (mla_status_t st = check_decompress_fp8(buffer_row_offsets, cache_offsets, buffer_length, weight_e4m3,
                                               weight_scale, N, K, m_gran, n_gran, k_gran, cache, layer_idx,
                                               k_latent_buffer, k_buffer, placeholder, need, none, D))
        return st;
    if (buffer_length == 0)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    hipError_t e;
    void* ws = scratch_on_current_device(e);
    if (!ws)
        return hip_failed(e);
    mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, buffer_length, weight_e4m3, N, K,
                                            cache, layer_idx, k_latent_buffer, k_buffer, D, none);
    set_fp8_workspace(a, weight_scale, ws);
    e = mla::launch_decompress_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_decompress_kv_paged_fp8(const uint32_t* buffer_row_offsets,
                                                 const uint32_t* cache_offsets, int32_t buffer_length,
                                                 const void* w_k_e4m3, const float* w_k_scale, int32_t N_k,
                                                 const void* w_v_e4m3, const float* w_v_scale, int32_t N_v,
                                                 int32_t K, int32_t m_gran, int32_t n_gran, int32_t k_gran,
                                                 const mla_paged_cache_t* cache, uint32_t layer_idx,
                                                 void* k_latent_buffer, void* k_buffer, void* v_buffer,
                                                 void* workspace, size_t workspace_bytes, void* stream)
{
    int64_t D = 0;
    Second v;
    v.w = w_v_e4m3;
    v.scale = w_v_scale;
    v.N = N_v;
    v.out = v_buffer;
    v.present = true;
    if (mla_status_t st = check_decompress_fp8(buffer_row_offsets, cache_offsets, buffer_length, w_k_e4m3,
                                               w_k_scale, N_k, K, m_gran, n_gran, k_gran, cache, layer_idx,
                                               k_latent_buffer, k_buffer, workspace, workspace_bytes, v, D))
        return st;
    if (buffer_length == 0)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, buffer_length, w_k_e4m3, N_k, K,
                                            cache, layer_idx, k_latent_buffer, k_buffer, D, v);
    set_fp8_workspace(a, w_k_scale, workspace);
    const hipError_t e = mla::launch_decompress_kv_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

namespace {

// The fp8-cache decompress calls (K alone, or K and V): validation in the
// documented order (pointers, shapes, dtype, alignment, ranges), then one
// gather of codes and scales and one product launch over both projections.
mla_status_t decompress_fp8_cache(const uint32_t* buffer_row_offsets, const uint32_t* cache_offsets,
                                  int32_t buffer_length, const void* weight_e4m3, const float* weight_scale,
                                  int32_t N, int32_t K, const mla_paged_cache_t* cache,
                                  const mla_cache_scales_t* cache_scales, uint32_t layer_idx,
                                  void* k_latent_buffer, float* k_latent_scales, void* k_buffer, const Second& v,
                                  void* stream)
{
    if (!cache || !cache_scales)
        return MLA_ERR_NULL_POINTER;
    const int32_t M = buffer_length;
    const bool work = M > 0;
    if (work && (!buffer_row_offsets || !cache_offsets || !weight_e4m3 || !weight_scale || !k_latent_buffer ||
                 !k_latent_scales || !k_buffer || !cache->blocks || !cache->page_table || !cache_scales->scales ||
                 (v.present && (!v.w || !v.scale || !v.out))))
        return MLA_ERR_NULL_POINTER;
    if (M < 0 || N <= 0 || K <= 0 || N % 128 || K % 128 || (int64_t)N * K >= (int64_t(1) << 31) ||
        !tile_fits_32bit(N, 2) || cache_scales->granularity != 128 ||
        (v.present && (v.N <= 0 || v.N % 128 || (int64_t)v.N * K >= (int64_t(1) << 31) || !tile_fits_32bit(v.N, 2))))
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    const int64_t D = (int64_t)cache->num_heads * cache->head_dim;
    const int64_t nblk = (D + 127) / 128;
    if (K > D || (int64_t)M * D >= (int64_t(1) << 31) || cache_scales->stride_token < nblk ||
        cache_scales->stride_page <= 0 || cache_scales->stride_layer < 0 || cache_scales->stride_kv < 0)
        return MLA_ERR_INVALID_SHAPE;
    if (cache->dtype != MLA_DTYPE_F8E4M3FN)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(weight_e4m3) || !aligned16(k_latent_buffer) || !aligned16(k_buffer) ||
        (reinterpret_cast<uintptr_t>(weight_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_latent_scales) & 3u) ||
        (reinterpret_cast<uintptr_t>(cache_scales->scales) & 3u) ||
        (v.present && (!aligned16(v.w) || !aligned16(v.out) || (reinterpret_cast<uintptr_t>(v.scale) & 3u))))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::DecompressArgs a = decompress_args(buffer_row_offsets, cache_offsets, M, weight_e4m3, N, K, cache,
                                            layer_idx, k_latent_buffer, k_buffer, D, v);
    a.W_scale = weight_scale;
    a.Ls = a.L;
    a.Ls.base = reinterpret_cast<const char*>(cache_scales->scales + (int64_t)layer_idx * cache_scales->stride_layer);
    a.Ls.stride_page = cache_scales->stride_page * 4;
    a.Ls.stride_token = cache_scales->stride_token * 4;
    a.Ls.stride_kv = cache_scales->stride_kv * 4;
    a.lat_scale = k_latent_scales;
    a.nblk = (int)nblk;
    const hipError_t e = mla::launch_decompress_fp8_cache(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

}  // namespace

MLA_API mla_status_t mla_decompress_k_paged_fp8_cache(const uint32_t* buffer_row_offsets,
                                                      const uint32_t* cache_offsets, int32_t buffer_length,
                                                      const void* weight_e4m3, const float* weight_scale,
                                                      int32_t N, int32_t K, const mla_paged_cache_t* cache,
                                                      const mla_cache_scales_t* cache_scales, uint32_t layer_idx,
                                                      void* k_latent_buffer, float* k_latent_scales,
                                                      void* k_buffer, void* stream)
{
    const Second none;
    return decompress_fp8_cache(buffer_row_offsets, cache_offsets, buffer_length, weight_e4m3, weight_scale, N, K,
                                cache, cache_scales, layer_idx, k_latent_buffer, k_latent_scales, k_buffer, none,
                                stream);
}

MLA_API mla_status_t mla_decompress_kv_paged_fp8_cache(const uint32_t* buffer_row_offsets,
                                                       const uint32_t* cache_offsets, int32_t buffer_length,
                                                       const void* w_k_e4m3, const float* w_k_scale, int32_t N_k,
                                                       const void* w_v_e4m3, const float* w_v_scale, int32_t N_v,
                                                       int32_t K, const mla_paged_cache_t* cache,
                                                       const mla_cache_scales_t* cache_scales, uint32_t layer_idx,
                                                       void* k_latent_buffer, float* k_latent_scales,
                                                       void* k_buffer, void* v_buffer, void* stream)
{
    Second v;
    v.w = w_v_e4m3;
    v.scale = w_v_scale;
    v.N = N_v;
    v.out = v_buffer;
    v.present = true;
    return decompress_fp8_cache(buffer_row_offsets, cache_offsets, buffer_length, w_k_e4m3, w_k_scale, N_k, K,
                                cache, cache_scales, layer_idx, k_latent_buffer, k_latent_scales, k_buffer, v,
                                stream);
}

MLA_API mla_status_t mla_absorb_q(const void* q, int32_t total_tokens, int32_t num_heads, int32_t d_nope,
                                  int32_t d_rope, const void* w_uk, int32_t kv_latent_dim, int32_t copy_rope,
                                  void* q_latent, void* stream)
{
    const int32_t T = total_tokens;
    const bool work = T > 0;
    if (work && (!q || !w_uk || !q_latent))
        return MLA_ERR_NULL_POINTER;
    const int64_t Dq = (int64_t)d_nope + d_rope;
    if (T < 0 || num_heads <= 0 || d_nope != 128 || d_rope < 0 || d_rope % 8 || kv_latent_dim <= 0 ||
        kv_latent_dim % 128 || (copy_rope != 0 && copy_rope != 1) ||
        ((int64_t)T + 128) * num_heads * Dq * 2 >= (int64_t(1) << 31) ||
        (int64_t)num_heads * kv_latent_dim * d_nope * 2 >= (int64_t(1) << 40))
        return MLA_ERR_INVALID_SHAPE;
    if (!aligned16(q) || !aligned16(w_uk) || !aligned16(q_latent))
        return MLA_ERR_MISALIGNED;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    mla::AbsorbArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.w = static_cast<const uint16_t*>(w_uk);
    a.out = static_cast<uint16_t*>(q_latent);
    a.T = T;
    a.H = num_heads;
    a.NL = kv_latent_dim;
    a.Dq = (int)Dq;
    a.R = copy_rope ? d_rope : 0;
    a.Do = kv_latent_dim + a.R;
    const hipError_t e = mla::launch_absorb_bf16(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_absorb_q_fp8(const void* q, int32_t total_tokens, int32_t num_heads, int32_t d_nope,
                                      int32_t d_rope, const void* w_uk_e4m3, const float* w_uk_scale,
                                      int32_t kv_latent_dim, int32_t m_gran, int32_t n_gran, int32_t k_gran,
                                      int32_t copy_rope, void* q_latent, void* stream)
{
    const int32_t T = total_tokens;
    const bool work = T > 0;
    if (work && (!q || !w_uk_e4m3 || !w_uk_scale || !q_latent))
        return MLA_ERR_NULL_POINTER;
    const int64_t Dq = (int64_t)d_nope + d_rope;
    if (T < 0 || num_heads <= 0 || d_nope != 128 || d_rope < 0 || d_rope % 8 || kv_latent_dim <= 0 ||
        kv_latent_dim % 128 || m_gran != 1 || n_gran != 128 || k_gran != 128 || (copy_rope != 0 && copy_rope != 1) ||
        ((int64_t)T + 128) * num_heads * Dq * 2 >= (int64_t(1) << 31))
        return MLA_ERR_INVALID_SHAPE;
    if (!aligned16(q) || !aligned16(w_uk_e4m3) || !aligned16(q_latent) ||
        (reinterpret_cast<uintptr_t>(w_uk_scale) & 3u))
        return MLA_ERR_MISALIGNED;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;
    mla::AbsorbArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.wq = static_cast<const uint8_t*>(w_uk_e4m3);
    a.wscale = w_uk_scale;
    a.out = static_cast<uint16_t*>(q_latent);
    a.T = T;
    a.H = num_heads;
    a.NL = kv_latent_dim;
    a.Dq = (int)Dq;
    a.R = copy_rope ? d_rope : 0;
    a.Do = kv_latent_dim + a.R;
    const hipError_t e = mla::launch_absorb_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_write_latent_paged(const void* kv_input, const uint32_t* input_row_offsets,
                                            int32_t total_tokens, const float* kv_norm_gamma, float epsilon,
                                            const float* freqs_cis, int32_t max_seq_len, int32_t K,
                                            const mla_paged_cache_t* cache, uint32_t layer_idx, void* stream)
{
    if (!cache)
        return MLA_ERR_NULL_POINTER;
    const bool work = total_tokens > 0;
    const int64_t D = (int64_t)cache->num_heads * cache->head_dim;
    const int64_t R = D - K;   // rope columns after the K latent ones
    if (work && (!kv_input || !input_row_offsets || !kv_norm_gamma || !cache->blocks || !cache->page_table ||
                 !cache->cache_lengths || (R > 0 && !freqs_cis)))
        return MLA_ERR_NULL_POINTER;
    if (total_tokens < 0 || K <= 0 || K % 8 || K > 512 || R < 0 || R % 8 || R > 512 || (R > 0 && max_seq_len <= 0) ||
        !(epsilon >= 0.0f))
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    if (cache->dtype != MLA_DTYPE_BF16)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(kv_input) || !aligned16(kv_norm_gamma) || !aligned16(freqs_cis))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::LatentWriteArgs a{};
    a.X = static_cast<const uint16_t*>(kv_input);
    a.iro = input_row_offsets;
    a.cache_len = cache->cache_lengths;
    a.gamma = kv_norm_gamma;
    a.freqs = freqs_cis;
    a.eps = epsilon;
    a.L = layer_view(cache, layer_idx);
    a.T = total_tokens;
    a.K = K;
    a.R = (int)R;
    a.D = (int)D;
    a.max_seq = R > 0 ? max_seq_len : 1;
    const hipError_t e = mla::launch_latent_write(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_write_latent_paged_fp8(const void* kv_input, const uint32_t* input_row_offsets,
                                                int32_t total_tokens, const float* kv_norm_gamma, float epsilon,
                                                const float* freqs_cis, int32_t max_seq_len, int32_t K,
                                                const mla_paged_cache_t* cache, const mla_cache_scales_t* cache_scales,
                                                uint32_t layer_idx, void* stream)
{
    if (!cache || !cache_scales)
        return MLA_ERR_NULL_POINTER;
    const bool work = total_tokens > 0;
    const int64_t D = (int64_t)cache->num_heads * cache->head_dim;
    const int64_t R = D - K;   // rope columns after the K latent ones
    if (work && (!kv_input || !input_row_offsets || !kv_norm_gamma || !cache->blocks || !cache->page_table ||
                 !cache->cache_lengths || !cache_scales->scales || (R > 0 && !freqs_cis)))
        return MLA_ERR_NULL_POINTER;
    const int64_t nblk = (D + 127) / 128;
    if (total_tokens < 0 || K <= 0 || K % 128 || K > 512 || R < 0 || R % 8 || R > 512 || D % 16 ||
        (R > 0 && max_seq_len <= 0) || !(epsilon >= 0.0f) || cache_scales->granularity != 128 ||
        cache_scales->stride_token < nblk || cache_scales->stride_page <= 0 || cache_scales->stride_layer < 0 ||
        cache_scales->stride_kv < 0)
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 1))
        return st;
    if (cache->dtype != MLA_DTYPE_F8E4M3FN)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(kv_input) || !aligned16(kv_norm_gamma) || !aligned16(freqs_cis) ||
        (reinterpret_cast<uintptr_t>(cache_scales->scales) & 3u))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::LatentWriteArgs a{};
    a.X = static_cast<const uint16_t*>(kv_input);
    a.iro = input_row_offsets;
    a.cache_len = cache->cache_lengths;
    a.gamma = kv_norm_gamma;
    a.freqs = freqs_cis;
    a.eps = epsilon;
    a.L = layer_view(cache, layer_idx);
    a.Ls = a.L;
    a.Ls.base = reinterpret_cast<const char*>(cache_scales->scales + (int64_t)layer_idx * cache_scales->stride_layer);
    a.Ls.stride_page = cache_scales->stride_page * 4;
    a.Ls.stride_token = cache_scales->stride_token * 4;
    a.Ls.stride_kv = cache_scales->stride_kv * 4;
    a.T = total_tokens;
    a.K = K;
    a.R = (int)R;
    a.D = (int)D;
    a.max_seq = R > 0 ? max_seq_len : 1;
    const hipError_t e = mla::launch_latent_write_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t kv_matmul_paged(const void* hidden_state, const uint32_t* input_row_offsets,
                                     int32_t total_tokens, int32_t hidden_dim, const void* weight,
                                     const mla_paged_cache_t* cache, uint32_t layer_idx, void* stream)
{
    if (!cache)
        return MLA_ERR_NULL_POINTER;
    const bool work = total_tokens > 0;
    if (work && (!hidden_state || !input_row_offsets || !weight || !cache->blocks || !cache->page_table ||
                 !cache->cache_lengths))
        return MLA_ERR_NULL_POINTER;
    if (total_tokens < 0 || hidden_dim <= 0 || hidden_dim % 64)
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_cache_shape(cache, 2))
        return st;
    const int64_t HD = (int64_t)cache->num_heads * cache->head_dim;
    if (HD % 64 || (int64_t)hidden_dim * 2 * HD * 2 >= (int64_t(1) << 31) || !tile_fits_32bit(hidden_dim, 2))
        return MLA_ERR_INVALID_SHAPE;
    if (cache->dtype != MLA_DTYPE_BF16)
        return MLA_ERR_INVALID_DTYPE;
    if (!aligned16(hidden_state) || !aligned16(weight))
        return MLA_ERR_MISALIGNED;
    if (mla_status_t st = check_cache_alignment(cache))
        return st;
    if (layer_idx >= cache->num_layers)
        return MLA_ERR_OUT_OF_RANGE;
    if (!work)
        return MLA_OK;
    if (mla_status_t st = check_device())
        return st;

    mla::KvMatmulArgs a{};
    a.H = static_cast<const uint16_t*>(hidden_state);
    a.iro = input_row_offsets;
    a.W = static_cast<const uint16_t*>(weight);
    a.cache_len = cache->cache_lengths;
    a.L = layer_view(cache, layer_idx);
    a.T = total_tokens;
    a.Kd = hidden_dim;
    a.N = (int)(2 * HD);
    a.HD = (int)HD;
    const hipError_t e = mla::launch_kv_matmul(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLA_OK : hip_failed(e);
}

MLA_API mla_status_t mla_check_indices(const uint32_t* row_offsets, const uint32_t* cache_offsets,
                                       int32_t rows, const mla_paged_cache_t* cache, int64_t* bad_request,
                                       void* stream)
{
    if (bad_request)
        *bad_request = -1;
    if (!cache || !row_offsets || !cache->page_table)
        return MLA_ERR_NULL_POINTER;
    if (!cache_offsets && !cache->cache_lengths)
        return MLA_ERR_NULL_POINTER;
    if (rows < 0 || cache->batch_size == 0 || cache->max_pages_per_seq == 0 || cache->page_size == 0 ||
        cache->num_pages == 0)
        return MLA_ERR_INVALID_SHAPE;
    if (mla_status_t st = check_device())
        return st;
    const size_t B = cache->batch_size, P = cache->max_pages_per_seq;
    std::vector<uint32_t> off(B + 1), co(cache_offsets ? B : 0), len(cache->cache_lengths ? B : 0), pt(B * P);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(off.data(), row_offsets, off.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && cache_offsets)
        e = hipMemcpyAsync(co.data(), cache_offsets, co.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && cache->cache_lengths)
        e = hipMemcpyAsync(len.data(), cache->cache_lengths, len.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(pt.data(), cache->page_table, pt.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_failed(e);

    auto fail = [&](int64_t b, mla_status_t st) {
        if (bad_request)
            *bad_request = b;
        return st;
    };
    if (off[0] != 0)
        return fail(0, MLA_ERR_INVALID_SHAPE);
    for (size_t b = 0; b < B; ++b)
        if (off[b + 1] < off[b])
            return fail((int64_t)b, MLA_ERR_INVALID_SHAPE);
    if (off[B] != (uint32_t)rows)
        return fail((int64_t)B, MLA_ERR_INVALID_SHAPE);
    for (size_t b = 0; b < B; ++b) {
        const uint64_t n = off[b + 1] - off[b];
        if (n == 0)
            continue;
        // Positions [first, first + n) of request b are read (cache_offsets given)
        // or written (appended after cache_lengths).
        const uint64_t first = cache_offsets ? co[b] : len[b];
        const uint64_t end = first + n;
        if (cache_offsets && cache->cache_lengths && end > len[b])
            return fail((int64_t)b, MLA_ERR_OUT_OF_RANGE);
        if (end > (uint64_t)P * cache->page_size)
            return fail((int64_t)b, MLA_ERR_OUT_OF_RANGE);
        for (uint64_t lp = first / cache->page_size; lp <= (end - 1) / cache->page_size; ++lp)
            if (pt[b * P + lp] >= cache->num_pages)
                return fail((int64_t)b, MLA_ERR_OUT_OF_RANGE);
    }
    return MLA_OK;
}

MLA_API const char* mla_status_string(mla_status_t s)
{
    switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_POINTER: return "null pointer";
    case MLA_ERR_INVALID_SHAPE: return "invalid shape";
    case MLA_ERR_INVALID_DTYPE: return "invalid dtype";
    case MLA_ERR_MISALIGNED: return "misaligned pointer or stride";
    case MLA_ERR_OUT_OF_RANGE: return "index out of range";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_UNSUPPORTED_DEVICE: return "current device is not a gfx950";
    case MLA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

MLA_API int32_t mla_last_hip_error(void) { return g_last_hip_error; }

MLA_API int32_t mla_abi_version(void) { return MLA_PAGED_ABI_VERSION; }
