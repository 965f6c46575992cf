// KV-cache maintenance kernels for gfx950: the slot scatter of new tokens
// (pa_reshape_and_cache, and the quantizing pa_reshape_and_cache_fp8) and
// the whole-block copy used by copy-on-write (pa_copy_blocks) and by
// swapping between the device pool and a pinned host pool (pa_swap_blocks).
// The scatter and the copies move stored elements as 16-byte granules, so
// they are bitwise and independent of the element format.
//
// Pool layout: cache[num_blocks][num_kv_heads][block_size][head_dim]; one
// token row of one head is head_dim * elem_bytes contiguous bytes (64..512,
// always a multiple of 16).

#include "pa_common.hpp"

namespace pa {

// One thread per 16-byte granule of the (token, K|V, head, granule) space.
// The granule index runs fastest over the row, then heads, then K/V, then
// tokens, so consecutive lanes read consecutive source bytes.
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                         u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                         const int64_t* __restrict__ slot_mapping, int64_t total_granules,
                         int granules_per_row, int num_kv_heads, int block_size,
                         int64_t num_slots) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total_granules) return;
    const int per_token = 2 * num_kv_heads * granules_per_row;
    const int64_t t = idx / per_token;
    const int rem = (int)(idx - t * per_token);
    const int which = rem / (num_kv_heads * granules_per_row);  // 0 = K, 1 = V
    const int hg = rem - which * num_kv_heads * granules_per_row;
    const int h = hg / granules_per_row;
    const int g = hg - h * granules_per_row;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t block = slot / block_size;
    const int64_t row = slot - block * block_size;
    const int64_t src = (t * num_kv_heads + h) * granules_per_row + g;
    const int64_t dst = ((block * num_kv_heads + h) * block_size + row) * granules_per_row + g;
    if (which == 0)
        k_cache[dst] = key[src];
    else
        v_cache[dst] = value[src];
}

// grid.y = pair, grid.z = K|V; each thread copies one 16-byte granule of
// the whole (all heads, all rows) block from the source pool to the
// destination pool (the same pool for copy-on-write; device and pinned host
// memory for swapping).
__global__ void __launch_bounds__(256)
copy_blocks_kernel(const u32x4* src_k, const u32x4* src_v, u32x4* dst_k, u32x4* dst_v,
                   const int64_t* __restrict__ block_pairs, int granules_per_block,
                   int64_t src_blocks, int64_t dst_blocks) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= granules_per_block) return;
    const int64_t src = block_pairs[2 * (int64_t)blockIdx.y];
    const int64_t dst = block_pairs[2 * (int64_t)blockIdx.y + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
    const u32x4* from = blockIdx.z == 0 ? src_k : src_v;
    u32x4* to = blockIdx.z == 0 ? dst_k : dst_v;
    to[dst * granules_per_block + g] = from[src * granules_per_block + g];
}

// Quantize-on-write: one thread per 16 output codes (16 elements of one
// token row of one head).  code = E4M3FN(x / scale[h]): the quotient is the
// IEEE float32 division, NaN stays NaN (code 0x7F), and magnitudes beyond
// 448 saturate to 448 before the round-to-nearest-even conversion.
template <Fmt SRC>
__global__ void __launch_bounds__(256)
reshape_and_cache_fp8_kernel(const char* __restrict__ key, const char* __restrict__ value,
                             uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                             const float* __restrict__ k_scale, const float* __restrict__ v_scale,
                             const int64_t* __restrict__ slot_mapping, int64_t total, int groups_per_row,
                             int num_kv_heads, int block_size, int head_dim, int64_t num_slots) {
    constexpr int SB = FmtBytes<SRC>::value;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int per_token = 2 * num_kv_heads * groups_per_row;
    const int64_t t = idx / per_token;
    const int rem = (int)(idx - t * per_token);
    const int which = rem / (num_kv_heads * groups_per_row);
    const int hg = rem - which * num_kv_heads * groups_per_row;
    const int h = hg / groups_per_row;
    const int g = hg - h * groups_per_row;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t block = slot / block_size;
    const int64_t row = slot - block * block_size;
    const char* src = (which == 0 ? key : value) + ((t * num_kv_heads + h) * head_dim + g * 16) * SB;
    const float scale = (which == 0 ? k_scale : v_scale)[h];
    float x[16];
    if constexpr (SRC == Fmt::F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = ((const float4*)src)[i];
            x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 v = ((const u32x4*)src)[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                x[8 * i + 2 * p] = SRC == Fmt::BF16 ? bf16_lo(w[p]) : f16_lo(w[p]);
                x[8 * i + 2 * p + 1] = SRC == Fmt::BF16 ? bf16_hi(w[p]) : f16_hi(w[p]);
            }
        }
    }
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float q[4];
        bool nan[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = __fdiv_rn(x[4 * i + j], scale);
            nan[j] = v != v;
            q[j] = nan[j] ? 0.f : fminf(fmaxf(v, -448.f), 448.f);
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
        uint32_t u = (uint32_t)w;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (nan[j]) u = (u & ~(0xffu << (8 * j))) | (0x7fu << (8 * j));
        packed[i] = u;
    }
    uint8_t* dst = (which == 0 ? k_cache : v_cache) + ((block * num_kv_heads + h) * block_size + row) * head_dim + g * 16;
    *(u32x4*)dst = u32x4{packed[0], packed[1], packed[2], packed[3]};
}

static bool valid_kv_dtype(int d) { return d >= PA_DTYPE_F32 && d <= PA_DTYPE_FP8_E4M3; }
static bool supported_dim(int d) { return d == 64 || d == 128; }
static bool supported_block(int b) { return b == 16 || b == 32; }

}  // namespace pa

extern "C" const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
        case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid or inconsistent size";
        case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown or unsupported dtype combination";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size or GQA group not built";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace too small";
        case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
        case PA_ERR_MEMORY: return "PA_ERR_MEMORY: a pool is neither device memory nor pinned host memory the device can address";
        case PA_ERR_CONTENT: return "PA_ERR_CONTENT: device contents break the call's contract (checked build)";
        case PA_ERR_SCRATCH: return "PA_ERR_SCRATCH: pa_decode_noalloc needs more workspace than its static scratch holds";
        default: return "unknown pa_status";
    }
}

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int kv_dtype, void* stream) {
    using namespace pa;
    if (!valid_kv_dtype(kv_dtype)) return PA_ERR_DTYPE;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_SHAPE;
    if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
    // rows and pool are moved as 16-byte granules
    if (((uintptr_t)key | (uintptr_t)value | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15u) return PA_ERR_SHAPE;
    const int granules_per_row = head_dim * dtype_bytes(kv_dtype) / 16;
    const int64_t total = (int64_t)num_tokens * 2 * num_kv_heads * granules_per_row;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffffLL) return PA_ERR_SHAPE;
#if PA_CHECK_CONTENTS
    const int checked = check::slots(slot_mapping, num_tokens, num_blocks, block_size, (hipStream_t)stream);
    if (checked != PA_OK) return checked;
#endif
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, (const u32x4*)key, (const u32x4*)value,
                       (u32x4*)k_cache, (u32x4*)v_cache, slot_mapping, total, granules_per_row,
                       num_kv_heads, block_size, (int64_t)num_blocks * block_size);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" int pa_reshape_and_cache_fp8(const void* key, const void* value, int src_dtype,
                                        void* k_cache, void* v_cache, const float* k_scale,
                                        const float* v_scale, const int64_t* slot_mapping,
                                        int num_tokens, int num_kv_heads, int head_dim,
                                        int block_size, int num_blocks, void* stream) {
    using namespace pa;
    if (src_dtype != PA_DTYPE_F32 && src_dtype != PA_DTYPE_F16 && src_dtype != PA_DTYPE_BF16)
        return PA_ERR_DTYPE;
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_SHAPE;
    if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_cache || !v_cache || !k_scale || !v_scale || !slot_mapping) return PA_ERR_NULL;
    // source rows are read, and codes stored, 16 bytes at a time
    if (((uintptr_t)key | (uintptr_t)value | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15u) return PA_ERR_SHAPE;
    const int groups_per_row = head_dim / 16;
    const int64_t total = (int64_t)num_tokens * 2 * num_kv_heads * groups_per_row;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffffLL) return PA_ERR_SHAPE;
    const int64_t slots = (int64_t)num_blocks * block_size;
    const hipStream_t s = (hipStream_t)stream;
#if PA_CHECK_CONTENTS
    const int checked = check::slots(slot_mapping, num_tokens, num_blocks, block_size, s);
    if (checked != PA_OK) return checked;
#endif
#define PA_LAUNCH_Q(F)                                                                          \
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<F>, dim3((unsigned)grid), dim3(256), 0, s, \
                       (const char*)key, (const char*)value, (uint8_t*)k_cache, (uint8_t*)v_cache,  \
                       k_scale, v_scale, slot_mapping, total, groups_per_row, num_kv_heads,     \
                       block_size, head_dim, slots)
    if (src_dtype == PA_DTYPE_BF16)
        PA_LAUNCH_Q(Fmt::BF16);
    else if (src_dtype == PA_DTYPE_F16)
        PA_LAUNCH_Q(Fmt::F16);
    else
        PA_LAUNCH_Q(Fmt::F32);
#undef PA_LAUNCH_Q
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

namespace pa {
// same_pool: a copy inside one pool (pa_copy_blocks) rather than between two (pa_swap_blocks)
static int launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int64_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                              int block_size, int src_blocks, int dst_blocks, int kv_dtype, bool same_pool,
                              void* stream) {
    if (!valid_kv_dtype(kv_dtype)) return PA_ERR_DTYPE;
    if (num_pairs < 0 || num_kv_heads <= 0 || src_blocks <= 0 || dst_blocks <= 0 || head_dim <= 0 ||
        block_size <= 0)
        return PA_ERR_SHAPE;
    if (!supported_dim(head_dim) || !supported_block(block_size)) return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs) return PA_ERR_NULL;
    if (((uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)dst_k | (uintptr_t)dst_v) & 15u) return PA_ERR_SHAPE;
    if (num_pairs > 65535) return PA_ERR_SHAPE;
    const int64_t granules = (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(kv_dtype) / 16;
    if (granules > 0x7fffffffLL) return PA_ERR_SHAPE;
    const unsigned gx = (unsigned)((granules + 255) / 256);
#if PA_CHECK_CONTENTS
    const int checked = check::pairs(block_pairs, num_pairs, src_blocks, dst_blocks, same_pool, (hipStream_t)stream);
    if (checked != PA_OK) return checked;
#else
    (void)same_pool;
#endif
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, (unsigned)num_pairs, 2), dim3(256), 0,
                       (hipStream_t)stream, (const u32x4*)src_k, (const u32x4*)src_v, (u32x4*)dst_k,
                       (u32x4*)dst_v, block_pairs, (int)granules, (int64_t)src_blocks, (int64_t)dst_blocks);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
}  // namespace pa

extern "C" int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                              int num_pairs, int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, int kv_dtype, void* stream) {
    return pa::launch_copy_blocks(k_cache, v_cache, k_cache, v_cache, block_pairs, num_pairs, num_kv_heads,
                                  head_dim, block_size, num_blocks, num_blocks, kv_dtype, true, stream);
}

namespace pa {
// True when kernels may dereference p: device memory, or pinned host memory
// mapped for the device at the same address.
static bool device_addressable(const void* p) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of an unknown pointer
        return false;
    }
    if (attr.type == hipMemoryTypeDevice) return true;
    if (attr.type == hipMemoryTypeHost) return attr.devicePointer == p;
    return false;
}
}  // namespace pa

extern "C" int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int64_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                              int block_size, int src_num_blocks, int dst_num_blocks, int kv_dtype,
                              void* stream) {
    // argument checks first (the same as for the launch), then the memory kinds
    if (num_pairs > 0 && src_k && src_v && dst_k && dst_v && block_pairs && num_pairs <= 65535 &&
        kv_dtype >= PA_DTYPE_F32 && kv_dtype <= PA_DTYPE_FP8_E4M3 && num_kv_heads > 0 && head_dim > 0 &&
        block_size > 0 && src_num_blocks > 0 && dst_num_blocks > 0 &&
        !(((uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)dst_k | (uintptr_t)dst_v) & 15u) &&
        pa::supported_dim(head_dim) && pa::supported_block(block_size)) {
        for (const void* p : {src_k, src_v, (const void*)dst_k, (const void*)dst_v, (const void*)block_pairs})
            if (!pa::device_addressable(p)) return PA_ERR_MEMORY;
    }
    return pa::launch_copy_blocks(src_k, src_v, dst_k, dst_v, block_pairs, num_pairs, num_kv_heads, head_dim,
                                  block_size, src_num_blocks, dst_num_blocks, kv_dtype, false, stream);
}
