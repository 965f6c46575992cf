// pa_decode entry points: host-side validation, workspace layout, the
// log-sum-exp reduce kernel, and dispatch to the partition kernels.

#include <math.h>

#include <mutex>

#include "pa_decode_kernel.hpp"

namespace pa {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int num_partitions(int max_seq_len, int partition_size) {
    return (max_seq_len + partition_size - 1) / partition_size;
}

// Workspace: m and l | acc[N][H][P_max][D] (float32) | plan (int32: count,
// then N * P_max work items) | skipped partitions per sequence (int32 [N],
// shared-prefix decode), each part starting on a 256-byte boundary.  m and l
// are either records (ML_REC float32 per (sequence, kv head, partition),
// sized for N * H * P_max, the most kv heads there can be) or, for calls
// whose partition kernel is the GQA-4 one, m[N][H][P_max] then l[N][H][P_max]
// (256-byte aligned) inside the same area.
static size_t plan_offset(int num_seqs, int num_heads, int head_dim, int max_parts) {
    const size_t rows = (size_t)num_seqs * num_heads * max_parts;
    return align256(rows * ML_REC * 4) + align256(rows * head_dim * 4);
}
static size_t skip_offset(int num_seqs, int num_heads, int head_dim, int max_parts) {
    return plan_offset(num_seqs, num_heads, head_dim, max_parts) +
           align256(4 * (PLAN_ITEMS_OFFSET + (size_t)num_seqs * max_parts));
}
static size_t workspace_bytes_for(int num_seqs, int num_heads, int head_dim, int max_parts) {
    return skip_offset(num_seqs, num_heads, head_dim, max_parts) + 4 * (size_t)num_seqs;
}

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 1024;

// Work order for the partition kernel: every (sequence, partition) item,
// largest first.  Workgroups are dispatched in index order, so giving the
// low indices to the full partitions and the high ones to the short
// remainders keeps the last workgroups short (largest-processing-time-first
// list scheduling).  One workgroup; a counting sort on the partition's size in
// blocks (sizes beyond PLAN_BUCKETS share the last bucket).  The order inside a
// bucket may vary between calls; the results do not, since every item is
// computed the same way whichever workgroup takes it.
__global__ void __launch_bounds__(PLAN_THREADS) decode_plan_kernel(const DecodeArgs a) {
    __shared__ int hist[PLAN_BUCKETS];
    __shared__ int scan[PLAN_BUCKETS];
    const int tid = threadIdx.x;
    const int B = a.block_size;
    const int P = a.partition_size;
    const int PB = P / B;  // blocks of a full partition
    const int NBK = min(PB, PLAN_BUCKETS);
    auto bucket = [&](int size) { return min(PB - size, NBK - 1); };  // 0 = full partitions
    for (int k = tid; k < PLAN_BUCKETS; k += PLAN_THREADS) hist[k] = 0;
    __syncthreads();
    // items of sequence i: its partitions from skip_parts[i] on
    auto first_part = [&](int i, int np) { return a.skip_parts ? min(max(a.skip_parts[i], 0), np) : 0; };
    for (int i = tid; i < a.num_seqs; i += PLAN_THREADS) {
        const int T = a.seq_lens[i];
        if (T <= 0 || T > a.max_seq_len || (T + B - 1) / B > a.max_blocks_per_seq) continue;
        const int np = (T + P - 1) / P;
        const int last = (T + B - 1) / B - (np - 1) * PB;
        const int p0 = first_part(i, np);
        if (p0 >= np) continue;
        if (np - 1 > p0) atomicAdd(&hist[0], np - 1 - p0);
        atomicAdd(&hist[bucket(last)], 1);
    }
    __syncthreads();
    if (tid < NBK) scan[tid] = hist[tid];
    __syncthreads();
    for (int off = 1; off < NBK; off <<= 1) {  // inclusive scan
        const int v = (tid < NBK && tid >= off) ? scan[tid - off] : 0;
        __syncthreads();
        if (tid < NBK) scan[tid] += v;
        __syncthreads();
    }
    if (tid < NBK) hist[tid] = scan[tid] - hist[tid];  // first slot of each bucket
    if (tid == 0) a.plan[0] = scan[NBK - 1];
    __syncthreads();
    for (int i = tid; i < a.num_seqs; i += PLAN_THREADS) {
        const int T = a.seq_lens[i];
        if (T <= 0 || T > a.max_seq_len || (T + B - 1) / B > a.max_blocks_per_seq) continue;
        const int np = (T + P - 1) / P;
        const int last = (T + B - 1) / B - (np - 1) * PB;
        for (int p = first_part(i, np); p < np; ++p) {
            const int pos = atomicAdd(&hist[bucket(p < np - 1 ? PB : last)], 1);
            a.plan[PLAN_ITEMS_OFFSET + pos] = i * a.max_partitions + p;
        }
    }
}

// Wave-wide max (every lane receives the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

constexpr int REDUCE_THREADS = 256;
constexpr int REDUCE_UNROLL = 8;

// Merge the partition states of each (sequence, query head) row with the
// log-sum-exp rule: M = max_p m_p, L = sum_p 2^(m_p - M) l_p, out = sum_p
// 2^(m_p - M) acc_p / L (m_p is in log2 units).
//
// A row takes TPR = (D / 4) * RG threads: thread (pg, c4) owns columns
// 4 c4 .. 4 c4 + 3 of partitions pg, pg + RG, pg + 2 RG, ..., loaded
// REDUCE_UNROLL at a time so that many loads are in flight; the first batch
// is loaded before the row maximum is known.  RG (partition groups per row)
// is chosen from the largest partition count, so short rows share a
// workgroup instead of idling most of one.  The groups' sums are added in
// group order, so the result does not depend on timing.  Also writes the
// rows the partition kernel does not: empty sequences (zeros) and invalid
// ones (NaN).
template <int D, int RG>
__global__ void __launch_bounds__(REDUCE_THREADS) decode_reduce_kernel(const DecodeArgs a) {
    constexpr int C4 = D / 4;
    constexpr int TPR = C4 * RG;
    constexpr int RPW = REDUCE_THREADS / TPR;  // rows per workgroup
    constexpr int U = REDUCE_UNROLL;
    static_assert(REDUCE_THREADS % TPR == 0, "rows must tile the workgroup");
    __shared__ float red_m[RPW][RG];
    __shared__ float red_l[RPW][RG];
    __shared__ float4 red_a[RPW][RG][C4];
    const int tid = threadIdx.x;
    const int rw = tid / TPR;
    const int rt = tid - rw * TPR;
    const int pg = rt / C4;
    const int c4 = rt - pg * C4;
    const size_t row = (size_t)blockIdx.x * RPW + rw;
    const bool in_grid = row < (size_t)a.num_seqs * a.num_heads;
    const int seq = in_grid ? (int)((unsigned)row / (unsigned)a.num_heads) : 0;  // in the grid: row < 2^31
    const int T = in_grid ? a.seq_lens[seq] : 0;
    auto store4 = [&](float4 o) {
        const size_t idx = row * D + 4 * c4;
        store_out(a.out, a.out_dtype, idx, o.x);
        store_out(a.out, a.out_dtype, idx + 1, o.y);
        store_out(a.out, a.out_dtype, idx + 2, o.z);
        store_out(a.out, a.out_dtype, idx + 3, o.w);
    };
    const bool bad = T < 0 || T > a.max_seq_len || (T + a.block_size - 1) / a.block_size > a.max_blocks_per_seq;
    if (in_grid && pg == 0 && (bad || T == 0)) {
        const float v = bad ? __builtin_nanf("") : 0.f;
        store4(float4{v, v, v, v});
    }
    // rows of one partition were finished by the partition kernel
    const int n_parts = (!in_grid || bad || T == 0) ? 0 : (T + a.partition_size - 1) / a.partition_size;
    const bool merge = n_parts > 1;
    const size_t base = row * a.max_partitions;
    // m and l of partition p: pm[p * ms], pl[p * ms]
    const int hq = in_grid ? (int)(row - (size_t)seq * a.num_heads) : 0;
    const int G = a.num_heads / a.num_kv_heads;
    const int kvh = hq / G;
    const int ms = a.ml_records ? ML_REC : 1;  // stride between partitions
    const float* pm = a.ml_records ? a.part_ml + ml_record(a, seq, kvh, 0) + (hq - kvh * G) : a.part_m + base;
    const float* pl = a.ml_records ? pm + ML_L : a.part_l + base;
    const float4* pacc = (const float4*)(a.part_acc + base * D) + c4;

    float mv[U], lv[U];
    float4 av[U];
    auto load_batch = [&](int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * RG;
            const bool have = merge && p < n_parts;
            mv[u] = have ? pm[(size_t)p * ms] : -INFINITY;
            lv[u] = have ? pl[(size_t)p * ms] : 0.f;
            av[u] = have ? pacc[(size_t)p * C4] : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    float4 A = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    auto add_batch = [&](int p0, float M) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = merge && p0 + u * RG < n_parts ? fast_exp2(mv[u] - M) : 0.f;
            L = fmaf(w, lv[u], L);
            A.x = fmaf(w, av[u].x, A.x);
            A.y = fmaf(w, av[u].y, A.y);
            A.z = fmaf(w, av[u].z, A.z);
            A.w = fmaf(w, av[u].w, A.w);
        }
    };

    load_batch(pg);
    float mx = mv[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, mv[u]);
    for (int p = pg + RG * U; merge && p < n_parts; p += RG) mx = fmaxf(mx, pm[(size_t)p * ms]);
    float M = mx;
    if constexpr (RG > 1) {  // with one group every thread of the row already holds the row's maximum
        if (c4 == 0) red_m[rw][pg] = mx;
        __syncthreads();
        M = red_m[rw][0];
#pragma unroll
        for (int r = 1; r < RG; ++r) M = fmaxf(M, red_m[rw][r]);
    }
    add_batch(pg, M);
    for (int p0 = pg + RG * U; merge && p0 < n_parts; p0 += RG * U) {
        load_batch(p0);
        add_batch(p0, M);
    }
    if constexpr (RG == 1) {  // the thread holds its columns' whole sums: no exchange
        if (merge) store4(float4{A.x / L, A.y / L, A.z / L, A.w / L});
        return;
    }
    red_a[rw][pg][c4] = A;
    if (c4 == 0) red_l[rw][pg] = L;
    __syncthreads();
    if (merge && pg == 0) {
        float4 S = red_a[rw][0][c4];
        float Ls = red_l[rw][0];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            const float4 v = red_a[rw][r][c4];
            S.x += v.x; S.y += v.y; S.z += v.z; S.w += v.w;
            Ls += red_l[rw][r];
        }
        store4(float4{S.x / Ls, S.y / Ls, S.z / Ls, S.w / Ls});
    }
}

template <int D, int RG>
static void launch_reduce(const DecodeArgs& a, hipStream_t stream) {
    constexpr int RPW = REDUCE_THREADS / (D / 4 * RG);
    const size_t rows = (size_t)a.num_seqs * a.num_heads;
    const dim3 grid((unsigned)((rows + RPW - 1) / RPW));
    hipLaunchKernelGGL((decode_reduce_kernel<D, RG>), grid, dim3(REDUCE_THREADS), 0, stream, a);
}

template <int D>
static void launch_reduce_for(const DecodeArgs& a, hipStream_t stream) {
    const int mp = a.max_partitions;
    if (mp <= REDUCE_UNROLL) launch_reduce<D, 1>(a, stream);
    else if (mp <= 2 * REDUCE_UNROLL) launch_reduce<D, 2>(a, stream);
    else if (mp <= 4 * REDUCE_UNROLL) launch_reduce<D, 4>(a, stream);
    else launch_reduce<D, 8>(a, stream);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Point the partition states and the plan into a workspace laid out as
// workspace_bytes_for describes (rows = N * H * P_max state rows).
static void bind_workspace(DecodeArgs& a, void* workspace, size_t rows, size_t plan_at) {
    a.part_ml = (float*)workspace;
    a.part_m = (float*)workspace;
    a.part_l = (float*)((char*)workspace + align256(rows * 4));
    a.part_acc = (float*)((char*)workspace + align256(rows * ML_REC * 4));
    a.plan = (int*)((char*)workspace + plan_at);
}

struct Prepared {
    DecodeArgs args;
    int head_dim;
    int group;
    int kv_dtype;
    int q_dtype;
    bool nothing_to_do;
};

static int prepare(Prepared& pr, void* out, int out_dtype, const void* q, int q_dtype,
                   const void* k_cache, const void* v_cache, int kv_dtype,
                   const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                   int max_seq_len, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, float scale, const float* k_scale,
                   const float* v_scale, int partition_size, void* workspace,
                   size_t workspace_bytes, bool bind_later = false) {
    const bool combo_ok = (kv_dtype == PA_DTYPE_F32 && q_dtype == PA_DTYPE_F32) ||
                          (kv_dtype == PA_DTYPE_F16 && q_dtype == PA_DTYPE_F16) ||
                          (kv_dtype == PA_DTYPE_BF16 && q_dtype == PA_DTYPE_BF16) ||
                          (kv_dtype == PA_DTYPE_FP8_E4M3 && q_dtype == PA_DTYPE_BF16);
    if (!combo_ok) return PA_ERR_DTYPE;
    if (out_dtype != PA_DTYPE_F32 && out_dtype != PA_DTYPE_F16 && out_dtype != PA_DTYPE_BF16)
        return PA_ERR_DTYPE;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
        max_blocks_per_seq < 0 || num_blocks <= 0 || partition_size <= 0 || block_size <= 0 ||
        head_dim <= 0)
        return PA_ERR_SHAPE;
    if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    const int group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
    if (partition_size % block_size != 0) return PA_ERR_SHAPE;
    if ((long long)max_blocks_per_seq * block_size < (long long)max_seq_len) return PA_ERR_SHAPE;
    const int max_parts = num_partitions(max_seq_len, partition_size);
    if (max_parts > 65535) return PA_ERR_SHAPE;
    if ((long long)num_seqs * num_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    // partition grid: one workgroup per (item, kv head), at most 512 threads each
    if ((long long)num_seqs * max_parts * num_kv_heads * 512 > 0xffffffffLL) return PA_ERR_SHAPE;
    pr.nothing_to_do = num_seqs == 0;
    if (pr.nothing_to_do) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
    if (kv_dtype == PA_DTYPE_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_SHAPE;
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, max_parts);
    if (!bind_later) {
        if (need > 0 && !workspace) return PA_ERR_NULL;
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
        if (need > 0 && !aligned16(workspace)) return PA_ERR_SHAPE;
    }

    const size_t rows = (size_t)num_seqs * num_heads * max_parts;
    DecodeArgs& a = pr.args;
    a.out = out;
    a.out_dtype = out_dtype;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.max_seq_len = max_seq_len;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.qk_scale_log2 = scale * kLog2e;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.partition_size = partition_size;
    a.max_partitions = max_parts;
    bind_workspace(a, workspace, rows, plan_offset(num_seqs, num_heads, head_dim, max_parts));
    a.inline_plan = num_seqs <= INLINE_PLAN_MAX_SEQS && partition_size / block_size <= INLINE_PLAN_MAX_BLOCKS;
    a.ml_records = partition_kernel_is_gqa4(kv_dtype, group) ? 0 : 1;
    a.skip_parts = nullptr;
    a.new_k = nullptr;
    a.cow_pairs = nullptr;
    a.cow_num = 0;
    a.new_v = nullptr;
    pr.head_dim = head_dim;
    pr.group = group;
    pr.kv_dtype = kv_dtype;
    pr.q_dtype = q_dtype;
    return PA_OK;
}

// the work order, when the partition workgroups do not compute it themselves
static int run_plan(const Prepared& pr, hipStream_t stream) {
    if (pr.args.max_partitions == 0 || pr.args.inline_plan) return PA_OK;
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, pr.args);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

static int run_partition(const Prepared& pr, hipStream_t stream) {
    if (pr.args.max_partitions == 0) return PA_OK;  // every sequence is empty
    const int sp = run_plan(pr, stream);
    if (sp != PA_OK) return sp;
    switch (pr.kv_dtype) {
        case PA_DTYPE_F32: return launch_partition_f32(pr.args, pr.head_dim, pr.group, stream);
        case PA_DTYPE_F16: return launch_partition_f16(pr.args, pr.head_dim, pr.group, stream);
        case PA_DTYPE_BF16: return launch_partition_bf16(pr.args, pr.head_dim, pr.group, stream);
        case PA_DTYPE_FP8_E4M3: return launch_partition_fp8_bf16q(pr.args, pr.head_dim, pr.group, stream);
    }
    return PA_ERR_DTYPE;
}

// Decode with append, for shapes whose partition kernel does not store the
// new tokens itself: one workgroup per sequence copies the K and V rows of
// its newest token (position seq_lens - 1) into that position's slot, as
// pa_reshape_and_cache would with the slot taken from the block table.
// Sequences with an invalid length or block id are skipped.
__global__ void __launch_bounds__(256) append_tokens_kernel(const u32x4* __restrict__ key,
                                                             const u32x4* __restrict__ value, u32x4* k_cache,
                                                             u32x4* v_cache, const DecodeArgs a, int granules_per_row) {
    const int seq = blockIdx.x;
    const int T = a.seq_lens[seq];
    const int B = a.block_size;
    if (T <= 0 || T > a.max_seq_len || (T + B - 1) / B > a.max_blocks_per_seq) return;
    const int pb = a.block_tables[(size_t)seq * a.max_blocks_per_seq + (T - 1) / B];
    if (pb < 0 || pb >= a.num_blocks) return;
    const int row = (T - 1) % B;
    const int per_tensor = a.num_kv_heads * granules_per_row;
    for (int i = threadIdx.x; i < 2 * per_tensor; i += blockDim.x) {
        const int which = i / per_tensor;  // 0 = K, 1 = V
        const int hg = i - which * per_tensor;
        const int h = hg / granules_per_row;
        const int g = hg - h * granules_per_row;
        const size_t src = ((size_t)seq * a.num_kv_heads + h) * granules_per_row + g;
        const size_t dst = (((size_t)pb * a.num_kv_heads + h) * B + row) * granules_per_row + g;
        if (which == 0)
            k_cache[dst] = key[src];
        else
            v_cache[dst] = value[src];
    }
}

// Shapes whose partition kernel stores the new tokens itself (and takes the
// launch's copy-on-write pairs): the GQA-4 kernel when a partition has at
// most 64 blocks (their ids sit in one vector register), and the generic
// kernel.  The FP8 matrix-core kernel does not.
static bool partition_kernel_is_mfma8(const Prepared& pr);
static bool partition_appends(const Prepared& pr) {
    if (partition_kernel_is_gqa4(pr.kv_dtype, pr.group))
        return pr.args.partition_size / pr.args.block_size <= 64;
    return !partition_kernel_is_mfma8(pr);
}

// The FP8 matrix-core kernel (it takes copy-on-write pairs, but stores no
// new tokens).
static bool partition_kernel_is_mfma8(const Prepared& pr) {
#ifndef PA_DISABLE_MFMA8
    return pr.kv_dtype == PA_DTYPE_FP8_E4M3 && pr.group == 8 && pr.head_dim == 128;
#else
    (void)pr;
    return false;
#endif
}

static int run_reduce(const Prepared& pr, hipStream_t stream) {
    if (pr.head_dim == 128)
        launch_reduce_for<128>(pr.args, stream);
    else
        launch_reduce_for<64>(pr.args, stream);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa

#define PA_DECODE_PARAMS                                                                          \
    void *out, int out_dtype, const void *q, int q_dtype, const void *k_cache, const void *v_cache, \
        int kv_dtype, const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens, \
        int max_seq_len, int num_seqs, int num_heads, int num_kv_heads, int head_dim,             \
        int block_size, int num_blocks, float scale, const float *k_scale, const float *v_scale,  \
        int partition_size, void *workspace, size_t workspace_bytes, void *stream
#define PA_DECODE_ARGS                                                                             \
    out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, max_blocks_per_seq,      \
        seq_lens, max_seq_len, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, \
        scale, k_scale, v_scale, partition_size, workspace, workspace_bytes

extern "C" size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim,
                                           int max_seq_len, int partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || partition_size <= 0)
        return 0;
    return pa::workspace_bytes_for(num_seqs, num_heads, head_dim,
                                   pa::num_partitions(max_seq_len, partition_size));
}

#if PA_CHECK_CONTENTS
#define PA_CHECK_SEQUENCES()                                                                               \
    do {                                                                                                   \
        const int checked = pa::check::sequences(seq_lens, block_tables, num_seqs, max_blocks_per_seq,     \
                                                 max_seq_len, block_size, num_blocks, (hipStream_t)stream); \
        if (checked != PA_OK) return checked;                                                              \
    } while (0)
#else
#define PA_CHECK_SEQUENCES() \
    do {                     \
    } while (0)
#endif

extern "C" int pa_decode_partition(PA_DECODE_PARAMS) {
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK || pr.nothing_to_do) return st;
    PA_CHECK_SEQUENCES();
    return pa::run_partition(pr, (hipStream_t)stream);
}

extern "C" int pa_decode_reduce(PA_DECODE_PARAMS) {
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK || pr.nothing_to_do) return st;
    PA_CHECK_SEQUENCES();
    return pa::run_reduce(pr, (hipStream_t)stream);
}

extern "C" int pa_decode(PA_DECODE_PARAMS) {
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK || pr.nothing_to_do) return st;
    PA_CHECK_SEQUENCES();
    const int s1 = pa::run_partition(pr, (hipStream_t)stream);
    if (s1 != PA_OK) return s1;
    return pa::run_reduce(pr, (hipStream_t)stream);
}

namespace pa {
// Arrange for the partition launch to store the newest tokens (key, value),
// or store them now with the copy kernel when that kernel does not.
static int prepare_append(Prepared& pr, const void* key, const void* value, void* k_cache, void* v_cache,
                          int head_dim, hipStream_t s) {
    if (partition_appends(pr)) {
        pr.args.new_k = key;
        pr.args.new_v = value;
        return PA_OK;
    }
    const int eb = pr.kv_dtype == PA_DTYPE_F32 ? 4 : pr.kv_dtype == PA_DTYPE_FP8_E4M3 ? 1 : 2;
    hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)pr.args.num_seqs), dim3(256), 0, s, (const u32x4*)key,
                       (const u32x4*)value, (u32x4*)k_cache, (u32x4*)v_cache, pr.args, head_dim * eb / 16);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
}  // namespace pa

extern "C" int pa_decode_append(PA_DECODE_PARAMS, const void* key, const void* value) {
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK || pr.nothing_to_do) return st;
    if (!key || !value) return PA_ERR_NULL;
    if (!pa::aligned16(key) || !pa::aligned16(value)) return PA_ERR_SHAPE;
    PA_CHECK_SEQUENCES();
    const hipStream_t s = (hipStream_t)stream;
    const int s0 = pa::prepare_append(pr, key, value, (void*)k_cache, (void*)v_cache, head_dim, s);
    if (s0 != PA_OK) return s0;
    const int s1 = pa::run_partition(pr, s);
    if (s1 != PA_OK) return s1;
    return pa::run_reduce(pr, s);
}

// Copy-on-write copies and decode with append in one launch where the
// partition kernel stores the new tokens; elsewhere pa_copy_blocks, then
// pa_decode_append.  With no new tokens (key and value both null): the
// copies and the decode, in one launch for the FP8 matrix-core shape, else
// pa_copy_blocks, then pa_decode.
extern "C" int pa_decode_append_cow(PA_DECODE_PARAMS, const void* key, const void* value,
                                    const int64_t* block_pairs, int num_pairs) {
    if (num_pairs < 0) return PA_ERR_SHAPE;
    if (num_pairs > 0 && !block_pairs) return PA_ERR_NULL;
    const bool tokens = key != nullptr || value != nullptr;
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK) return st;
    const bool fused = num_pairs > 0 && !pr.nothing_to_do && pr.args.max_partitions > 0 &&
                       num_pairs <= pa::COW_MAX_PAIRS &&
                       (tokens ? pa::partition_appends(pr) : pa::partition_kernel_is_mfma8(pr)) &&
                       (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
    if (!fused) {
        if (tokens && (!key || !value)) return PA_ERR_NULL;
        const int c = pa_copy_blocks((void*)k_cache, (void*)v_cache, block_pairs, num_pairs, num_kv_heads,
                                     head_dim, block_size, num_blocks, kv_dtype, stream);
        if (c != PA_OK) return c;
        return tokens ? pa_decode_append(PA_DECODE_ARGS, stream, key, value) : pa_decode(PA_DECODE_ARGS, stream);
    }
    if (tokens && (!key || !value)) return PA_ERR_NULL;
    if (tokens && (!pa::aligned16(key) || !pa::aligned16(value))) return PA_ERR_SHAPE;
    PA_CHECK_SEQUENCES();
#if PA_CHECK_CONTENTS
    const int cp = pa::check::pairs(block_pairs, num_pairs, num_blocks, num_blocks, true, (hipStream_t)stream);
    if (cp != PA_OK) return cp;
#endif
    const hipStream_t s = (hipStream_t)stream;
    pr.args.new_k = key;
    pr.args.new_v = value;
    pr.args.cow_pairs = block_pairs;
    pr.args.cow_num = num_pairs;
    const int s1 = pa::run_partition(pr, s);
    if (s1 != PA_OK) return s1;
    return pa::run_reduce(pr, s);
}

extern "C" int pa_decode_shared_prefix(PA_DECODE_PARAMS, const int32_t* group_start, const int32_t* group_prefix,
                                       int num_groups, int max_group_size, int max_prefix_len, const void* key,
                                       const void* value) {
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS);
    if (st != PA_OK || pr.nothing_to_do) return st;
    if (num_groups < 0 || max_group_size < 0 || max_prefix_len < 0) return PA_ERR_SHAPE;
    if (num_groups > 0 && (!group_start || !group_prefix)) return PA_ERR_NULL;
    if (!key != !value) return PA_ERR_NULL;  // both or neither
    if (key && (!pa::aligned16(key) || !pa::aligned16(value))) return PA_ERR_SHAPE;
    const hipStream_t s = (hipStream_t)stream;
#if PA_CHECK_CONTENTS
    {
        std::vector<int32_t> lens, tables;
        int checked = pa::check::sequences(seq_lens, block_tables, num_seqs, max_blocks_per_seq, max_seq_len,
                                           block_size, num_blocks, lens, tables, s);
        if (checked == PA_OK && num_groups > 0)
            checked = pa::check::groups(group_start, group_prefix, num_groups, num_seqs, max_blocks_per_seq,
                                        block_size, lens, tables, key != nullptr, s);
        if (checked != PA_OK) return checked;
    }
#endif
    if (key) {
        const int sa = pa::prepare_append(pr, key, value, (void*)k_cache, (void*)v_cache, head_dim, s);
        if (sa != PA_OK) return sa;
    }
    // nothing to share, or a shape the matrix-core tile does not cover: plain decode
    if (num_groups == 0 || max_prefix_len < partition_size || max_group_size == 0 || ((uintptr_t)out & 15u) ||
        !pa::prefix_states_supported(pr.kv_dtype, pr.q_dtype, pr.head_dim, block_size, pr.group)) {
        const int s1 = pa::run_partition(pr, s);
        if (s1 != PA_OK) return s1;
        return pa::run_reduce(pr, s);
    }
    int32_t* skip = (int32_t*)((char*)workspace + pa::skip_offset(num_seqs, num_heads, head_dim,
                                                                  pr.args.max_partitions));
    if (pa::prefix_fused_supported(pr.kv_dtype, pr.q_dtype, pr.head_dim, block_size, pr.group)) {
        // the skips, the work order, then the shared and the decode partitions in one launch
        pr.args.skip_parts = skip;
        int sf = pa::launch_prefix_skips(pr.args, group_start, group_prefix, num_groups, max_group_size,
                                         max_prefix_len, skip, s);
        if (sf == PA_OK) sf = pa::run_plan(pr, s);
        if (sf == PA_OK)
            sf = pa::launch_prefix_fused(pr.args, pr.kv_dtype, group_start, group_prefix, num_groups, max_group_size,
                                         max_prefix_len, skip, s);
        if (sf != PA_OK) return sf;
        return pa::run_reduce(pr, s);
    }
    const int s0 = pa::launch_prefix_states(pr.args, pr.kv_dtype, pr.group, group_start, group_prefix, num_groups,
                                            max_group_size, max_prefix_len, skip, s);
    if (s0 != PA_OK) return s0;
    pr.args.skip_parts = skip;
    const int s1 = pa::run_partition(pr, s);
    if (s1 != PA_OK) return s1;
    return pa::run_reduce(pr, s);
}

// ------------------------------------------------------------ pa_decode_noalloc
//
// pa_decode with its workspace in a static device array instead of the
// caller's buffer, for callers that cannot allocate.  The array is a
// file-scope __device__ variable: every GPU the library runs on holds its own
// copy (PA_DECODE_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code
// never uses the variable's name as an address (on the host it is only a
// stand-in); its device address is looked up once per device with that device
// current and kept in scratch_ptr.

static __device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace pa {

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[SCRATCH_MAX_DEVICES];

// Device address of `scratch` on the device that runs `stream`.
static int scratch_for_stream(hipStream_t stream, void** out) {
    int current = 0;
    if (hipGetDevice(&current) != hipSuccess) return PA_ERR_LAUNCH;
    int dev = current;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return PA_ERR_LAUNCH;
        dev = (int)d;
    }
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != current && hipSetDevice(dev) != hipSuccess) return PA_ERR_LAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != current) (void)hipSetDevice(current);
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return PA_ERR_LAUNCH;
        }
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return PA_OK;
}

}  // namespace pa

extern "C" int pa_decode_noalloc(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                                 const void* v_cache, int kv_dtype, const int32_t* block_tables,
                                 int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_seqs,
                                 int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 float scale, const float* k_scale, const float* v_scale, int partition_size,
                                 void* stream) {
    // every argument is checked before the device is touched
    void* workspace = nullptr;
    const size_t workspace_bytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
    pa::Prepared pr;
    const int st = pa::prepare(pr, PA_DECODE_ARGS, /*bind_later=*/true);
    if (st != PA_OK || pr.nothing_to_do) return st;
    const int mp = pr.args.max_partitions;
    if (pa::workspace_bytes_for(num_seqs, num_heads, head_dim, mp) > workspace_bytes) return PA_ERR_SCRATCH;
    const int sp = pa::scratch_for_stream((hipStream_t)stream, &workspace);
    if (sp != PA_OK) return sp;
    pa::bind_workspace(pr.args, workspace, (size_t)num_seqs * num_heads * mp,
                       pa::plan_offset(num_seqs, num_heads, head_dim, mp));
    PA_CHECK_SEQUENCES();
    const int s1 = pa::run_partition(pr, (hipStream_t)stream);
    if (s1 != PA_OK) return s1;
    return pa::run_reduce(pr, (hipStream_t)stream);
}
