// Shared-prefix decode: the partitions of a prompt that several sequences
// share (the beams of one prompt, forked with every block shared) are read
// once for all of them.
//
// Sequences form groups (group_start); the first group_prefix[g] tokens of
// every member of group g live in the same physical blocks, named by the
// members' tables (the leader's -- the group's first sequence -- are read).
// With partition size P, the first floor(group_prefix[g] / P) partitions are
// whole shared partitions.  For each (group, kv head, shared partition) one
// workgroup runs the multi-query tile of pa_mq_mfma.hpp with every member's
// G query heads as columns (64 / G members per workgroup) over the
// partition's P keys, and writes each member's partition state (m, l, acc)
// into the same workspace slots the decode partition kernel uses; a member
// with a single partition gets its output row directly.  The decode
// partition kernel then skips those partitions (skip_parts) and the reduce
// kernel merges all of a sequence's partitions as usual.
//
// For 4-head groups the shared partitions and the decode partitions run in
// one launch (shared_prefix_fused_kernel): its first workgroups compute the
// shared partitions, the rest are the GQA-4 partition kernel's workgroups.
// Both kinds are short and would each leave the device partly idle.  The
// skips are then written by a small kernel before that launch.
//
// A member that holds fewer tokens than the shared partitions (or whose
// length is invalid) is not shared: its skip is 0 and the decode kernels
// compute it alone.  A leader shorter than the shared partitions disables
// sharing for its group.
#include "pa_decode_gqa.hpp"
#include "pa_mq_mfma.hpp"

#ifndef PA_PREFIX_STAGES
#define PA_PREFIX_STAGES 4
#endif

namespace pa {

struct PrefixArgs {
    DecodeArgs d;
    MqPool pool;
    const int32_t* group_start;   // [num_groups + 1]
    const int32_t* group_prefix;  // [num_groups] shared tokens
    int num_groups;
    int chunks;                   // member chunks per group in the grid
    int parts;                    // shared partitions per group in the grid
    int member_cap;               // members per group the grid covers (chunks * columns per workgroup)
    bool write_skips;             // the states' workgroups write the skips (else prefix_skip_kernel does)
    int32_t* skip;                // [num_seqs] read by the decode plan
};

// The members of group grp and the number of shared partitions the group's
// workgroups compute (0: none).  The skips and the states are both decided
// from this, so they match.
struct GroupShare {
    int s0, s1;       // members [s0, s1)
    bool members_ok;  // the range lies inside the batch
    int nparts;
};

template <int BS>
__device__ inline bool length_ok(const DecodeArgs& d, int T) {
    return T > 0 && T <= d.max_seq_len && (T + BS - 1) / BS <= d.max_blocks_per_seq;
}

template <int BS>
__device__ inline GroupShare group_share(const PrefixArgs& a, int grp) {
    const DecodeArgs& d = a.d;
    const int P = d.partition_size;
    GroupShare gs;
    gs.s0 = a.group_start[grp];
    gs.s1 = a.group_start[grp + 1];
    gs.members_ok = 0 <= gs.s0 && gs.s0 <= gs.s1 && gs.s1 <= d.num_seqs;
    gs.nparts = 0;
    if (gs.members_ok && gs.s1 > gs.s0) {
        const int pre = a.group_prefix[grp];
        const int T0 = d.seq_lens[gs.s0];
        gs.nparts = pre > 0 ? min(pre / P, a.parts) : 0;  // never more than the grid covers
        // the leader must hold them, and with new tokens have a partition of its own (as member_shares)
        if (!length_ok<BS>(d, T0) || T0 < gs.nparts * P || (d.new_k != nullptr && T0 == gs.nparts * P))
            gs.nparts = 0;
    }
    return gs;
}

// whether a member of length T shares the group's partitions.  When the call
// stores each sequence's newest token, a member must also have a partition of
// its own (T beyond the shared partitions): the workgroup that computes it is
// the one that stores the token.  A member whose newest token falls inside the
// shared partitions breaks the call's contract; it is then computed alone, so
// that its token is at least stored and its own row is consistent.
template <int BS>
__device__ inline bool member_shares(const PrefixArgs& a, const GroupShare& gs, int T) {
    const int shared = gs.nparts * a.d.partition_size;
    return gs.nparts > 0 && length_ok<BS>(a.d, T) && (a.d.new_k != nullptr ? T > shared : T >= shared);
}

// The skips of group grp's members, and of the sequences before the first
// group and after the last one, which no group covers (256 threads).
// Members past the grid's chunks are computed alone.
template <int BS>
__device__ inline void write_group_skips(const PrefixArgs& a, int grp, const GroupShare& gs) {
    const int n = a.d.num_seqs;
    if (gs.members_ok)
        for (int i = gs.s0 + (int)threadIdx.x; i < gs.s1; i += 256)
            a.skip[i] = (i - gs.s0 < a.member_cap && member_shares<BS>(a, gs, a.d.seq_lens[i])) ? gs.nparts : 0;
    if (grp == 0)
        for (int i = threadIdx.x; i < min(max(gs.s0, 0), n); i += 256) a.skip[i] = 0;
    if (grp == a.num_groups - 1)
        for (int i = max(gs.s1, 0) + (int)threadIdx.x; i < n; i += 256) a.skip[i] = 0;
}

// one workgroup per group
template <int BS>
__global__ void __launch_bounds__(256) prefix_skip_kernel(const PrefixArgs a) {
    const GroupShare gs = group_share<BS>(a, blockIdx.x);
    write_group_skips<BS>(a, blockIdx.x, gs);
}

// The work of workgroup bid of the shared partitions' grid.
template <Fmt KV, int D, int BS, int G>
__device__ __forceinline__ void prefix_states(const PrefixArgs& a, unsigned bid) {
    using Sh = MqShape<D, BS, G, 1, PA_PREFIX_STAGES>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const DecodeArgs& d = a.d;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int n = lane & 15;
    const int H = d.num_kv_heads;
    const int P = d.partition_size;

    int rest = (int)bid;
    const int kvh = rest % H;
    rest /= H;
    const int chunk = rest % a.chunks;
    rest /= a.chunks;
    const int part = rest % a.parts;
    const int grp = rest / a.parts;

    const GroupShare gs = group_share<BS>(a, grp);
    const int s0 = gs.s0, s1 = gs.s1, nparts = gs.nparts;
    if (a.write_skips && part == 0 && chunk == 0 && kvh == 0) write_group_skips<BS>(a, grp, gs);
    if (!gs.members_ok || part >= nparts) return;
    const int members = s1 - s0;
    const int mem_lo = chunk * Sh::TQ;
    if (mem_lo >= members) return;

    // this lane's column: member mem_lo + wave * (16 / G) + n / G, head n % G
    const int mi = mem_lo + wave * Sh::PER_WAVE + n / G;
    const int seq = s0 + (mi < members ? mi : 0);
    const int head = kvh * G + n % G;
    const int T = d.seq_lens[seq];
    MqTask<1> t;
    t.bt = d.block_tables + (size_t)s0 * d.max_blocks_per_seq;
    t.key_begin = part * P;
    t.key_end = (part + 1) * P;
    t.kv_len = t.key_end;
    t.kvh = kvh;
    t.cvalid[0] = mi < members && member_shares<BS>(a, gs, T);
    t.cpos[0] = t.key_end - 1;
    t.qptr[0] = (const char*)d.q + ((size_t)seq * d.num_heads + head) * D * 2;
    t.wave_cols = mem_lo + wave * Sh::PER_WAVE < members;
    t.wpos_min = t.key_end - 1;
    t.wpos_max = t.key_end - 1;

    float m1[1], l1[1];
    f32x4 acc1[1][2][4];
    bool bad;
    mq_tile<KV, D, BS, G, 1, PA_PREFIX_STAGES, true, true>(a.pool, t, smem, m1, l1, acc1, bad);
    const float m = m1[0], l = l1[0];
    const f32x4(&acc)[2][4] = acc1[0];

    if (!t.cvalid[0]) return;
    const size_t row = (size_t)seq * d.num_heads + head;
    const float nan = __builtin_nanf("");
    // dims 64 a + 16 b + 4 g + i: four consecutive dims (i = 0..3) per store
    if ((T + P - 1) / P == 1) {  // the sequence is this one shared partition: finish its row
        const float inv = bad ? nan : 1.f / l;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                store_out4(d.out, d.out_dtype, row * D + 64 * aa + 16 * b + 4 * g, acc[aa][b] * inv);
        return;
    }
    const size_t pidx = row * d.max_partitions + part;
    if (g == 0) {  // the column's m and l, in the call's layout
        float* pm = d.part_m + pidx;
        float* pl = d.part_l + pidx;
        if (d.ml_records) {
            pm = d.part_ml + ml_record(d, seq, kvh, part) + (head - kvh * G);
            pl = pm + ML_L;
        }
        __builtin_nontemporal_store(bad ? nan : m, pm);
        __builtin_nontemporal_store(bad ? nan : l, pl);
    }
    const float one = bad ? nan : 1.f;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            __builtin_nontemporal_store(acc[aa][b] * one, (f32x4*)&d.part_acc[pidx * D + 64 * aa + 16 * b + 4 * g]);
}

template <Fmt KV, int D, int BS, int G>
__global__ void __launch_bounds__(256, 2) prefix_states_kernel(const PrefixArgs a) {
    prefix_states<KV, D, BS, G>(a, blockIdx.x);
}

// The shared partitions (workgroups below prefix_grid) and the decode
// partitions of a 4-head-group batch in one launch.  The two kinds run
// concurrently and share no data: the first write the partition slots below
// each member's skip (or a one-partition member's output row) and read only
// blocks of the shared partitions; the others write the slots from the skip on
// and, with APPEND, store each sequence's newest token, which lies past its
// group's shared tokens and so in a block the first kind does not read.
template <Fmt KV, int BS, bool APPEND>
__global__ void __launch_bounds__(256, 2) shared_prefix_fused_kernel(const PrefixArgs a, unsigned prefix_grid) {
    if (blockIdx.x < prefix_grid)
        prefix_states<KV, 128, BS, 4>(a, blockIdx.x);
    else
        gqa4_partition<KV, 128, BS, 4, PA_GQA_STAGES, APPEND>(a.d, blockIdx.x - prefix_grid);
}
static_assert(PA_GQA_WAVES == 4, "the combined launch runs both kinds of workgroup with 256 threads");

// Grid sizes for groups of G heads: member chunks and shared partitions per
// group.  Returns the number of shared-partition workgroups, or -1 when it
// does not fit a grid.
template <int D, int BS, int G>
static long long size_prefix_grid(PrefixArgs& a, int max_group_size, int max_prefix_len) {
    using Sh = MqShape<D, BS, G, 1, PA_PREFIX_STAGES>;
    a.chunks = max((max_group_size + Sh::TQ - 1) / Sh::TQ, 1);
    a.parts = max(max_prefix_len / a.d.partition_size, 1);  // at least one: part 0 writes the skips
    a.member_cap = a.chunks * Sh::TQ;
    const long long grid = (long long)a.num_groups * a.chunks * a.parts * a.d.num_kv_heads;
    return grid > 0x7fffffffLL ? -1 : grid;
}

template <Fmt KV, int D, int BS, int G>
static int launch_prefix(PrefixArgs& a, int max_group_size, int max_prefix_len, hipStream_t stream) {
    using Sh = MqShape<D, BS, G, 1, PA_PREFIX_STAGES>;
    auto kernel = prefix_states_kernel<KV, D, BS, G>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const long long grid = size_prefix_grid<D, BS, G>(a, max_group_size, max_prefix_len);
    if (grid < 0) return PA_ERR_SHAPE;
    if (grid == 0) return PA_OK;
    a.write_skips = true;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), Sh::LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <Fmt KV, int BS>
static int dispatch_prefix_group(PrefixArgs& a, int group, int mgs, int mpl, hipStream_t s) {
    switch (group) {
        case 1: return launch_prefix<KV, 128, BS, 1>(a, mgs, mpl, s);
        case 2: return launch_prefix<KV, 128, BS, 2>(a, mgs, mpl, s);
        case 4: return launch_prefix<KV, 128, BS, 4>(a, mgs, mpl, s);
        case 8: return launch_prefix<KV, 128, BS, 8>(a, mgs, mpl, s);
    }
    return PA_ERR_UNSUPPORTED;
}

bool prefix_states_supported(int kv_dtype, int q_dtype, int head_dim, int block_size, int group) {
    return ((kv_dtype == PA_DTYPE_BF16 && q_dtype == PA_DTYPE_BF16) ||
            (kv_dtype == PA_DTYPE_F16 && q_dtype == PA_DTYPE_F16)) &&
           head_dim == 128 && (block_size == 16 || block_size == 32) &&
           (group == 1 || group == 2 || group == 4 || group == 8);
}

static PrefixArgs make_prefix_args(const DecodeArgs& d, const int32_t* group_start, const int32_t* group_prefix,
                                   int num_groups, int32_t* skip) {
    PrefixArgs a;
    a.d = d;
    a.pool.k_cache = d.k_cache;
    a.pool.v_cache = d.v_cache;
    a.pool.num_kv_heads = d.num_kv_heads;
    a.pool.num_blocks = d.num_blocks;
    a.pool.qk_scale_log2 = d.qk_scale_log2;
    a.group_start = group_start;
    a.group_prefix = group_prefix;
    a.num_groups = num_groups;
    a.write_skips = false;
    a.skip = skip;
    return a;
}

int launch_prefix_states(const DecodeArgs& d, int kv_dtype, int group, const int32_t* group_start,
                         const int32_t* group_prefix, int num_groups, int max_group_size, int max_prefix_len,
                         int32_t* skip, hipStream_t stream) {
    PrefixArgs a = make_prefix_args(d, group_start, group_prefix, num_groups, skip);
    if (kv_dtype == PA_DTYPE_BF16)
        return d.block_size == 16 ? dispatch_prefix_group<Fmt::BF16, 16>(a, group, max_group_size, max_prefix_len, stream)
                                  : dispatch_prefix_group<Fmt::BF16, 32>(a, group, max_group_size, max_prefix_len, stream);
    return d.block_size == 16 ? dispatch_prefix_group<Fmt::F16, 16>(a, group, max_group_size, max_prefix_len, stream)
                              : dispatch_prefix_group<Fmt::F16, 32>(a, group, max_group_size, max_prefix_len, stream);
}

#ifndef PA_DISABLE_GQA4
bool prefix_fused_supported(int kv_dtype, int q_dtype, int head_dim, int block_size, int group) {
    return prefix_states_supported(kv_dtype, q_dtype, head_dim, block_size, group) && group == 4;
}

template <int BS>
static int launch_skips_for(PrefixArgs& a, int max_group_size, int max_prefix_len, hipStream_t stream) {
    if (size_prefix_grid<128, BS, 4>(a, max_group_size, max_prefix_len) < 0) return PA_ERR_SHAPE;
    if (a.num_groups == 0) return PA_OK;
    hipLaunchKernelGGL(prefix_skip_kernel<BS>, dim3((unsigned)a.num_groups), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_prefix_skips(const DecodeArgs& d, const int32_t* group_start, const int32_t* group_prefix,
                        int num_groups, int max_group_size, int max_prefix_len, int32_t* skip, hipStream_t stream) {
    PrefixArgs a = make_prefix_args(d, group_start, group_prefix, num_groups, skip);
    return d.block_size == 16 ? launch_skips_for<16>(a, max_group_size, max_prefix_len, stream)
                              : launch_skips_for<32>(a, max_group_size, max_prefix_len, stream);
}

template <Fmt KV, int BS, bool APPEND>
static int launch_fused_as(PrefixArgs& a, int max_group_size, int max_prefix_len, hipStream_t stream) {
    using Sp = MqShape<128, BS, 4, 1, PA_PREFIX_STAGES>;
    using Sg = GqaShape<KV, 128, 16, 4, PA_GQA_STAGES>;
    constexpr int LDS_G = APPEND ? Sg::LDS_APPEND : Sg::LDS;
    constexpr int LDS = Sp::LDS > LDS_G ? Sp::LDS : LDS_G;
    auto kernel = shared_prefix_fused_kernel<KV, BS, APPEND>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const long long prefix_grid = size_prefix_grid<128, BS, 4>(a, max_group_size, max_prefix_len);
    if (prefix_grid < 0) return PA_ERR_SHAPE;
    const long long grid =
        (a.num_groups > 0 ? prefix_grid : 0) + (long long)a.d.num_seqs * a.d.max_partitions * a.d.num_kv_heads;
    if (grid > 0x7fffffffLL) return PA_ERR_SHAPE;
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), LDS, stream, a,
                       (unsigned)(a.num_groups > 0 ? prefix_grid : 0));
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <Fmt KV, int BS>
static int launch_fused_for(PrefixArgs& a, int mgs, int mpl, hipStream_t s) {
    return a.d.new_k != nullptr ? launch_fused_as<KV, BS, true>(a, mgs, mpl, s)
                                : launch_fused_as<KV, BS, false>(a, mgs, mpl, s);
}

int launch_prefix_fused(const DecodeArgs& d, int kv_dtype, const int32_t* group_start, const int32_t* group_prefix,
                        int num_groups, int max_group_size, int max_prefix_len, int32_t* skip, hipStream_t stream) {
    PrefixArgs a = make_prefix_args(d, group_start, group_prefix, num_groups, skip);
    if (kv_dtype == PA_DTYPE_BF16)
        return d.block_size == 16 ? launch_fused_for<Fmt::BF16, 16>(a, max_group_size, max_prefix_len, stream)
                                  : launch_fused_for<Fmt::BF16, 32>(a, max_group_size, max_prefix_len, stream);
    return d.block_size == 16 ? launch_fused_for<Fmt::F16, 16>(a, max_group_size, max_prefix_len, stream)
                              : launch_fused_for<Fmt::F16, 32>(a, max_group_size, max_prefix_len, stream);
}
#else
bool prefix_fused_supported(int, int, int, int, int) { return false; }
int launch_prefix_skips(const DecodeArgs&, const int32_t*, const int32_t*, int, int, int, int32_t*, hipStream_t) {
    return PA_ERR_UNSUPPORTED;
}
int launch_prefix_fused(const DecodeArgs&, int, const int32_t*, const int32_t*, int, int, int, int32_t*, hipStream_t) {
    return PA_ERR_UNSUPPORTED;
}
#endif

}  // namespace pa
