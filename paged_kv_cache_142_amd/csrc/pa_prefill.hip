// Multi-query (prefill / chunked prefill) attention over paged K/V on the
// gfx950 matrix cores: pa_prefill.
//
// Sequence i has T = seq_lens[i] cached tokens; its Q = query_start[i+1] -
// query_start[i] packed query rows are its last Q tokens (row j at position
// T - Q + j) and each attends to the cached tokens 0 .. its position.
//
// Work decomposition: one workgroup per (query tile, kv head).  A tile holds
// TQ = 128 / G query tokens of one sequence, i.e. 128 (token, query head)
// columns for the G query heads of the kv head; each of the four waves owns
// 32 of them (two column blocks of 16).  The workgroup runs the multi-query
// tile of pa_mq_mfma.hpp over the keys 0 .. (its last position); column
// (token at position p) sees keys 0 .. p.  The K/V copies keep the cache
// hint: every tile of a sequence reads its keys again.
//
// The grid holds only real tiles (at most total_q / TQ + num_seqs of them):
// each workgroup finds its tile from the query counts, in the order "highest
// tile index first" (tile j of a full prefill sees (j + 1) TQ keys, so this is
// longest-first), sequences in index order within an index.  Launching a
// grid sized for max_query_len instead leaves most workgroups of the early
// (high) tile indices empty, and those hold dispatch slots while the long
// tiles wait.
//
// The weights enter the value products as single 16-bit values, normalised
// by the sum of those rounded weights (the tile's single form): error at most
// 2^-9 (bf16) or 2^-12 (f16) of the spread of the values a row averages,
// against 16 significant bits and a second product per value block in the
// split form (PA_PREFILL_SPLIT=true builds that form instead).
//
// A block id outside the pool makes the tile's output rows NaN (the tile
// never uses it as an address); so does an invalid sequence length.
#include "pa_mq_mfma.hpp"

#ifndef PA_PREFILL_CB
#define PA_PREFILL_CB 2
#endif
#ifndef PA_PREFILL_STREAM
#define PA_PREFILL_STREAM false
#endif
#ifndef PA_PREFILL_SPLIT
#define PA_PREFILL_SPLIT false
#endif

namespace pa {

constexpr int PREFILL_CB = PA_PREFILL_CB;

struct PrefillArgs {
    void* out;
    int out_dtype;
    const void* q;
    const int32_t* query_start;
    int total_q;
    MqPool pool;
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* seq_lens;
    int max_seq_len;
    int num_seqs;
    int num_heads;
    int tiles;  // upper bound of the query tiles of one sequence
};

// A sequence's query range and length, as one lane loads them.
struct PrefillSeq {
    int q0, q1, T;
};

// Tiles of the sequence whose range `r` holds (0 for rows that cannot be
// addressed).
template <int TQ>
__device__ __forceinline__ int prefill_tiles(const PrefillArgs& a, const PrefillSeq& r) {
    if (r.q0 < 0 || r.q1 < r.q0 || r.q1 > a.total_q) return 0;
    return (r.q1 - r.q0 + TQ - 1) / TQ;
}

__device__ __forceinline__ PrefillSeq prefill_seq(const PrefillArgs& a, int i) {
    if (i >= a.num_seqs) return PrefillSeq{0, 0, 0};
    return PrefillSeq{a.query_start[i], a.query_start[i + 1], a.seq_lens[i]};
}

// The p-th tile of the order "highest tile index first, then sequence
// index", computed by one wavefront (sequences spread over the lanes in
// chunks of 64).  With c(j) = sum_i max(tiles_i - j, 0), the items of tile
// index j are c(j+1) .. c(j) - 1: a binary search on j, then the r-th
// sequence (in index order) that has more than j tiles.  The sequence's
// query range and length come back with it (loaded with the counts).
template <int TQ>
__device__ bool prefill_item(const PrefillArgs& a, int p, int& seq, int& tile, PrefillSeq& sr) {
    const int lane = threadIdx.x & 63;
    const PrefillSeq r0 = prefill_seq(a, lane);  // the first chunk stays in registers
    const int t0 = prefill_tiles<TQ>(a, r0);
    auto count_from = [&](int j) {  // c(j), uniform
        int x = max(t0 - j, 0);
        for (int c = 64; c < a.num_seqs; c += 64) x += max(prefill_tiles<TQ>(a, prefill_seq(a, c + lane)) - j, 0);
        return __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63);
    };
    if (p >= count_from(0)) return false;
    int lo = 0, hi = a.tiles;  // c(lo) > p >= c(hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (count_from(mid) > p)
            lo = mid;
        else
            hi = mid;
    }
    int r = p - count_from(lo + 1);
    for (int c = 0; c < a.num_seqs; c += 64) {
        const PrefillSeq rc = c == 0 ? r0 : prefill_seq(a, c + lane);
        const bool has = prefill_tiles<TQ>(a, rc) > lo;
        const uint64_t m = __builtin_amdgcn_ballot_w64(has);
        const int cnt = __builtin_popcountll(m);
        if (r < cnt) {
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const uint64_t hit = __builtin_amdgcn_ballot_w64(has && below == r);
            if (hit == 0) return false;  // cannot happen for r < cnt
            const int l = __builtin_ctzll(hit);
            seq = c + l;
            tile = lo;
            sr.q0 = __builtin_amdgcn_readlane(rc.q0, l);
            sr.q1 = __builtin_amdgcn_readlane(rc.q1, l);
            sr.T = __builtin_amdgcn_readlane(rc.T, l);
            return true;
        }
        r -= cnt;
    }
    return false;
}

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 4
#endif
template <Fmt KV, int D, int BS, int G>
__global__ void __launch_bounds__(PA_PREFILL_WAVES * 64, 8 / PA_PREFILL_WAVES) prefill_mfma_kernel(const PrefillArgs a) {
    using Sh = MqShape<D, BS, G, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int n = lane & 15;

    // ---- (sequence, tile, kv head) of this workgroup
    const int H = a.pool.num_kv_heads;
    const int kvh = (int)(blockIdx.x % H);
    int seq, tile;
    PrefillSeq sr;
    if (!prefill_item<Sh::TQ>(a, (int)(blockIdx.x / H), seq, tile, sr)) return;
    const int q0 = sr.q0, q1 = sr.q1, T = sr.T;  // the range can be addressed: the sequence has tiles
    const int Q = q1 - q0;
    const int tok_lo = tile * Sh::TQ;
    if (tok_lo >= Q) return;
    const int tok_hi = min(tok_lo + Sh::TQ, Q);
    const bool bad_seq = T <= 0 || T > a.max_seq_len || Q > T ||
                         (T + BS - 1) / BS > a.max_blocks_per_seq;
    if (bad_seq) {  // NaN rows for this tile
        for (int o = threadIdx.x; o < (tok_hi - tok_lo) * G * D; o += Sh::W * 64) {
            const int tk = o / (G * D);
            const int rr = o - tk * G * D;
            const size_t row = (size_t)(q0 + tok_lo + tk) * a.num_heads + kvh * G + rr / D;
            store_out(a.out, a.out_dtype, row * D + rr % D, __builtin_nanf(""));
        }
        return;
    }

    // this lane's column in block cb: token tok_lo + wave * PER_WAVE +
    // (16 cb + n) / G, head n % G
    MqTask<PREFILL_CB> t;
    const int chead = kvh * G + n % G;
    int ctok[PREFILL_CB];
    t.bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    t.key_begin = 0;
    t.key_end = T - Q + tok_hi;  // one past the last position of the tile
    t.kv_len = T;
    t.kvh = kvh;
#pragma unroll
    for (int cb = 0; cb < PREFILL_CB; ++cb) {
        ctok[cb] = tok_lo + wave * Sh::PER_WAVE + (16 * cb + n) / G;
        t.cvalid[cb] = ctok[cb] < tok_hi;
        t.cpos[cb] = T - Q + ctok[cb];
        t.qptr[cb] = (const char*)a.q +
                     ((size_t)(q0 + (t.cvalid[cb] ? ctok[cb] : tok_lo)) * a.num_heads + chead) * D * 2;
    }
    const int wtok_lo = tok_lo + wave * Sh::PER_WAVE;
    const int wtok_hi = min(wtok_lo + Sh::PER_WAVE, tok_hi);
    t.wave_cols = wtok_lo < tok_hi;
    t.wpos_min = T - Q + wtok_lo;
    t.wpos_max = T - Q + wtok_hi - 1;

    float m[PREFILL_CB], l[PREFILL_CB];
    f32x4 acc[PREFILL_CB][2][4];
    bool bad;
    mq_tile<KV, D, BS, G, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_STREAM, PA_PREFILL_SPLIT, PA_PREFILL_WAVES>(a.pool, t, smem, m,
                                                                                                    l, acc, bad);

    // ---- output: column n of each block, dims 64 a + 16 b + 4 g + i, four
    // consecutive dims (i = 0..3) per store
#pragma unroll
    for (int cb = 0; cb < PREFILL_CB; ++cb) {
        if (!t.cvalid[cb]) continue;
        const float inv = bad ? __builtin_nanf("") : 1.f / l[cb];
        const size_t base = ((size_t)(q0 + ctok[cb]) * a.num_heads + chead) * D;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                store_out4(a.out, a.out_dtype, base + 64 * aa + 16 * b + 4 * g, acc[cb][aa][b] * inv);
    }
}

template <Fmt KV, int D, int BS, int G>
static int launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    using Sh = MqShape<D, BS, G, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>;
    auto kernel = prefill_mfma_kernel<KV, D, BS, G>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    // every real tile: at most total_q / TQ + num_seqs of them
    const size_t items = (size_t)(a.total_q + Sh::TQ - 1) / Sh::TQ + (size_t)a.num_seqs;
    const size_t grid = items * a.pool.num_kv_heads;
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(Sh::W * 64), Sh::LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <Fmt KV, int D, int BS>
static int dispatch_prefill_group(PrefillArgs& a, int group, int max_query_len, hipStream_t stream) {
    auto tiles = [&](int tq) { return (max_query_len + tq - 1) / tq; };
    switch (group) {
        case 1: a.tiles = tiles(MqShape<D, BS, 1, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>::TQ); return launch_prefill<KV, D, BS, 1>(a, stream);
        case 2: a.tiles = tiles(MqShape<D, BS, 2, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>::TQ); return launch_prefill<KV, D, BS, 2>(a, stream);
        case 4: a.tiles = tiles(MqShape<D, BS, 4, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>::TQ); return launch_prefill<KV, D, BS, 4>(a, stream);
        case 8: a.tiles = tiles(MqShape<D, BS, 8, PREFILL_CB, PA_MQ_STAGES, PA_PREFILL_WAVES>::TQ); return launch_prefill<KV, D, BS, 8>(a, stream);
    }
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa

extern "C" int pa_prefill(void* out, int out_dtype, const void* q, int q_dtype, const int32_t* query_start,
                          int total_q, int max_query_len, const void* k_cache, const void* v_cache, int kv_dtype,
                          const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                          int max_seq_len, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, float scale, void* stream) {
    using namespace pa;
    const bool combo_ok = (kv_dtype == PA_DTYPE_BF16 && q_dtype == PA_DTYPE_BF16) ||
                          (kv_dtype == PA_DTYPE_F16 && q_dtype == PA_DTYPE_F16);
    if (kv_dtype < PA_DTYPE_F32 || kv_dtype > PA_DTYPE_FP8_E4M3 || q_dtype < PA_DTYPE_F32 ||
        q_dtype > PA_DTYPE_FP8_E4M3)
        return PA_ERR_DTYPE;
    if (out_dtype != PA_DTYPE_F32 && out_dtype != PA_DTYPE_F16 && out_dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
    if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        max_seq_len < 0 || max_blocks_per_seq < 0 || num_blocks <= 0 || head_dim <= 0 || block_size <= 0)
        return PA_ERR_SHAPE;
    if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
    if (max_query_len > max_seq_len) return PA_ERR_SHAPE;
    if ((long long)max_blocks_per_seq * block_size < (long long)max_seq_len) return PA_ERR_SHAPE;
    if (!combo_ok) return PA_ERR_UNSUPPORTED;
    const int group = num_heads / num_kv_heads;
    if (head_dim != 128 || (block_size != 16 && block_size != 32) ||
        (group != 1 && group != 2 && group != 4 && group != 8))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || total_q == 0 || max_query_len == 0) return PA_OK;
    if (!out || !q || !query_start || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
    if ((((uintptr_t)out) | ((uintptr_t)q) | ((uintptr_t)k_cache) | ((uintptr_t)v_cache)) & 15u) return PA_ERR_SHAPE;
    const long long items_max = (total_q + 7) / 8 + (long long)num_seqs;  // the smallest tile is 8 tokens
    if (items_max * num_kv_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
#if PA_CHECK_CONTENTS
    {
        std::vector<int32_t> lens, tables;
        int checked = check::sequences(seq_lens, block_tables, num_seqs, max_blocks_per_seq, max_seq_len, block_size,
                                       num_blocks, lens, tables, (hipStream_t)stream);
        if (checked == PA_OK)
            checked = check::queries(query_start, num_seqs, total_q, max_query_len, lens, (hipStream_t)stream);
        if (checked != PA_OK) return checked;
    }
#endif
    PrefillArgs a;
    a.out = out;
    a.out_dtype = out_dtype;
    a.q = q;
    a.query_start = query_start;
    a.total_q = total_q;
    a.pool.k_cache = k_cache;
    a.pool.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.max_seq_len = max_seq_len;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.pool.num_kv_heads = num_kv_heads;
    a.pool.num_blocks = num_blocks;
    a.pool.qk_scale_log2 = scale * kLog2e;
    a.tiles = 0;
    const hipStream_t s = (hipStream_t)stream;
    if (kv_dtype == PA_DTYPE_BF16)
        return block_size == 16 ? dispatch_prefill_group<Fmt::BF16, 128, 16>(a, group, max_query_len, s)
                                : dispatch_prefill_group<Fmt::BF16, 128, 32>(a, group, max_query_len, s);
    return block_size == 16 ? dispatch_prefill_group<Fmt::F16, 128, 16>(a, group, max_query_len, s)
                            : dispatch_prefill_group<Fmt::F16, 128, 32>(a, group, max_query_len, s);
}
