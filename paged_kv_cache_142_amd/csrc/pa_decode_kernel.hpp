// Split-KV paged decode attention for gfx950: the partition kernel.
//
// One workgroup per (sequence, kv head, KV partition); W wavefronts per
// workgroup.  Wave w walks logical blocks w, w+W, w+2W, ... of the
// partition.  For each block it copies the (block, kv head) K tile and V
// tile (block_size x head_dim elements each, contiguous in the pool) from
// global memory straight into its own S-stage LDS ring with 16-byte
// asynchronous copies (global_load_lds_dwordx4), S-1 blocks ahead of the
// block it computes on, so several KiB per wave stay in flight without
// holding registers.  The physical block id is read once per block, with a
// scalar load, when the block's copy is issued.
//
// Register layout of the compute: lane l handles token row r = l / LPR of
// every group of R = 64/LPR rows and the 8 elements of "column" c = l % LPR
// of that row (LPR = head_dim / 8).  Each K row is therefore spread over
// LPR consecutive lanes of one DPP row, so a q.k dot product is a per-lane
// partial (dot2 instructions for 16-bit data) followed by a 3- or 4-step DPP
// butterfly that leaves the full score in every lane of the group.  The V
// row sits in the same lanes, so the score a lane holds is exactly the
// weight it needs for its V elements: no score exchange is required.  All
// G query heads of the kv head are computed from the same LDS tile (the
// tile is loaded once per workgroup and shared across the GQA group).
//
// Every lane keeps an online-softmax state (m, l, acc[8]) per query head
// for its row subset, updated per 16-token chunk with the recurrence
//     m' = max(m, max_j s_j); alpha = 2^(m - m'); l' = alpha l + sum_j 2^(s_j - m');
//     acc' = alpha acc + sum_j 2^(s_j - m') v_j
// (scores are pre-multiplied by log2 e, so base-2 exponentials give the
// natural-base softmax).  At the end the row subsets of a wave are merged
// with cross-lane shuffles and the waves of the workgroup through LDS, using
// the same rule; the merged (m, l, acc) goes to the workspace, or, when the
// sequence has a single partition, acc / l goes straight to the output.
#pragma once

#include <type_traits>

#include "pa_common.hpp"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
    void* out;
    int out_dtype;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* seq_lens;
    int max_seq_len;
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int block_size;
    int num_blocks;
    float qk_scale_log2;  // scale * log2(e)
    const float* k_scale;
    const float* v_scale;
    int partition_size;
    int max_partitions;
    // m and l of the partition states, in one of two layouts over the same
    // workspace area, chosen per call (every kernel of a call uses its layout):
    // ml_records = 1: records of ML_REC floats, one per (sequence, kv head,
    // partition), [num_seqs][num_kv_heads][max_partitions] at part_ml;
    // ml_records = 0: part_m and part_l, [num_seqs][num_heads][max_partitions]
    // each (the GQA-4 kernel, whose few states read faster this way).
    int ml_records;
    float* part_ml;
    float* part_m;
    float* part_l;
    float* part_acc;  // [num_seqs][num_heads][max_partitions][head_dim]
    // Work order written by the plan kernel: plan[0] = number of (sequence,
    // partition) items, plan[PLAN_ITEMS_OFFSET + k] = seq * max_partitions +
    // partition of the k-th item, largest first.
    int* plan;
    // 1: no plan kernel ran; every partition workgroup derives its item from
    // seq_lens itself (at most 64 sequences and 64 blocks per partition).
    int inline_plan;
    // Leading partitions of each sequence computed elsewhere (the shared
    // prefix of its group, by the prefix kernel); nullptr: none.  Those
    // partitions have no items here; their states are in the workspace.
    const int32_t* skip_parts;
    // Decode with append: the K and V rows [num_seqs][num_kv_heads][head_dim]
    // of each sequence's newest token (position seq_lens - 1), stored into
    // its slot by the workgroup that owns the sequence's last partition;
    // nullptr: the tokens are already in the pool.
    const void* new_k;
    const void* new_v;
    // Copy-on-write copies run in the same launch as decode with append (the
    // GQA-4 kernel): cow_pairs[2 i] -> cow_pairs[2 i + 1] (source, destination
    // block), cow_num pairs (at most COW_MAX_PAIRS); 0: none.  The launch's
    // last 2 cow_num workgroups copy them, and partition workgroups read a
    // destination block from its source (the same content once copied).
    const int64_t* cow_pairs;
    int cow_num;
};

// Pairs that one launch takes (one per lane of the partition workgroups'
// check); more go through a launch of their own.  The copying workgroups run
// in the launch's tail: with 16 pairs the step was 1.5 us faster than with
// the separate copy launch, with 40 pairs 2.8 us slower.
constexpr int COW_MAX_PAIRS = 16;

constexpr int PLAN_ITEMS_OFFSET = 64;

// Partition-state record of m and l: m of head g of the kv head's group at
// [g], l at [ML_L + g], the rest zero; 64 bytes on a 64-byte boundary.
// Kernels that compute a whole group write it with one 16-lane store, so that
// it reaches memory whole: scattered 4-byte stores of m and l, partial writes
// among the K/V reads, cost the long-context FP8 partition launch 4.3% (a
// timing-only variant without them); 64- and 128-byte records measured the
// same.
constexpr int ML_REC = 16;
constexpr int ML_L = 8;

// Whether a call's partition kernel is the GQA-4 one (groups of four query
// heads over 16-bit K/V; the per-format dispatch makes the same choice).  Its
// calls keep m and l in per-row arrays (ml_records = 0): on the gqa workload
// the reduce read the records 0.6 us slower than the arrays, while the
// kernel itself gained nothing from them.  Every other partition kernel
// writes records.
inline bool partition_kernel_is_gqa4(int kv_dtype, int group) {
#ifdef PA_DISABLE_GQA4
    (void)kv_dtype;
    (void)group;
    return false;
#else
    return group == 4 && (kv_dtype == PA_DTYPE_BF16 || kv_dtype == PA_DTYPE_F16);
#endif
}
__device__ __forceinline__ size_t ml_record(const DecodeArgs& a, int seq, int kvh, int part) {
    return (((size_t)seq * a.num_kv_heads + kvh) * a.max_partitions + part) * ML_REC;
}

// Lanes 0..ML_REC-1 of one wave store a record: lane j's value is m of head j (j <
// G), l of head j - ML_L (ML_L <= j < ML_L + G), zero otherwise; NaN in place
// of m and l when bad.  m_of(g) and l_of(g) give head g's values; each lane
// evaluates only the one its element needs (g differs between lanes).  Every
// lane of the wave may call it; only lanes below ML_REC store.
template <int G, bool STREAM, typename MOf, typename LOf>
__device__ __forceinline__ void store_ml_record(float* rec, int lane, bool bad, MOf m_of, LOf l_of) {
    static_assert(G <= ML_L, "a record holds at most ML_L heads");
    const bool is_l = lane >= ML_L;
    const int g = is_l ? lane - ML_L : lane;
    float v = 0.f;
    if (g < G) v = bad ? __builtin_nanf("") : (is_l ? l_of(g) : m_of(g));
    if (lane < ML_REC) {
        if constexpr (STREAM)
            __builtin_nontemporal_store(v, rec + lane);
        else
            rec[lane] = v;
    }
}
constexpr int INLINE_PLAN_MAX_SEQS = 64;
constexpr int INLINE_PLAN_MAX_BLOCKS = 64;

// Inclusive prefix sum over the 64 lanes of a wavefront (DPP row shifts
// within rows of 16 lanes, then row broadcasts across rows).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 into rows 2, 3
    return x;
}

// The k-th (sequence, partition) item of the largest-first order, computed
// by one wavefront from the sequence lengths (one sequence per lane):
// first every partition of full size PB = partition_size / block_size, in
// (sequence, partition) order; then the partial last partitions, by size in
// blocks from PB - 1 down to 1, sequences in index order within a size.
// Sequences that are empty or invalid have no items.  Returns false when k
// is past the last item.  The partial partitions are ranked by a radix
// select on the key (PB - size) * 64 + sequence, one ballot per key bit.
__device__ __forceinline__ bool inline_plan_item(const DecodeArgs& a, int k, int& seq, int& part) {
    const int lane = threadIdx.x & 63;
    const int B = a.block_size;
    const int P = a.partition_size;
    const int PB = P / B;
    const int T = lane < a.num_seqs ? a.seq_lens[lane] : 0;
    const int skip = (a.skip_parts && lane < a.num_seqs) ? a.skip_parts[lane] : 0;
    const bool ok = T > 0 && T <= a.max_seq_len && (T + B - 1) / B <= a.max_blocks_per_seq;
    const int np = ok ? (T + P - 1) / P : 0;
    const int rem = ok ? (T + B - 1) / B - (np - 1) * PB : 0;  // blocks of the last partition
    // full partitions from `skip` on (the skipped ones are full); the last
    // partition is a partial item unless it is skipped too
    const int sk = ok ? min(max(skip, 0), np) : 0;
    const int nfull = ok ? max(np - (rem < PB ? 1 : 0) - sk, 0) : 0;
    const bool has_partial = ok && rem < PB && sk < np;
    const int incl = wave_inclusive_sum(nfull);
    const int F = __builtin_amdgcn_readlane(incl, 63);
    uint64_t cand = __builtin_amdgcn_ballot_w64(has_partial);  // sequences with a partial partition item
    if (k >= F + __builtin_popcountll(cand)) return false;
    if (k < F) {
        const uint64_t past = __builtin_amdgcn_ballot_w64(incl > k);
        if (past == 0) return false;  // cannot happen for k < F; keeps every index in range regardless
        const int s = __builtin_ctzll(past);
        seq = s;
        part = __builtin_amdgcn_readlane(sk, s) + k - (__builtin_amdgcn_readlane(incl, s) -
                                                        __builtin_amdgcn_readlane(nfull, s));
        return s < a.num_seqs && part >= 0 && part < __builtin_amdgcn_readlane(np, s);
    }
    k -= F;
    const int key = ((PB - rem) << 6) | lane;  // PB <= 64: 12 bits
#pragma unroll
    for (int b = 11; b >= 0; --b) {
        const uint64_t zero = cand & __builtin_amdgcn_ballot_w64(((key >> b) & 1) == 0);
        const int c = __builtin_popcountll(zero);
        if (k < c) {
            cand = zero;
        } else {
            k -= c;
            cand &= ~zero;
        }
    }
    if (cand == 0) return false;  // cannot happen for k < popcount; as above
    seq = __builtin_ctzll(cand);
    part = __builtin_amdgcn_readlane(np, seq) - 1;
    return seq < a.num_seqs && part >= 0;
}

// The (sequence, kv head, partition) of partition workgroup bid (normally
// the block index): bid = item * num_kv_heads + kv head, items in the plan's
// order.  Returns false for workgroups past the last item.
__device__ __forceinline__ bool partition_work_item(const DecodeArgs& a, unsigned bid, int& seq, int& kvh,
                                                    int& part) {
    const int item = bid / a.num_kv_heads;
    kvh = bid - item * a.num_kv_heads;
    if (a.inline_plan) return inline_plan_item(a, item, seq, part);
    if (item >= load_uniform(a.plan)) return false;
    const int code = load_uniform(a.plan + PLAN_ITEMS_OFFSET + item);
    seq = code / a.max_partitions;
    part = code - seq * a.max_partitions;
    return true;
}

__device__ __forceinline__ bool partition_work_item(const DecodeArgs& a, int& seq, int& kvh, int& part) {
    return partition_work_item(a, blockIdx.x, seq, kvh, part);
}

__device__ __forceinline__ void store_out(void* out, int dtype, size_t idx, float v) {
    if (dtype == PA_DTYPE_F32)
        ((float*)out)[idx] = v;
    else if (dtype == PA_DTYPE_BF16)
        ((uint16_t*)out)[idx] = f32_to_bf16_bits(v);
    else
        ((_Float16*)out)[idx] = (_Float16)v;
}

// Position of element d of a row of the waves' merge area in LDS: in every
// odd stretch of 32 elements the 16-byte granules swap in pairs.  A lane
// holds 8 consecutive elements of a row (granules 2c and 2c + 1) and writes
// them with two 16-byte stores.  A 16-byte store goes to LDS eight lanes at a
// time over 128 bytes of banks, so unswapped the lanes c and c + 4 of each
// eight would hit the same banks.  Rows read by consecutive threads still
// cover each bank once.
__device__ __forceinline__ int merge_pos(int d) { return d ^ (((d >> 5) & 1) << 2); }

// Placement of a lane's 8 elements inside one token row of format KV.
template <Fmt KV, int D>
struct LaneRow {
    static constexpr int EB = FmtBytes<KV>::value;
    static constexpr int LPR = D / 8;
    static constexpr int NW = 2 * EB;  // 32-bit words that hold 8 elements

    // 4-byte elements take two 16-byte pieces (c and c + LPR) so that each
    // load instruction of the wave covers consecutive 16-byte granules.
    __device__ static __forceinline__ int dim(int c, int e) {
        if constexpr (EB == 4)
            return e < 4 ? c * 4 + e : (c + LPR) * 4 + (e - 4);
        else
            return c * 8 + e;
    }

    __device__ static __forceinline__ void load(const char* row, int c, uint32_t (&w)[NW]) {
        if constexpr (EB == 4) {
            const u32x4 a = *(const u32x4*)(row + c * 16);
            const u32x4 b = *(const u32x4*)(row + (c + LPR) * 16);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else if constexpr (EB == 2) {
            const u32x4 a = *(const u32x4*)(row + c * 16);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        } else {
            const u32x2 a = *(const u32x2*)(row + c * 8);
            w[0] = a.x; w[1] = a.y;
        }
    }

    // The 8 elements as float32 (unscaled FP8 codes for FP8).
    __device__ static __forceinline__ void to_f32(const uint32_t (&w)[NW], float (&v)[8]) {
        if constexpr (KV == Fmt::F32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(w[e]);
        } else if constexpr (KV == Fmt::BF16) {
#pragma unroll
            for (int p = 0; p < 4; ++p) { v[2 * p] = bf16_lo(w[p]); v[2 * p + 1] = bf16_hi(w[p]); }
        } else if constexpr (KV == Fmt::F16) {
#pragma unroll
            for (int p = 0; p < 4; ++p) { v[2 * p] = f16_lo(w[p]); v[2 * p + 1] = f16_hi(w[p]); }
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[p], false);
                const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[p], true);
                v[4 * p] = a.x; v[4 * p + 1] = a.y; v[4 * p + 2] = b.x; v[4 * p + 3] = b.y;
            }
        }
    }
};

// Query operand of one head (lane's 8 elements) and the q.k partial product.
template <Fmt KV, Fmt Q>
struct QK;

template <>
struct QK<Fmt::F32, Fmt::F32> {
    struct Op {
        float x[8];
        __device__ __forceinline__ void pin() {
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(x[e]));
        }
    };
    using KOp = Op;
    template <int D>
    __device__ static __forceinline__ Op load_q(const char* qrow, int c) {
        constexpr int LPR = D / 8;
        const float4 a = *(const float4*)(qrow + c * 16);
        const float4 b = *(const float4*)(qrow + (c + LPR) * 16);
        return Op{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
    }
    __device__ static __forceinline__ KOp prep_k(const uint32_t (&w)[8]) {
        KOp k;
#pragma unroll
        for (int e = 0; e < 8; ++e) k.x[e] = __uint_as_float(w[e]);
        return k;
    }
    __device__ static __forceinline__ float dot(const Op& q, const KOp& k) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q.x[e], k.x[e], s);
        return s;
    }
};

struct Packed16Op {
    uint32_t w[4];
    __device__ __forceinline__ void pin() {
#pragma unroll
        for (int p = 0; p < 4; ++p) asm volatile("" : "+v"(w[p]));
    }
};

template <>
struct QK<Fmt::BF16, Fmt::BF16> {
    using Op = Packed16Op;
    using KOp = Packed16Op;
    template <int D>
    __device__ static __forceinline__ Op load_q(const char* qrow, int c) {
        const u32x4 a = *(const u32x4*)(qrow + c * 16);
        return Op{{a.x, a.y, a.z, a.w}};
    }
    __device__ static __forceinline__ KOp prep_k(const uint32_t (&w)[4]) { return KOp{{w[0], w[1], w[2], w[3]}}; }
    __device__ static __forceinline__ float dot(const Op& q, const KOp& k) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w[p]),
                                                __builtin_bit_cast(bf16x2, k.w[p]), s, false);
        return s;
    }
};

template <>
struct QK<Fmt::F16, Fmt::F16> {
    using Op = Packed16Op;
    using KOp = Packed16Op;
    template <int D>
    __device__ static __forceinline__ Op load_q(const char* qrow, int c) {
        const u32x4 a = *(const u32x4*)(qrow + c * 16);
        return Op{{a.x, a.y, a.z, a.w}};
    }
    __device__ static __forceinline__ KOp prep_k(const uint32_t (&w)[4]) { return KOp{{w[0], w[1], w[2], w[3]}}; }
    __device__ static __forceinline__ float dot(const Op& q, const KOp& k) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q.w[p]), __builtin_bit_cast(f16x2, k.w[p]), s,
                                       false);
        return s;
    }
};

// FP8 keys are widened to bfloat16 pairs (exact: every E4M3 value is a
// bfloat16 value) once per row and shared by all G heads.
template <>
struct QK<Fmt::FP8, Fmt::BF16> {
    using Op = Packed16Op;
    using KOp = Packed16Op;
    template <int D>
    __device__ static __forceinline__ Op load_q(const char* qrow, int c) {
        const u32x4 a = *(const u32x4*)(qrow + c * 16);
        return Op{{a.x, a.y, a.z, a.w}};
    }
    __device__ static __forceinline__ KOp prep_k(const uint32_t (&w)[2]) {
        KOp k;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            k.w[2 * p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[p], 1.0f, false));
            k.w[2 * p + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[p], 1.0f, true));
        }
        return k;
    }
    __device__ static __forceinline__ float dot(const Op& q, const KOp& k) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w[p]),
                                                __builtin_bit_cast(bf16x2, k.w[p]), s, false);
        return s;
    }
};

template <Fmt KV, int D, int BS, int G, int W, int S>
struct PartitionShape {
    static constexpr int EB = FmtBytes<KV>::value;
    static constexpr int LPR = D / 8;
    static constexpr int R = 64 / LPR;
    static constexpr int ROWB = D * EB;
    static constexpr int TILE = BS * ROWB;
    static constexpr int DMA_PER_TILE = TILE / 1024;
    static constexpr int DMA_PER_BLOCK = 2 * DMA_PER_TILE;
    static constexpr int STAGE = 2 * TILE;
    static constexpr int RING = S * STAGE;  // per wave
    static constexpr int PASSES = 16 / R;   // row groups per 16-token chunk
    static constexpr int CHUNKS = BS / 16;
    // cross-wave merge area: m[W][G], l[W][G], invalid[W] (padded), acc[W][G][D]
    static constexpr int MERGE_HEAD = ((2 * W * G + W) * 4 + 15) / 16 * 16;
    static constexpr int MERGE = W > 1 ? MERGE_HEAD + W * G * D * 4 : 0;
    static constexpr int LDS = (W * RING > MERGE) ? W * RING : MERGE;
    static_assert(TILE % 1024 == 0, "a tile must be a whole number of 1 KiB wave copies");
    static_assert((S - 1) * DMA_PER_BLOCK <= 63, "vmcnt can count at most 63 copies");
    static_assert(LDS <= 160 * 1024, "LDS budget of one CU");
    static_assert(ROWB % 16 == 0 && ROWB / 16 <= 64, "a row is copied as 16-byte granules, one per lane");
};

// Copy-on-write pairs in a decode launch: lane j < cow_num holds pair j
// (source, destination).  load_cow_pair reads the lane's pair as given, as
// four 32-bit words (the two little-endian int64 ids); cow_pair_ids checks it
// once it has arrived, so that the caller can make the read resident together
// with its other early reads (pin_cow_pair) instead of waiting for it on its
// own.  Lanes past the pairs read the last one and are marked unused by the
// check.  The read takes no branch (a branch would make the compiler wait for
// it at once): a launch without pairs reads 16 bytes of the new keys instead,
// which every decode-with-append launch has, and the check marks all lanes
// unused.
struct CowPair {
    u32x4 w;
};
__device__ __forceinline__ CowPair load_cow_pair(const DecodeArgs& a, int lane) {
    static_assert(COW_MAX_PAIRS <= 64, "one pair per lane");
    const int64_t* p = a.cow_num > 0 ? a.cow_pairs + 2 * min(lane, a.cow_num - 1) : (const int64_t*)a.new_k;
    const uint64_t s = (uint64_t)p[0], d = (uint64_t)p[1];
    return {{(uint32_t)s, (uint32_t)(s >> 32), (uint32_t)d, (uint32_t)(d >> 32)}};
}
__device__ __forceinline__ void pin_cow_pair(CowPair& p) {
    asm volatile("" : "+v"(p.w[0]), "+v"(p.w[1]), "+v"(p.w[2]), "+v"(p.w[3]));
}
// The pair's block ids; -1 for lanes past the pairs and for pairs outside
// the pool, which are skipped as by pa_copy_blocks.
__device__ __forceinline__ void cow_pair_ids(const DecodeArgs& a, const CowPair& p, int lane, int& cow_src,
                                             int& cow_dst) {
    const int64_t s = (int64_t)(((uint64_t)p.w[1] << 32) | p.w[0]);
    const int64_t d = (int64_t)(((uint64_t)p.w[3] << 32) | p.w[2]);
    const bool use = lane < a.cow_num && s >= 0 && s < a.num_blocks && d >= 0 && d < a.num_blocks;
    cow_src = use ? (int)s : -1;
    cow_dst = use ? (int)d : -1;
}

// The block a partition workgroup reads for physical block pb (wave-uniform):
// the pair's source when pb is a destination of this launch (the same content
// once copied; the copying workgroups run beside the partition ones), else
// pb.  One compare of the pair lanes against pb and a ballot; every lane of
// the wave must call it.
__device__ __forceinline__ int cow_source(int cow_src, int cow_dst, int pb) {
    const uint64_t hit = __builtin_amdgcn_ballot_w64(cow_dst == pb);
    if (hit != 0) pb = __builtin_amdgcn_readlane(cow_src, (int)__builtin_ctzll(hit));
    return pb;
}

// Copy-on-write copies in a decode launch: each (pair, tensor) block copy is
// split into chunks of COW_BATCH * NT 16-byte granules, one workgroup of NT
// threads each, so that every copying workgroup needs one round of loads.
constexpr int COW_BATCH = 8;  // granules per thread in flight
template <Fmt KV, int D, int BS, int NT>
__host__ __device__ inline int cow_chunks(int num_kv_heads) {
    const int granules = num_kv_heads * BS * (D * FmtBytes<KV>::value / 16);
    return (granules + COW_BATCH * NT - 1) / (COW_BATCH * NT);
}

// Copying workgroup w of the launch: chunk w % C of pair w / C / 2, tensor
// w / C % 2 (K, then V), C = cow_chunks: that part of the destination block
// (all kv heads, all rows) from the source block, as pa_copy_blocks does.
// When the destination is some sequence's last block, the row of that
// sequence's new token is written from the new token instead of from the
// source (the partition workgroups read the source for that block and store
// nothing there).  These workgroups are the last of the launch, so their
// chain of dependent memory accesses is kept short: the owner search (each
// sequence's length, then its last block id) runs beside the copy's loads,
// and no store waits for another.
template <Fmt KV, int D, int BS, int NT>
__device__ void cow_copy_block(const DecodeArgs& a, unsigned w) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int ROW_G = D * FmtBytes<KV>::value / 16;  // 16-byte granules per row
    constexpr int U = COW_BATCH;
    const int H = a.num_kv_heads;
    const int chunks = cow_chunks<KV, D, BS, NT>(H);
    const int pt = (int)(w / (unsigned)chunks);
    const int chunk = (int)w - pt * chunks;
    const int p = pt >> 1;
    const int z = pt & 1;
    const int s0 = (int)threadIdx.x;
    // a launch given no new tokens (copies and decode only) writes no row
    // from them: the owner search is skipped
    const bool tokens = a.new_k != nullptr;
    // the first sequences' lengths, loaded with the pair
    const int T0 = tokens && s0 < a.num_seqs ? a.seq_lens[s0] : 0;
    const int64_t src = a.cow_pairs[2 * p];
    const int64_t dst = a.cow_pairs[2 * p + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;  // skipped pair
    const int granules = H * BS * ROW_G;  // one tensor's block: [kv head][row][granule]
    u32x4* pool = (u32x4*)(z == 0 ? a.k_cache : a.v_cache);
    const u32x4* from = pool + (size_t)src * granules;
    u32x4* to = pool + (size_t)dst * granules;
    const u32x4* tok = (const u32x4*)(z == 0 ? a.new_k : a.new_v);  // [seq][kv head][granule]
    int* who = (int*)smem;  // the sequence whose last block is dst, and its new token's row
    if (threadIdx.x == 0) who[0] = -1;

    const int i0 = chunk * U * NT + s0;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (i0 + u * NT < granules) v[u] = from[i0 + u * NT];
    auto owns = [&](int s, int T) {
        return T > 0 && T <= a.max_seq_len && (T + BS - 1) / BS <= a.max_blocks_per_seq &&
               a.block_tables[(size_t)s * a.max_blocks_per_seq + (T - 1) / BS] == (int)dst;
    };
    const bool mine = tokens && s0 < a.num_seqs && owns(s0, T0);
    __syncthreads();  // who[0] is initialised
    // one sequence for valid input (destinations belong to one sequence)
    if (mine) { who[0] = s0; who[1] = (T0 - 1) % BS; }
    for (int s = s0 + NT; tokens && s < a.num_seqs; s += NT) {
        const int T = a.seq_lens[s];
        if (owns(s, T)) { who[0] = s; who[1] = (T - 1) % BS; }
    }
    __syncthreads();
    const int s = who[0];
    const int row = s >= 0 ? who[1] : -1;
    // the new token's granules are loaded together, then everything is stored
    u32x4 t[U];
    bool take[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT;
        take[u] = s >= 0 && i < granules && (i / ROW_G) % BS == row;
        if (take[u]) t[u] = tok[((size_t)s * H + i / (BS * ROW_G)) * ROW_G + i % ROW_G];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (i0 + u * NT < granules) to[i0 + u * NT] = take[u] ? t[u] : v[u];
}

// Wait until at most n whole blocks (0 <= n <= N) of copies are in flight.
template <int PER_BLOCK, int N>
__device__ __forceinline__ void wait_blocks_in_flight(int n) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= N) {
            wait_vmcnt<N * PER_BLOCK>();
            return;
        }
        wait_blocks_in_flight<PER_BLOCK, N - 1>(n);
    }
}

// The partition workgroup's work (generic kernel).  APPEND: decode with
// append, with the launch's copy-on-write pairs (the kernel below).
template <Fmt KV, Fmt Q, int D, int BS, int G, int W, int S, bool APPEND>
__device__ __forceinline__ void generic_partition(const DecodeArgs& a, unsigned bid) {
    using Sh = PartitionShape<KV, D, BS, G, W, S>;
    using Row = LaneRow<KV, D>;
    using Dot = QK<KV, Q>;
    constexpr int LPR = Sh::LPR, R = Sh::R, ROWB = Sh::ROWB, TILE = Sh::TILE;
    constexpr int QB = FmtBytes<Q>::value;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane / LPR;
    const int c = lane % LPR;
    int seq, kvh, part;
    if (!partition_work_item(a, bid, seq, kvh, part)) return;

    const int T = load_uniform(a.seq_lens + seq);
    // copy-on-write pairs of this launch (decode with append only)
    const bool cow = APPEND && a.cow_num > 0;
    CowPair pair{{0u, 0u, 0u, 0u}};
    if constexpr (APPEND) pair = load_cow_pair(a, lane);
    if (T <= 0 || T > a.max_seq_len) return;  // empty or invalid rows: written by the reduce kernel
    if ((T + BS - 1) / BS > a.max_blocks_per_seq) return;
    const int P = a.partition_size;
    const int n_parts = (T + P - 1) / P;
    if (part >= n_parts) return;

    const int tok0 = part * P;
    const int tok1 = min(tok0 + P, T);
    const int lb0 = tok0 / BS;
    const int nblk = (tok1 - tok0 + BS - 1) / BS;
    // this wave's blocks: a contiguous, balanced share of the partition
    const int kb0 = nblk * wave / W;
    const int nbw = nblk * (wave + 1) / W - kb0;
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq + lb0 + kb0;
    // physical ids of the wave's blocks, one per lane (64 at a time); read
    // with readlane when a block's copy is issued
    int ids = lane < nbw ? bt[lane] : 0;
    const int hq0 = kvh * G;

    // Decode with append: the wave that stages the sequence's last block
    // holds the newest token's K and V rows of this kv head in registers (one
    // 16-byte granule of each per lane), writes them over that row of the
    // staged block once the block has landed, and stores them into the pool;
    // the attention never depends on when the store reaches memory.  Kept in
    // registers rather than LDS, so that the appending kernel's LDS footprint
    // (and with it the workgroups resident per CU) is the plain kernel's.
    const bool appends = APPEND && part == n_parts - 1 && nbw > 0 && kb0 + nbw == nblk;
    const int new_row = (T - 1) % BS;  // row of the newest token in its block
    constexpr int NEWG = ROWB / 16;    // 16-byte granules of a row
    u32x4 new_kg = {0u, 0u, 0u, 0u}, new_vg = {0u, 0u, 0u, 0u};
    if (appends && lane < NEWG) {
        const size_t src = ((size_t)seq * a.num_kv_heads + kvh) * ROWB + lane * 16;
        new_kg = *(const u32x4*)((const char*)a.new_k + src);
        new_vg = *(const u32x4*)((const char*)a.new_v + src);
    }

    // Query operands of the G heads (the lane's 8 elements of each).
    typename Dot::Op qop[G];
    {
        const char* qbase = (const char*)a.q + ((size_t)seq * a.num_heads + hq0) * D * QB;
#pragma unroll
        for (int g = 0; g < G; ++g) qop[g] = Dot::template load_q<D>(qbase + (size_t)g * D * QB, c);
        // make the queries resident before any asynchronous copy is queued, so
        // the compiler's own wait for them cannot also wait for the copies
#pragma unroll
        for (int g = 0; g < G; ++g) qop[g].pin();
        if constexpr (APPEND) {  // the pairs and the new rows too, loaded first
            pin_cow_pair(pair);
            asm volatile("" : "+v"(new_kg[0]), "+v"(new_kg[1]), "+v"(new_kg[2]), "+v"(new_kg[3]));
            asm volatile("" : "+v"(new_vg[0]), "+v"(new_vg[1]), "+v"(new_vg[2]), "+v"(new_vg[3]));
        }
    }
    int cow_src = -1, cow_dst = -1;
    if constexpr (APPEND) cow_pair_ids(a, pair, lane, cow_src, cow_dst);
    float qk_scale = a.qk_scale_log2;
    // The value scale is needed only by the final stores, but a load issued
    // there would add a memory round trip to every workgroup's end; both
    // scales are loaded here and made resident before the copies, like the
    // queries.
    float vs = 1.f;
    if constexpr (KV == Fmt::FP8) {
        float ks = load_uniform(a.k_scale + kvh);
        vs = load_uniform(a.v_scale + kvh);
        asm volatile("" : "+v"(ks), "+v"(vs));
        qk_scale *= ks;
    }

    const char* kc = (const char*)a.k_cache;
    const char* vc = (const char*)a.v_cache;
    char* ring = smem + wave * Sh::RING;
    const uint32_t ring_lds = lds_addr_of(smem) + (uint32_t)(wave * Sh::RING);
    int invalid = 0;

    auto issue = [&](int k, int stage) {
        if (k > 0 && (k & 63) == 0) {
            ids = k + lane < nbw ? bt[k + lane] : 0;
            // wait for the new ids here: otherwise the compiler waits (for every
            // copy in flight) before each block's readlane, reloaded or not
            asm volatile("" : "+v"(ids));
        }
        int pb = __builtin_amdgcn_readlane(ids, k & 63);
        if ((unsigned)pb >= (unsigned)a.num_blocks) { invalid = 1; pb = 0; }
        if (cow) pb = cow_source(cow_src, cow_dst, pb);
        const size_t tile = ((size_t)pb * a.num_kv_heads + kvh) * TILE + (size_t)lane * 16;
        const uint32_t dst = ring_lds + (uint32_t)(stage * Sh::STAGE);
#pragma unroll
        for (int i = 0; i < Sh::DMA_PER_TILE; ++i) dma16_to_lds_stream(kc + tile + i * 1024, dst + i * 1024);
#pragma unroll
        for (int i = 0; i < Sh::DMA_PER_TILE; ++i) dma16_to_lds_stream(vc + tile + i * 1024, dst + TILE + i * 1024);
    };

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    // One 16-token chunk of a staged block.  MASKED: the block may hold rows
    // at or beyond T (only the sequence's last block), whose scores become
    // -inf and whose values are ignored.
    auto chunk = [&](const char* kb, int row_tok0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const char* vb = kb + TILE;
        float s[Sh::PASSES][G];
        float v[Sh::PASSES][8];
#pragma unroll
        for (int j = 0; j < Sh::PASSES; ++j) {
            uint32_t kw[Row::NW];
            Row::load(kb + (j * R + r) * ROWB, c, kw);
            const auto kop = Dot::prep_k(kw);
#pragma unroll
            for (int g = 0; g < G; ++g) s[j][g] = group_sum<LPR>(Dot::dot(qop[g], kop));
        }
#pragma unroll
        for (int j = 0; j < Sh::PASSES; ++j) {
            uint32_t vw[Row::NW];
            Row::load(vb + (j * R + r) * ROWB, c, vw);
            Row::to_f32(vw, v[j]);
        }
#pragma unroll
        for (int j = 0; j < Sh::PASSES; ++j) {
            const bool ok = !MASKED || (row_tok0 + j * R + r < T);
#pragma unroll
            for (int g = 0; g < G; ++g) s[j][g] = ok ? mul_rounded(s[j][g], qk_scale) : -INFINITY;
            if constexpr (MASKED) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[j][e] = ok ? v[j][e] : 0.f;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = s[0][g];
#pragma unroll
            for (int j = 1; j < Sh::PASSES; ++j) mx = fmaxf(mx, s[j][g]);
            const float mn = fmaxf(m[g], mx);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[g] - mu);
            float p[Sh::PASSES];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < Sh::PASSES; ++j) { p[j] = fast_exp2(s[j][g] - mu); psum += p[j]; }
            l[g] = fmaf(l[g], alpha, psum);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float t = acc[g][e] * alpha;
#pragma unroll
                for (int j = 0; j < Sh::PASSES; ++j) t = fmaf(p[j], v[j][e], t);
                acc[g][e] = t;
            }
            m[g] = mn;
        }
    };

    // ---- main loop: S-stage ring, S-1 blocks of copies ahead of compute
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        if (k < nbw) issue(k, k);
    int stage = 0;
    for (int k = 0; k < nbw; ++k) {
        if (k + S - 1 < nbw) issue(k + S - 1, stage == 0 ? S - 1 : stage - 1);
        wait_blocks_in_flight<Sh::DMA_PER_BLOCK, S - 1>(min(S - 1, nbw - 1 - k));
        if (appends && k == nbw - 1) {
            // the block's own id (the ids window holding it is the current one)
            const int pb = __builtin_amdgcn_readlane(ids, k & 63);
            // a copy-on-write destination gets the token from its copying workgroup
            const bool stores = !cow || cow_source(cow_src, cow_dst, pb) == pb;
            if (lane < NEWG) {
                const u32x4 kg = new_kg, vg = new_vg;
                char* row = ring + stage * Sh::STAGE + new_row * ROWB + lane * 16;
                *(u32x4*)row = kg;
                *(u32x4*)(row + TILE) = vg;
                if (stores && (unsigned)pb < (unsigned)a.num_blocks) {
                    const size_t dst = ((size_t)pb * a.num_kv_heads + kvh) * TILE + (size_t)new_row * ROWB + lane * 16;
                    *(u32x4*)((char*)a.k_cache + dst) = kg;
                    *(u32x4*)((char*)a.v_cache + dst) = vg;
                }
            }
        }
        const char* kb = ring + stage * Sh::STAGE;
        const int blk_tok0 = (lb0 + kb0 + k) * BS;
        if (blk_tok0 + BS <= T) {
#pragma unroll
            for (int ch = 0; ch < Sh::CHUNKS; ++ch)
                chunk(kb + ch * 16 * ROWB, blk_tok0 + ch * 16, std::false_type{});
        } else {
#pragma unroll
            for (int ch = 0; ch < Sh::CHUNKS; ++ch)
                chunk(kb + ch * 16 * ROWB, blk_tok0 + ch * 16, std::true_type{});
        }
        stage = stage + 1 == S ? 0 : stage + 1;
    }

    // ---- merge the row subsets of this wave (lanes l, l^LPR, l^2LPR, ...)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], off);
            const float lo = __shfl_xor(l[g], off);
            const float mn = fmaxf(m[g], mo);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float f0 = fast_exp2(m[g] - mu);
            const float f1 = fast_exp2(mo - mu);
            l[g] = l[g] * f0 + lo * f1;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * f0 + __shfl_xor(acc[g][e], off) * f1;
            m[g] = mn;
        }
    }

    auto emit = [&](int g, int d, float L, float A, int bad) {
        const int hq = hq0 + g;
        const size_t row = (size_t)seq * a.num_heads + hq;
        if (n_parts == 1) {
            store_out(a.out, a.out_dtype, row * D + d, bad ? __builtin_nanf("") : A / L * vs);
        } else {
            const size_t pidx = row * a.max_partitions + part;
            store_state_stream(&a.part_acc[pidx * D + d], bad ? __builtin_nanf("") : A * vs);
        }
    };
    float* const ml_rec = a.part_ml + ml_record(a, seq, kvh, part);

    if constexpr (W == 1) {
        // lane 0's m and l, the values its rows' accumulators were merged with
        auto lane0 = [](float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)); };
        auto pick = [&](const float (&x)[G], int g) {  // x[g] of lane 0, g per lane
            float r = lane0(x[0]);
#pragma unroll
            for (int gg = 1; gg < G; ++gg) r = g == gg ? lane0(x[gg]) : r;
            return r;
        };
        if (n_parts > 1)
            store_ml_record<G, true>(ml_rec, lane, invalid != 0, [&](int g) { return pick(m, g); },
                                     [&](int g) { return pick(l, g); });
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) emit(g, Row::dim(c, e), l[g], acc[g][e], invalid);
        }
    } else {
        __syncthreads();  // every wave is done with its ring; reuse the LDS for the merge
        float* wm = (float*)smem;
        float* wl = wm + W * G;
        int* winv = (int*)(wl + W * G);
        float* wacc = (float*)(smem + Sh::MERGE_HEAD);
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) { wm[wave * G + g] = m[g]; wl[wave * G + g] = l[g]; }
            winv[wave] = invalid;
        }
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float* row = wacc + (wave * G + g) * D;  // elements e < 4 and e >= 4 are 4 consecutive dims each
                *(float4*)(row + merge_pos(Row::dim(c, 0))) = float4{acc[g][0], acc[g][1], acc[g][2], acc[g][3]};
                *(float4*)(row + merge_pos(Row::dim(c, 4))) = float4{acc[g][4], acc[g][5], acc[g][6], acc[g][7]};
            }
        }
        __syncthreads();
        int bad = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) bad |= winv[w];
        auto merged_m = [&](int g) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < W; ++w) M = fmaxf(M, wm[w * G + g]);
            return M;
        };
        auto merged_l = [&](int g) {
            const float M = merged_m(g);
            const float mu = M == -INFINITY ? 0.f : M;
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) L = fmaf(fast_exp2(wm[w * G + g] - mu), wl[w * G + g], L);
            return L;
        };
        if (n_parts > 1 && wave == 0) store_ml_record<G, true>(ml_rec, lane, bad != 0, merged_m, merged_l);
        for (int o = threadIdx.x; o < G * D; o += W * 64) {
            const int g = o / D;
            const int d = o - g * D;
            const float M = merged_m(g);
            const float mu = M == -INFINITY ? 0.f : M;
            float L = 0.f, A = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float f = fast_exp2(wm[w * G + g] - mu);
                L = fmaf(f, wl[w * G + g], L);
                A = fmaf(f, wacc[(w * G + g) * D + merge_pos(d)], A);
            }
            emit(g, d, L, A, bad);
        }
    }
}

template <Fmt KV, Fmt Q, int D, int BS, int G, int W, int S, bool APPEND>
__global__ void __launch_bounds__(W * 64)
decode_partition_kernel(const DecodeArgs a) {
    if constexpr (APPEND) {
        // decode with append: the copy-on-write pairs' workgroups come last,
        // where the tail of the partition work leaves slots idle (nothing here
        // reads their destinations)
        const unsigned parts = (unsigned)a.num_seqs * (unsigned)a.max_partitions * (unsigned)a.num_kv_heads;
        if (blockIdx.x >= parts) {
            cow_copy_block<KV, D, BS, W * 64>(a, blockIdx.x - parts);
            return;
        }
    }
    generic_partition<KV, Q, D, BS, G, W, S, APPEND>(a, blockIdx.x);
}

// Launch one partition-kernel instantiation (sets the LDS attribute once).
template <Fmt KV, Fmt Q, int D, int BS, int G, int W, int S, bool APPEND>
int launch_partition_as(const DecodeArgs& a, hipStream_t stream) {
    using Sh = PartitionShape<KV, D, BS, G, W, S>;
    constexpr int LDS = Sh::LDS;
    auto kernel = decode_partition_kernel<KV, Q, D, BS, G, W, S, APPEND>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const size_t copies = APPEND ? 2 * (size_t)a.cow_num * cow_chunks<KV, D, BS, W * 64>(a.num_kv_heads) : 0;
    const dim3 grid((unsigned)(copies + (size_t)a.num_seqs * a.max_partitions * a.num_kv_heads));
    hipLaunchKernelGGL(kernel, grid, dim3(W * 64), LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// The plain kernel, or the one that also stores the new tokens and makes the
// launch's copy-on-write copies (decode with append): separate
// instantiations, so that the plain one carries none of it.
template <Fmt KV, Fmt Q, int D, int BS, int G, int W, int S>
int launch_partition(const DecodeArgs& a, hipStream_t stream) {
    return a.new_k != nullptr ? launch_partition_as<KV, Q, D, BS, G, W, S, true>(a, stream)
                              : launch_partition_as<KV, Q, D, BS, G, W, S, false>(a, stream);
}

// Shared-prefix partition states (pa_decode_prefix.hip): whether the
// matrix-core tile covers the shape, and the launch that writes the states of
// every group's shared partitions plus the per-sequence skip counts.
bool prefix_states_supported(int kv_dtype, int q_dtype, int head_dim, int block_size, int group);
int launch_prefix_states(const DecodeArgs& d, int kv_dtype, int group, const int32_t* group_start,
                         const int32_t* group_prefix, int num_groups, int max_group_size, int max_prefix_len,
                         int32_t* skip, hipStream_t stream);
// 4-head groups: the skips first (a small kernel), then, after the plan if
// any, one launch for the shared partitions and the decode partitions.
bool prefix_fused_supported(int kv_dtype, int q_dtype, int head_dim, int block_size, int group);
int launch_prefix_skips(const DecodeArgs& d, const int32_t* group_start, const int32_t* group_prefix,
                        int num_groups, int max_group_size, int max_prefix_len, int32_t* skip, hipStream_t stream);
int launch_prefix_fused(const DecodeArgs& d, int kv_dtype, const int32_t* group_start, const int32_t* group_prefix,
                        int num_groups, int max_group_size, int max_prefix_len, int32_t* skip, hipStream_t stream);

// Per-format dispatch over head_dim, block_size and group size; defined in
// one translation unit per KV format.
int launch_partition_f32(const DecodeArgs& a, int head_dim, int group, hipStream_t stream);
int launch_partition_f16(const DecodeArgs& a, int head_dim, int group, hipStream_t stream);
int launch_partition_bf16(const DecodeArgs& a, int head_dim, int group, hipStream_t stream);
int launch_partition_fp8_bf16q(const DecodeArgs& a, int head_dim, int group, hipStream_t stream);

// Waves per workgroup and ring depth of the default variant.
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 2
#endif
#ifndef PA_DECODE_STAGES
#define PA_DECODE_STAGES 2
#endif

// Ring depth and waves per workgroup for a shape: the defaults, reduced
// until the copies of S-1 blocks fit the vmcnt counter (63) and the rings of
// all waves fit in the 160 KiB of LDS a workgroup may use.
template <Fmt KV, int D, int BS>
constexpr int stages_for() {
    constexpr int stage = 2 * BS * D * FmtBytes<KV>::value;
    int s = PA_DECODE_STAGES;
    while (s > 2 && ((s - 1) * (stage / 1024) > 63 || s * stage > 160 * 1024)) --s;
    return s;
}

template <Fmt KV, int D, int BS, int S>
constexpr int waves_for() {
    int w = PA_DECODE_WAVES;
    while (w > 1 && w * S * 2 * BS * D * FmtBytes<KV>::value > 160 * 1024) w /= 2;
    return w;
}

template <Fmt KV, Fmt Q, int D, int BS>
int dispatch_group(const DecodeArgs& a, int group, hipStream_t stream) {
    constexpr int S = stages_for<KV, D, BS>();
    constexpr int W = waves_for<KV, D, BS, S>();
    switch (group) {
        case 1: return launch_partition<KV, Q, D, BS, 1, W, S>(a, stream);
        case 2: return launch_partition<KV, Q, D, BS, 2, W, S>(a, stream);
        case 4: return launch_partition<KV, Q, D, BS, 4, W, S>(a, stream);
        case 8: return launch_partition<KV, Q, D, BS, 8, W, S>(a, stream);
    }
    return PA_ERR_UNSUPPORTED;
}

#define PA_DEFINE_PARTITION_DISPATCH(NAME, KVF, QF)                                  \
    int NAME(const DecodeArgs& a, int head_dim, int group, hipStream_t stream) {     \
        const int bs = a.block_size;                                                 \
        if (head_dim == 128 && bs == 16) return dispatch_group<KVF, QF, 128, 16>(a, group, stream); \
        if (head_dim == 128 && bs == 32) return dispatch_group<KVF, QF, 128, 32>(a, group, stream); \
        if (head_dim == 64 && bs == 16) return dispatch_group<KVF, QF, 64, 16>(a, group, stream);   \
        if (head_dim == 64 && bs == 32) return dispatch_group<KVF, QF, 64, 32>(a, group, stream);   \
        return PA_ERR_UNSUPPORTED;                                                   \
    }

}  // namespace pa
