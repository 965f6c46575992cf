// Multi-query attention tile on the gfx950 matrix cores, shared by the
// prefill kernel (pa_prefill.hip) and the shared-prefix kernel
// (pa_decode_prefix.hip).
//
// A workgroup of four waves computes 64 CB query columns -- (token or
// sequence, query head) pairs of one kv head, CB blocks of 16 per wave --
// over a contiguous range of keys read through one block-table row.  The keys
// are walked in steps of 32 (two blocks of 16 or one of 32): the step's K and
// V rows are copied once into LDS (the four waves issue a quarter of the
// 16-byte asynchronous copies each) and serve all the columns; inside a wave
// each K and V operand read from LDS serves its CB column blocks.  An
// S-stage ring holds the two steps being computed (the score products of
// step k + 1 run beside the value products of step k) and S - 2 steps of
// copies in flight; one barrier per step separates "everyone finished step
// k-1" from "step k+S-1 may overwrite its stage".
//
// Per wave, with v_mfma_f32_16x16x32 (bf16 or f16 operands, f32
// accumulation) and lane = 16 g + n (g = 0..3, n = 0..15):
//   scores   S^T[key][column] = K Q^T: A = K rows (lane supplies row n of
//            the 16-key half, elements 32 c + 8 g .. + 7 for the c-th of four
//            products over head_dim 128), B = the wave's query columns.  The
//            lane receives column n's scores for keys 4 g + i, i = 0..3, of
//            each half.
//   softmax  per column: the lane's 8 weights against a reference maximum
//            uniform over the column's lanes, which moves (rescaling the
//            accumulators) only when a weight passes 2^MQ_SLACK; keys after
//            the column's last visible position get weight 0.
//   values   O^T[dim][column] += V^T P^T: B = the lane's own p; A = V^T,
//            the lane supplying dim 16 j + n of its 8 keys, delivered in
//            that order by two transposing LDS reads per 16-dim block j.  The
//            lane receives column n's dims 16 j + 4 g + i.  Two forms of p
//            (the SPLIT template argument):
//            - split: a 16-bit high part and the rounded remainder, two
//              products, so p keeps about 16 significant bits; the column
//              sum l adds the unrounded p.
//            - single: p rounded to the 16-bit format, one product; l is
//              the sum of the rounded weights, accrued on the matrix cores
//              (an all-ones A against P^T).  The output is then a convex
//              combination of the values with each weight off by at most
//              half an ulp of the format (2^-9 relative for bf16, 2^-12 for
//              f16), so its error is at most that fraction of the spread of
//              the values, and no bias remains from a rounded numerator over
//              an unrounded denominator.
// K rows sit in LDS XOR-swizzled by 16-byte granule (row t, granule x at
// slot x ^ (t mod 16)) and V rows by pairs of granules (x ^ 2 (t mod 8)),
// both through the copies' source addresses, so that the reads above spread
// over the banks (a transposing read touches one 32-byte dim block of 16
// rows, whose t mod 8 take every value twice).  The K operand's element
// order matters as much: with granule 4 c + g (the four lane groups of one
// product read 64 consecutive bytes of their rows) the 16-byte reads run at
// the full LDS rate on gfx950; with granule 4 g + c they ran at half of it
// (a read-throughput probe of both patterns).
//
// The physical block ids of the key range are loaded into LDS first (in
// windows of ID_CAP blocks).  An id outside the pool is never used as an
// address: block 0 is read instead and `bad` is set.  Rows at or beyond the
// task's kv_len (the tail of a sequence's last block) are dropped: their
// scores are masked and their values zeroed.
#pragma once

#include <type_traits>

#include "pa_decode_kernel.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <Fmt F> struct MfmaOps;
template <> struct MfmaOps<Fmt::BF16> {
    typedef bf16x8 vec;
    typedef bf16x2 pair;
    __device__ static __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MfmaOps<Fmt::F16> {
    typedef f16x8 vec;
    typedef f16x2 pair;
    __device__ static __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Two-part 16-bit form of 8 weights: hi = round(p), lo = round(p - hi), so
// that hi + lo keeps about 16 significant bits of p.  Pairs are converted
// together (one packed conversion each for hi and lo).
template <Fmt KV>
__device__ __forceinline__ void mq_split8(const float (&p)[8], typename MfmaOps<KV>::vec& hi,
                                          typename MfmaOps<KV>::vec& lo) {
    using pair = typename MfmaOps<KV>::pair;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const pair h = __builtin_convertvector(f32x2{p[e], p[e + 1]}, pair);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const pair r = __builtin_convertvector(f32x2{p[e] - hf[0], p[e + 1] - hf[1]}, pair);
        hi[e] = h[0];
        hi[e + 1] = h[1];
        lo[e] = r[0];
        lo[e + 1] = r[1];
    }
}

// 8 weights rounded to the 16-bit format, one packed conversion per pair.
template <Fmt KV>
__device__ __forceinline__ void mq_round8(const float (&p)[8], typename MfmaOps<KV>::vec& hi) {
    using pair = typename MfmaOps<KV>::pair;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const pair h = __builtin_convertvector(f32x2{p[e], p[e + 1]}, pair);
        hi[e] = h[0];
        hi[e + 1] = h[1];
    }
}

// Maxima as single instructions (no NaN canonicalisation of the operands:
// the scores come from the matrix cores and are never signalling NaNs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Maximum and sum over the four 16-lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float mq_max_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float mq_sum_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

#ifndef PA_MQ_STAGES
#define PA_MQ_STAGES 4
#endif

// D: head_dim; BS: block size; G: query heads per kv head; CB: 16-column
// blocks per wave; STAGES: LDS ring depth.
template <int D, int BS, int G, int CB = 1, int STAGES = PA_MQ_STAGES, int WAVES = 4>
struct MqShape {
    static constexpr int S = STAGES;              // LDS stages (S - 1 steps of copies in flight)
    static constexpr int W = WAVES;               // waves per workgroup
    static constexpr int COLS = 16 * CB;          // query columns per wave
    static constexpr int TQ = W * COLS / G;       // query tokens (or sequences) per workgroup
    static constexpr int PER_WAVE = COLS / G;     // query tokens (or sequences) per wave
    static constexpr int STEP = 32;               // keys per step
    static constexpr int BPS = STEP / BS;         // blocks per step
    static constexpr int ROWB = D * 2;            // bytes of one K or V row
    static constexpr int HALF = STEP * ROWB;      // K (or V) rows of one step
    static constexpr int STAGE = 2 * HALF;
    static constexpr int COPIES = STAGE / 1024;   // 1 KiB copies per step
    static constexpr int COPIES_PER_WAVE = COPIES / W;
    static constexpr int ID_CAP = 2048;           // block ids held in LDS
    static constexpr int IDS_AT = S * STAGE;
    static constexpr int LDS = IDS_AT + ID_CAP * 4 + (W * 4 + 15) / 16 * 16;
    static_assert(D == 128, "the lane roles assume head_dim 128");
    static_assert(BS == 16 || BS == 32, "block size");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group");
    static_assert(CB == 1 || CB == 2, "column blocks per wave");
    static_assert(COPIES % W == 0 && COPIES / 2 % COPIES_PER_WAVE == 0, "a wave copies only K or only V");
    static_assert(BS % (4 * COPIES_PER_WAVE) == 0, "a wave's copies of one step stay inside one block");
    static_assert(LDS <= 160 * 1024, "LDS budget");

    static_assert(ID_CAP % BPS == 0, "a step's blocks never straddle an id window");
    static_assert(S >= 3, "two resident steps (the pipelined loop) plus one being refilled");
    static_assert((S - 2) * COPIES_PER_WAVE <= 63, "vmcnt holds the copies of S - 2 steps");
};

// How far (log2 units) a column's running maximum may rise above the
// reference its weights are taken against before the reference is moved and
// the accumulators rescaled: weights stay below 2^8, far from float overflow.
constexpr float MQ_SLACK = 8.f;
constexpr float kMqSlackWeight = 256.f;  // 2^MQ_SLACK

// Waits until at most `later` (< N + 1) steps of C copies each, issued after
// the one needed now, are still in flight.
template <int C, int N>
__device__ __forceinline__ void wait_later_steps(int later) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= N)
            wait_vmcnt<N * C>();
        else
            wait_later_steps<C, N - 1>(later);
    }
}

// Four consecutive output elements (idx a multiple of 4).
__device__ __forceinline__ void store_out4(void* out, int dtype, size_t idx, f32x4 v) {
    if (dtype == PA_DTYPE_F32) {
        *(f32x4*)((float*)out + idx) = v;
    } else if (dtype == PA_DTYPE_BF16) {
        const uint32_t lo = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        *(u32x2*)((uint16_t*)out + idx) = u32x2{lo, hi};
    } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        *(h4*)((_Float16*)out + idx) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    }
}

// The pool and the score scale.
struct MqPool {
    const void* k_cache;
    const void* v_cache;
    int num_kv_heads;
    int num_blocks;
    float qk_scale_log2;  // scale * log2(e)
};

// One workgroup's tile: the key range (block aligned start), and this lane's
// column in each of the wave's CB column blocks.
template <int CB>
struct MqTask {
    const int32_t* bt;       // block-table row that holds the key range
    int key_begin;           // first key; a multiple of the block size
    int key_end;             // one past the last key any column sees
    int kv_len;              // rows at or beyond this key hold no data
    int kvh;
    const void* qptr[CB];    // the column's query row (read only when cvalid)
    bool cvalid[CB];         // the lane's column exists
    int cpos[CB];            // last key the lane's column sees
    bool wave_cols;          // the wave has at least one column
    int wpos_min;            // smallest and largest last-visible key over the wave's columns
    int wpos_max;
};

// Runs the tile.  On return every lane holds, for each column block cb, its
// column's reference m[cb] (log2 units, uniform over the column's lanes; at
// most MQ_SLACK below the column's largest scaled score, -inf if it saw no
// key), the sum l[cb] = sum 2^(c s - m) over all its keys, and the
// unnormalised accumulators acc[cb][a][b][i] = sum 2^(c s - m) v for dims
// 64 a + 16 b + 4 g + i, so that (m, l, acc) is a partition state in the
// decode kernels' sense; `bad` is set when the table named a block outside
// the pool.  All threads of the workgroup must call it.  STREAM marks the
// K/V copies non-temporal (data read once).
template <Fmt KV, int D, int BS, int G, int CB, int STAGES, bool STREAM, bool SPLIT, int WAVES = 4>
__device__ void mq_tile(const MqPool& pool, const MqTask<CB>& t, char* smem, float (&m)[CB], float (&l)[CB],
                        f32x4 (&acc)[CB][2][4], bool& bad) {
    using Sh = MqShape<D, BS, G, CB, STAGES, WAVES>;
    using Ops = MfmaOps<KV>;
    using vec = typename Ops::vec;
    constexpr int ROWB = Sh::ROWB, STEP = Sh::STEP, BPS = Sh::BPS, S = Sh::S, CPW = Sh::COPIES_PER_WAVE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int n = lane & 15;
    const int H = pool.num_kv_heads;
    const int kvh = t.kvh;

    // ---- queries of this lane's columns (zero for missing columns).  A
    // negative score scale is moved into the queries (an exact sign flip), so
    // that the scale c applied below is never negative and max(c s) = c max(s).
    const uint32_t qsign = pool.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
    const float c_scale = fabsf(pool.qk_scale_log2);

    // ---- block ids of the key range into LDS, in windows of ID_CAP.  Each
    // wave records in its own flag whether an id it loaded was outside the
    // pool.  The first window's ids are loaded before the queries: loads
    // return in order, so the ids can be waited for (and the first copies
    // issued) while the queries, whose latency is the longest of the tile's
    // start, are still in flight.
    int* ids = (int*)(smem + Sh::IDS_AT);
    int* bad_flags = ids + Sh::ID_CAP;  // [W], written only by their waves
    const int blk0 = t.key_begin / BS;                  // first block of the range
    const int nblk = (t.key_end - 1) / BS + 1 - blk0;   // blocks of the range
    constexpr int IDS_PER_THREAD = Sh::ID_CAP / (Sh::W * 64);
    bool wave_bad = false;
    auto fetch_ids = [&](int first, int (&v)[IDS_PER_THREAD]) {
        const int cnt = min(Sh::ID_CAP, nblk - first);
#pragma unroll
        for (int r = 0; r < IDS_PER_THREAD; ++r) {
            const int j = (int)threadIdx.x + r * Sh::W * 64;
            v[r] = t.bt[blk0 + first + min(j, cnt - 1)];  // (cnt >= 1) entries past cnt are not written
        }
        return cnt;
    };
    auto write_ids = [&](const int (&v)[IDS_PER_THREAD], int cnt) {
        bool out_of_pool = false;
#pragma unroll
        for (int r = 0; r < IDS_PER_THREAD; ++r) {
            const int j = (int)threadIdx.x + r * Sh::W * 64;
            if (j < cnt) {
                int id = v[r];
                if ((unsigned)id >= (unsigned)pool.num_blocks) {
                    out_of_pool = true;
                    id = 0;
                }
                ids[j] = id;
            }
        }
        wave_bad = wave_bad || __builtin_amdgcn_ballot_w64(out_of_pool) != 0;
        if (lane == 0) bad_flags[wave] = wave_bad;
    };
    auto load_ids = [&](int first) {
        int v[IDS_PER_THREAD];
        const int cnt = fetch_ids(first, v);
        write_ids(v, cnt);
    };
    int window = 0;  // first block (relative to blk0) held in `ids`
    int ids0[IDS_PER_THREAD];
    const int cnt0 = fetch_ids(0, ids0);
    __builtin_amdgcn_sched_barrier(0);  // every id load is issued before the query loads
    // the queries of the lane's columns (converted after the first copies landed)
    u32x4 qraw[CB][4];
    vec qop[CB][4];  // [cb][c]: elements 32 c + 8 g .. + 7 of the lane's column
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const u32x4* qp = (const u32x4*)t.qptr[cb] + g;
#pragma unroll
        for (int c = 0; c < 4; ++c) qraw[cb][c] = qp[4 * c];
    }
    __builtin_amdgcn_sched_barrier(0);
    write_ids(ids0, cnt0);
    // the ids are visible to every wave; the queries may still be in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- copies of one step: wave w copies CPW 1 KiB pieces (waves 0 .. W/2-1
    // the K pieces, the others the V pieces); each covers 4 rows of 256 bytes,
    // and the CPW pieces of a wave are 4 CPW consecutive rows of one block.
    // So a wave reads one block id per step (a uniform LDS read) and its
    // copies differ only in a fixed per-lane offset inside the block.
    const bool wave_v = wave * CPW >= Sh::COPIES / 2;
    const uint64_t block_bytes = (uint64_t)H * BS * ROWB;
    const uint32_t lds0 = lds_addr_of(smem);
    const int wrow0 = (wave_v ? wave * CPW - Sh::COPIES / 2 : wave * CPW) * 4;  // the wave's first row in the step
    const int wblk = wrow0 / BS;                                                 // its block, relative to the step's first
    const char* cp_pool = (const char*)(wave_v ? pool.v_cache : pool.k_cache);
    uint32_t cp_off[CPW];  // the piece's row and granule inside one block
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int row = wrow0 + 4 * j + lane / 16;  // key row inside the step
        const int slot = lane % 16;                 // 16-byte slot in the LDS row
        const int gran = wave_v ? (slot ^ ((row & 7) << 1)) : (slot ^ (row & 15));
        cp_off[j] = (uint32_t)(((kvh * BS) + row % BS) * ROWB + gran * 16);
    }
    const uint32_t cp_dst0 = (uint32_t)((wave_v ? Sh::HALF : 0) + wrow0 * ROWB);  // LDS offset inside a stage
    // the physical block this wave copies for step k (its ids window is loaded)
    auto read_id = [&](int k) {
        const int b0 = k * BPS - window;  // the step's first block in `ids`
        // a block past the range (the step's second, in the last step) rereads the first
        const int use = k * BPS + wblk < nblk ? b0 + wblk : b0;
        return ids[use];
    };
    auto issue = [&](int k, int stage, int id) {
        const uint32_t pb = (uint32_t)__builtin_amdgcn_readfirstlane(id);
        const char* src = cp_pool + pb * block_bytes;
        const uint32_t dst = lds0 + (uint32_t)(stage * Sh::STAGE) + cp_dst0;
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            if constexpr (STREAM)
                dma16_to_lds_stream_s(src, cp_off[j], dst + (uint32_t)(j * 1024));
            else
                dma16_to_lds_s(src, cp_off[j], dst + (uint32_t)(j * 1024));
        }
    };

#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        m[cb] = -INFINITY;
        l[cb] = 0.f;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[cb][aa][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int cpos[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) cpos[cb] = t.cvalid[cb] ? t.cpos[cb] : -1;  // missing columns see no key

    // LDS read offsets that do not depend on the step
    const int kslot[4] = {(0 + g) ^ n, (4 + g) ^ n, (8 + g) ^ n, (12 + g) ^ n};

    auto stage_of = [&](int k) { return smem + (k % S) * Sh::STAGE; };

    // scores of step k, both 16-key halves: sc[cb][h][i] is key k0 + 16 h +
    // 4 g + i; each K operand read from LDS serves every column block
    f32x4 sc[CB][2];
    auto qk = [&](int k) {
        const char* kb = stage_of(k);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) sc[cb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const vec ka = __builtin_bit_cast(vec, *(const u32x4*)(kb + (16 * h + n) * ROWB + kslot[cc] * 16));
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) sc[cb][h] = Ops::mma(ka, qop[cb][cc], sc[cb][h]);
            }
    };

    // Weights of step k from its scores.  Online softmax with a lazily moved
    // reference: p = 2^(c s - m) against the column's reference m, which
    // moves to the running maximum only when that exceeds m by more than
    // MQ_SLACK (so p <= 2^MQ_SLACK); l and acc always refer to the current m.
    // The common part computes p against the current m for every column
    // block without a branch (so that it can run between the value products
    // of the previous step); the rare move, which also rescales acc, follows
    // per block and recomputes the weights.
    vec phi[CB], plo[CB];
    // Without the split, the column sums of the rounded weights accrue on the
    // matrix cores: lacc[cb] = sum over keys of (all-ones 16 x 32) P^T, every
    // element the column's sum.
    f32x4 lacc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) lacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t one2 = KV == Fmt::BF16 ? 0x3F803F80u : 0x3C003C00u;  // two 16-bit ones
    const vec ones = __builtin_bit_cast(vec, u32x4{one2, one2, one2, one2});
    auto softmax = [&](int k, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int k0 = t.key_begin + k * STEP;
        bool ok[CB][2][4];
        float l0[CB];
        bool move[CB];
        float pmax;  // largest weight of the last weights() call (lane-local)
        auto weights = [&](int cb, float nmu) {
            float p[8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[4 * h + i] = fast_exp2(fmaf(sc[cb][h][i], c_scale, nmu));
                    if constexpr (MASKED) p[4 * h + i] = ok[cb][h][i] ? p[4 * h + i] : 0.f;
                }
            pmax = max3f(max3f(p[0], p[1], p[2]), max3f(p[3], p[4], p[5]), max2f(p[6], p[7]));
            if constexpr (SPLIT) {
                mq_split8<KV>(p, phi[cb], plo[cb]);
                return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            } else {
                mq_round8<KV>(p, phi[cb]);
                return 0.f;  // the sum of the rounded weights accrues in lacc
            }
        };
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) ok[cb][h][i] = !MASKED || k0 + 16 * h + 4 * g + i <= cpos[cb];
            l0[cb] = l[cb];
            const bool fresh = m[cb] == -INFINITY;  // no reference yet: weights against 0
            l[cb] = l0[cb] + weights(cb, fresh ? 0.f : -m[cb]);  // (SPLIT only; else unused)
            // The reference moves when a weight passes 2^MQ_SLACK, or at the
            // column's first visible key.  (A weight is 2^(c s - m): it passes
            // 2^MQ_SLACK exactly when the scaled score passes m + MQ_SLACK, up
            // to the rounding of the exponent's argument.)
            bool vis = true;
            if constexpr (MASKED) {
                vis = false;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vis = vis || ok[cb][h][i];
            }
            move[cb] = pmax > kMqSlackWeight || (fresh && vis);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (__builtin_amdgcn_ballot_w64(move[cb]) != 0) {
                // the column's largest scaled score (uniform over its lanes)
                auto mval = [&](int h, int i) { return ok[cb][h][i] ? sc[cb][h][i] : -INFINITY; };
                float mx = max3f(max3f(mval(0, 0), mval(0, 1), mval(0, 2)), max3f(mval(0, 3), mval(1, 0), mval(1, 1)),
                                 max3f(mval(1, 2), mval(1, 3), -INFINITY));
                mx = mq_max_groups(mx);
                const float mxs = mx == -INFINITY ? -INFINITY : mx * c_scale;  // c >= 0: max of the scaled scores
                const float mn = fmaxf(m[cb], mxs);
                const float mu = mn == -INFINITY ? 0.f : mn;
                const float alpha = fast_exp2(m[cb] - mu);
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[cb][aa][b] *= alpha;
                if constexpr (!SPLIT) lacc[cb] *= alpha;
                m[cb] = mn;
                l[cb] = l0[cb] * alpha + weights(cb, -mu);
            }
        }
    };
    // acc += V^T P^T for step k.  The operand of dims 16 j .. 16 j + 15 comes
    // from two transposing LDS reads (ds_read_b64_tr_b16), one per 16-key
    // half h: in each group of 16 lanes, lane l names the 8 bytes of V row
    // 16 h + 4 g + l / 4 at dims 16 j + 4 (l % 4) .. + 3, and lane n receives
    // dim 16 j + n of keys 16 h + 4 g + i, i = 0..3 -- the keys of its
    // weights phi[4 h + i].  Rows past the data are zeroed (they may hold
    // anything, and 0 * NaN is NaN).
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int tr_row = 4 * g + (n >> 2);          // row inside a 16-key half
    const int tr_gran = (n & 3) >> 1;             // granule inside the 32-byte dim block
    const int tr_off = (n & 1) * 8;               // byte inside the granule
    auto pv = [&](int k, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int k0 = t.key_begin + k * STEP;
        const __attribute__((address_space(3))) char* vb =
            (const __attribute__((address_space(3))) char*)(stage_of(k) + Sh::HALF);
        uint32_t keep[2][2] = {{~0u, ~0u}, {~0u, ~0u}};  // per half: elements (0, 1) and (2, 3)
        if constexpr (MASKED) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const int key = k0 + 16 * h + 4 * g + 2 * w;
                    keep[h][w] = (key < t.kv_len ? 0xffffu : 0u) | (key + 1 < t.kv_len ? 0xffff0000u : 0u);
                }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            u32x4 op;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 16 * h + tr_row;
                const int slot = (2 * j + tr_gran) ^ ((row & 7) << 1);
                const v4i16 e = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(vb + row * ROWB + slot * 16 + tr_off));
                const u32x2 d = __builtin_bit_cast(u32x2, e);
                op[2 * h] = d[0] & keep[h][0];
                op[2 * h + 1] = d[1] & keep[h][1];
            }
            const vec A = __builtin_bit_cast(vec, op);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                acc[cb][j >> 2][j & 3] = Ops::mma(A, phi[cb], acc[cb][j >> 2][j & 3]);
                if constexpr (SPLIT) acc[cb][j >> 2][j & 3] = Ops::mma(A, plo[cb], acc[cb][j >> 2][j & 3]);
            }
            if constexpr (!SPLIT) {
                if (j == 0) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) lacc[cb] = Ops::mma(ones, phi[cb], lacc[cb]);
                }
            }
        }
    };

    // ---- main loop over 32-key steps, software pipelined: iteration k
    // issues the score products of step k + 1 and the value products of
    // step k, then turns step k + 1's scores into weights while those run.
    // Steps k and k + 1 are resident (S - 2 steps of copies in flight); the
    // first S - 1 steps never need a new id window (S - 1 < ID_CAP / BPS).
    // Steps before k_plain need no mask for any column of this wave (all
    // their keys are visible and hold data); steps from k_vis on hold no key
    // any column of the wave sees.
    const int nsteps = (t.key_end - t.key_begin + STEP - 1) / STEP;
    const int steps_per_window = Sh::ID_CAP / BPS;
    const int lim = min(t.wpos_min + 1, t.kv_len) - t.key_begin;
    const int k_plain = __builtin_amdgcn_readfirstlane(t.wave_cols ? min(max(lim, 0) / STEP, nsteps) : 0);
    const int vis = t.wpos_max - t.key_begin;
    const int k_vis = __builtin_amdgcn_readfirstlane(t.wave_cols && vis >= 0 ? min(vis / STEP + 1, nsteps) : 0);
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        if (k < nsteps) issue(k, k, read_id(k));
    // The id of the next step to copy is read one iteration ahead, so that
    // its LDS latency is not waited for at the copy; not across a window
    // boundary (the next window is not loaded yet).
    int next_id = S - 1 < nsteps ? read_id(S - 1) : 0;
    // wait until this wave's copies of steps <= `need` are complete, then
    // the barrier: everyone's copies up to `need` landed
    auto landed = [&](int need) {
        const int issued = min(need == 0 ? S - 2 : need + S - 3, nsteps - 1);  // last step issued so far
        wait_later_steps<CPW, S - 2>(issued - need);
        __syncthreads();
    };
    auto advance = [&](int k) {
        landed(min(k + 1, nsteps - 1));  // steps k and k + 1; step k - 1 is finished everywhere
        const int kn = k + S - 1;        // the step whose copies go out now, into step k-1's stage
        if (kn < nsteps) {
            if (kn % steps_per_window == 0) {  // its ids are in the next window
                window = kn * BPS;
                load_ids(window);
                __syncthreads();
                next_id = read_id(kn);
            }
            issue(kn, kn % S, next_id);
            if (kn + 1 < nsteps && (kn + 1) % steps_per_window != 0) next_id = read_id(kn + 1);
        }
    };
    // Operands of the lane's columns (zero for missing columns).  A negative
    // score scale is moved into the queries (an exact sign flip), so that the
    // scale c applied below is never negative and max(c s) = c max(s).
    auto take_queries = [&] {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                qop[cb][c] = __builtin_bit_cast(vec, t.cvalid[cb] ? (qraw[cb][c] ^ qsign) : u32x4{0, 0, 0, 0});
    };
    if (nsteps > 0) {
        landed(0);
        take_queries();
        if (k_vis > 0) {
            qk(0);
            if (k_plain > 0)
                softmax(0, std::false_type{});
            else
                softmax(0, std::true_type{});
        }
    }
    int k = 0;
    for (; k + 1 < k_plain; ++k) {  // steps k and k + 1 plain
        advance(k);
        qk(k + 1);
        pv(k, std::false_type{});
        softmax(k + 1, std::false_type{});
    }
    if (k < k_plain) {  // step k plain, k + 1 masked (or past the wave's keys)
        advance(k);
        if (k + 1 < k_vis) qk(k + 1);
        pv(k, std::false_type{});
        if (k + 1 < k_vis) softmax(k + 1, std::true_type{});
        ++k;
    }
    for (; k < nsteps; ++k) {
        advance(k);
        if (k + 1 < k_vis) qk(k + 1);
        if (k < k_vis) pv(k, std::true_type{});
        if (k + 1 < k_vis) softmax(k + 1, std::true_type{});
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) l[cb] = SPLIT ? mq_sum_groups(l[cb]) : lacc[cb][0];
    bad = false;
#pragma unroll
    for (int w = 0; w < Sh::W; ++w) bad = bad || bad_flags[w] != 0;
}

}  // namespace pa
