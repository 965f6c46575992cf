// Partition kernel for query-head groups of G = 8 with FP8 (E4M3FN) KV and
// bfloat16 queries, head_dim 128: the score and value steps on matrix cores.
//
// With eight query heads sharing each K/V row, a 16-token slice of the
// scores is a 16 x 8 x 128 product and the value update an 8 x 16 x 128
// one: dense enough for v_mfma_f32_16x16x32_bf16.  Both operands are exact
// in bfloat16 (every E4M3FN value is a bfloat16 value; q is bfloat16), so
// the score products are exact and accumulate in float32 as on the vector
// path.  The softmax weights p are float32; for the value product each p is
// split into p_hi = bf16(p) and p_lo = bf16(p - p_hi) and both halves are
// multiplied by the (exact) values, which keeps about 16 significant bits of
// p (relative error below 2^-17), at the cost of a second value MFMA.
//
// Decomposition, staging and merge are those of decode_partition_kernel: one
// workgroup per (sequence, kv head, KV partition), W waves that each stream
// a contiguous share of the partition through a private S-stage LDS ring
// with asynchronous 16-byte copies.  The unit of work is a step of 32 tokens
// (two blocks of 16 or one of 32).
//
// Lane roles (lane = 16 g + n, g = 0..3, n = 0..15).  Columns of every MFMA
// are query heads (n < 8 real, n >= 8 zero), so each lane owns one head:
//   scores   S^T[token][head] = K q^T.  A = K rows, B = q^T.  The lane
//            supplies K row sigma(n) of the 16-token half (sigma transposes
//            the 4 x 4 grid of rows, for conflict-free LDS reads) and the
//            query elements 32 g .. 32 g + 31 of head n; the result gives
//            lane (g, n) the scores of head n for tokens 4 i + g, i = 0..3,
//            of each half.
//   softmax  per head: the lane's 8 scores, then a max across the four lane
//            groups (permlane swaps); the running max is uniform over the
//            head's lanes, the running sum is a per-lane partial summed at
//            the end.
//   values   O^T[dim][head] += V^T P^T.  A = V^T: the lane supplies the
//            value column of its "row" n for the 8 tokens whose scores it
//            holds (read as 32-bit words, 4 columns per word, byte-permuted
//            and widened to bfloat16); B = P^T is exactly the lane's own p.
//            The result gives lane (g, n) head n's accumulators for the 32
//            columns 64 a + 16 g + [0, 16), a = 0, 1; the rescale factor of
//            the online softmax is therefore the lane's own.
//
// LDS layout of a staged step: K rows (32 x 128 bytes) then V rows, each row
// permuted by 16-byte granule.  The copy engine writes lane l's 16 bytes at
// granule l of each 1 KiB copy, so the permutation is applied through each
// lane's source address.  K row t keeps granule x at slot x ^ swk(t), V row t
// at slot x ^ swv(t); swk and swv are chosen so that the reads above spread
// over all banks.
#pragma once

#include "pa_decode_kernel.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, int BS, int W, int S>
struct MfmaShape {
    static constexpr int G = 8;
    static constexpr int UNIT = 32;                 // tokens per step
    static constexpr int BPU = UNIT / BS;           // blocks per step
    static constexpr int ROWB = D;                  // one byte per element
    static constexpr int NG = ROWB / 16;            // 16-byte granules per row
    static constexpr int TILE = BS * ROWB;          // one block's K (or V) tile
    static constexpr int DMA_PER_TILE = TILE / 1024;
    static constexpr int UNIT_BYTES = UNIT * ROWB;  // K (or V) rows of one step
    static constexpr int STAGE = 2 * UNIT_BYTES;
    static constexpr int DMA_PER_UNIT = 2 * UNIT_BYTES / 1024;
    static constexpr int NC = D / 32;               // score MFMAs per 16 tokens
    static constexpr int NA = D / 64;               // value column groups
    static constexpr int RING = S * STAGE;          // per wave
    static constexpr int MERGE_HEAD = ((2 * W * G + W) * 4 + 15) / 16 * 16;
    static constexpr int MERGE = MERGE_HEAD + W * G * D * 4;
    static constexpr int LDS = W * RING > MERGE ? W * RING : MERGE;
    static_assert(D == 128, "the lane roles assume 128-byte rows");
    static_assert(BS == 16 || BS == 32, "block size");
    static_assert(TILE % 1024 == 0, "a tile must be a whole number of 1 KiB wave copies");
    static_assert((S - 1) * DMA_PER_UNIT <= 63, "vmcnt can count at most 63 copies");
    static_assert(LDS <= 160 * 1024, "LDS budget of one CU");
};

// sigma: transpose of the 4 x 4 grid of a half's 16 rows (an involution).
__device__ __forceinline__ int mfma_sigma(int x) { return (x & 3) * 4 + (x >> 2); }
// K granule permutation of row t: makes the 16 rows read by one half-wave
// instruction land on distinct (row parity, slot) pairs.
__device__ __forceinline__ int mfma_swk(int t) {
    const int m = mfma_sigma(t & 15);
    return (m & 7) ^ ((m >> 3) << 2);
}
// V granule permutation of row t: rows 4 i + g of the four lane groups are
// read together; flip the 64-byte half of rows with g in {1, 2}.
__device__ __forceinline__ int mfma_swv(int t) { return ((t ^ (t >> 1)) & 1) << 2; }

// Eight E4M3FN codes (two words) widened exactly to eight bfloat16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return __builtin_bit_cast(bf16x8, r);
}

// Two E4M3FN codes (bytes 0/1, or 2/3 for HI) as a packed bfloat16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Maximum over the four 16-lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float max_over_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

#ifndef PA_MFMA_WAVES_PER_SIMD
#define PA_MFMA_WAVES_PER_SIMD 2
#endif

// COW: the launch also makes its copy-on-write copies (up to COW_MAX_PAIRS
// pairs, no new tokens): the copying workgroups come last in the grid, and a
// partition workgroup reads a destination block from its pair's source,
// checked per block when its copies are issued.
template <int D, int BS, int W, int S, bool COW>
__global__ void __launch_bounds__(W * 64, PA_MFMA_WAVES_PER_SIMD)
decode_partition_mfma8_kernel(const DecodeArgs a) {
    using Sh = MfmaShape<D, BS, W, S>;
    constexpr int G = Sh::G, ROWB = Sh::ROWB, TILE = Sh::TILE, BPU = Sh::BPU, NA = Sh::NA;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    if constexpr (COW) {
        const unsigned parts = (unsigned)a.num_seqs * (unsigned)a.max_partitions * (unsigned)a.num_kv_heads;
        if (blockIdx.x >= parts) {
            cow_copy_block<Fmt::FP8, D, BS, W * 64>(a, blockIdx.x - parts);
            return;
        }
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;   // lane group
    const int n = lane & 15;   // query head of the lane (real for n < G)

    int seq, kvh, part;
    if (!partition_work_item(a, seq, kvh, part)) return;
    const int P = a.partition_size;
    const int lb0 = part * P / BS;
    // Block ids of the partition, one lane per block (up to 64), fetched with
    // the sequence length; part < ceil(max_seq_len / P) keeps lb0 inside the
    // table row, and entries past the sequence's last block are never used.
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq + lb0;
    const int id_lim = min(min(P / BS, 64), a.max_blocks_per_seq - lb0);
    int ids = lane < id_lim ? bt[lane] : 0;
    const int T = load_uniform(a.seq_lens + seq);
    float k_scale = load_uniform(a.k_scale + kvh);
    // the value scale is used only by the final stores; loaded here, with the
    // ids, it adds no memory round trip to the workgroup's end
    float vs = load_uniform(a.v_scale + kvh);
    CowPair pair{{0u, 0u, 0u, 0u}};
    if constexpr (COW) pair = load_cow_pair(a, lane);
    // Query operand: head n's elements 32 g .. 32 g + 31 (zero for n >= G).
    bf16x8 qop[Sh::NC];
    {
        const int hq = kvh * G + (n < G ? n : 0);
        const u32x4* qp =
            (const u32x4*)((const char*)a.q + (((size_t)seq * a.num_heads + hq) * D + 32 * g) * 2);
#pragma unroll
        for (int c = 0; c < Sh::NC; ++c) {
            const u32x4 v = qp[c];
            qop[c] = __builtin_bit_cast(bf16x8, n < G ? v : u32x4{0, 0, 0, 0});
        }
    }
    // make ids and queries resident before any asynchronous copy is queued:
    // the compiler does not see those copies and would otherwise wait for them
    asm volatile("" : "+v"(ids), "+v"(k_scale), "+v"(vs));
#pragma unroll
    for (int c = 0; c < Sh::NC; ++c) asm volatile("" : "+v"(qop[c]));
    int cow_src = -1, cow_dst = -1;
    if constexpr (COW) {
        pin_cow_pair(pair);
        cow_pair_ids(a, pair, lane, cow_src, cow_dst);
    }
    if (T <= 0 || T > a.max_seq_len) return;
    if ((T + BS - 1) / BS > a.max_blocks_per_seq) return;
    const int n_parts = (T + P - 1) / P;
    if (part >= n_parts) return;
    const int tok0 = part * P;
    const int tok1 = min(tok0 + P, T);
    const int nblk = (tok1 - tok0 + BS - 1) / BS;
    const int nunits = (nblk + BPU - 1) / BPU;
    // this wave's steps: a contiguous, balanced share of the partition
    const int u0 = nunits * wave / W;
    const int nuw = nunits * (wave + 1) / W - u0;
    const float qk_scale = a.qk_scale_log2 * k_scale;

    // Source offsets of this lane's 16 bytes in each 1 KiB copy of a K tile
    // and a V tile (the granule permutations depend only on the row inside
    // the tile, the same for both blocks of a 32-token step at BS = 16).
    uint32_t koff[Sh::DMA_PER_TILE], voff[Sh::DMA_PER_TILE];
#pragma unroll
    for (int j = 0; j < Sh::DMA_PER_TILE; ++j) {
        const int pos = 64 * j + lane;
        const int t = pos / Sh::NG;
        const int s = pos % Sh::NG;
        koff[j] = (uint32_t)(t * ROWB + (s ^ mfma_swk(t)) * 16);
        voff[j] = (uint32_t)(t * ROWB + (s ^ mfma_swv(t)) * 16);
    }

    const char* kc = (const char*)a.k_cache;
    const char* vc = (const char*)a.v_cache;
    char* ring = smem + wave * Sh::RING;
    const uint32_t ring_lds = lds_addr_of(smem) + (uint32_t)(wave * Sh::RING);
    int invalid = 0;

    // Issue the copies of step u into ring stage `stage`.  Every step queues
    // the same number of copies (a block past the partition's end re-copies
    // the step's first block, whose rows the mask then drops), so the
    // in-flight counts below stay exact.
    auto issue = [&](int u, int stage) {
        const uint32_t dst = ring_lds + (uint32_t)(stage * Sh::STAGE);
        size_t first = 0;
#pragma unroll
        for (int b = 0; b < BPU; ++b) {
            const int idx = (u0 + u) * BPU + b;  // block index inside the partition
            size_t tile = first;
            if (b == 0 || idx < nblk) {
                int pb = idx < 64 ? __builtin_amdgcn_readlane(ids, idx) : bt[idx];
                if ((unsigned)pb >= (unsigned)a.num_blocks) { invalid = 1; pb = 0; }
                if constexpr (COW) pb = cow_source(cow_src, cow_dst, pb);
                tile = ((size_t)pb * a.num_kv_heads + kvh) * TILE;
                if (b == 0) first = tile;
            }
#pragma unroll
            for (int j = 0; j < Sh::DMA_PER_TILE; ++j)
                dma16_to_lds_stream(kc + tile + koff[j], dst + b * TILE + j * 1024);
#pragma unroll
            for (int j = 0; j < Sh::DMA_PER_TILE; ++j)
                dma16_to_lds_stream(vc + tile + voff[j], dst + Sh::UNIT_BYTES + b * TILE + j * 1024);
        }
    };

    // per-lane state of head n: running max (uniform over the head's lanes),
    // partial sum, and accumulators acc[a][b][i] for column 64a + 16g + 4i + b
    float m = -INFINITY, l = 0.f;
    f32x4 acc[NA][4];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[aa][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS read offsets that do not depend on the step
    const int krow = mfma_sigma(n);            // K row read for A (per half)
    const int kslot0 = (2 * g) ^ mfma_swk(krow);
    const int kslot1 = (2 * g + 1) ^ mfma_swk(krow);
    const int vsw = mfma_swv(g);               // rows 4 i + g share bits 0..1 with g

    auto step = [&](const char* st, int utok0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const char* kb = st;
        const char* vb = st + Sh::UNIT_BYTES;
        // ---- scores of both 16-token halves: sc[h][i] is token 16h + 4i + g
        f32x4 sc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const char* rowp = kb + (16 * h + krow) * ROWB;
            const u32x4 k0 = *(const u32x4*)(rowp + kslot0 * 16);
            const u32x4 k1 = *(const u32x4*)(rowp + kslot1 * 16);
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k0.x, k0.y), qop[0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k0.z, k0.w), qop[1], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k1.x, k1.y), qop[2], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k1.z, k1.w), qop[3], c, 0, 0, 0);
            sc[h] = c;
        }
        float s[2][4];
        bool ok[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ok[h][i] = !MASKED || utok0 + 16 * h + 4 * i + g < tok1;
                s[h][i] = ok[h][i] ? mul_rounded(sc[h][i], qk_scale) : -INFINITY;
            }
        // ---- online softmax of head n
        float mx = s[0][0];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[h][i]);
        mx = max_over_groups(mx);
        const float mn = fmaxf(m, mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        if (__builtin_amdgcn_ballot_w64(mn != m) != 0) {
            const float alpha = fast_exp2(m - mu);
            l *= alpha;
#pragma unroll
            for (int aa = 0; aa < NA; ++aa)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[aa][b] *= alpha;
        }
        m = mn;
        bf16x8 phi, plo;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[h][i] - mu);
                l += p;
                const __bf16 ph = (__bf16)p;
                phi[4 * h + i] = ph;
                plo[4 * h + i] = (__bf16)(p - (float)ph);
            }
        // ---- values: word (16 a + n) of rows 16h + 4i + g, i.e. columns
        // 64 a + 4 n + b for b = 0..3, one MFMA per (a, b)
#pragma unroll
        for (int aa = 0; aa < NA; ++aa) {
            const int voffs = ((4 * aa + (n >> 2)) ^ vsw) * 16 + (n & 3) * 4;
            uint32_t w[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    w[h][i] = *(const uint32_t*)(vb + (16 * h + 4 * i + g) * ROWB + voffs);
                    if constexpr (MASKED) w[h][i] = ok[h][i] ? w[h][i] : 0u;
                }
            u32x4 vop[4];  // [b]: element 4h + i is byte b of w[h][i]
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ip = 0; ip < 2; ++ip) {
                    const uint32_t w0 = w[h][2 * ip], w1 = w[h][2 * ip + 1];
                    const uint32_t x = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // b0 b0' b1 b1'
                    const uint32_t y = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // b2 b2' b3 b3'
                    vop[0][2 * h + ip] = fp8x2_to_bf16x2<false>(x);
                    vop[1][2 * h + ip] = fp8x2_to_bf16x2<true>(x);
                    vop[2][2 * h + ip] = fp8x2_to_bf16x2<false>(y);
                    vop[3][2 * h + ip] = fp8x2_to_bf16x2<true>(y);
                }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16x8 A = __builtin_bit_cast(bf16x8, vop[b]);
                acc[aa][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, phi, acc[aa][b], 0, 0, 0);
                acc[aa][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, plo, acc[aa][b], 0, 0, 0);
            }
        }
    };

    // ---- main loop: S-stage ring, S-1 steps of copies ahead of compute
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        if (k < nuw) issue(k, k);
    int stage = 0;
    for (int k = 0; k < nuw; ++k) {
        if (k + S - 1 < nuw) issue(k + S - 1, stage == 0 ? S - 1 : stage - 1);
        wait_blocks_in_flight<Sh::DMA_PER_UNIT, S - 1>(min(S - 1, nuw - 1 - k));
        const char* st = ring + stage * Sh::STAGE;
        const int utok0 = tok0 + (u0 + k) * Sh::UNIT;
        if (utok0 + Sh::UNIT <= tok1)
            step(st, utok0, std::false_type{});
        else
            step(st, utok0, std::true_type{});
        stage = stage + 1 == S ? 0 : stage + 1;
    }

    // ---- merge: the lane groups' partial sums, then the waves by log-sum-exp
    {
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
    }
    __syncthreads();  // every wave is done with its ring; reuse the LDS
    float* wm = (float*)smem;
    float* wl = wm + W * G;
    int* winv = (int*)(wl + W * G);
    float* wacc = (float*)(smem + Sh::MERGE_HEAD);  // [W][G][D]
    if (lane == 0) winv[wave] = invalid;
    if (n < G) {
        if (g == 0) { wm[wave * G + n] = m; wl[wave * G + n] = l; }
        // granule x (columns 4x .. 4x + 3) of head n's row sits at x ^ n, so
        // that the eight heads' stores of one instruction spread over the banks
        float* dst = wacc + (wave * G + n) * D;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(float4*)(dst + ((16 * aa + 4 * g + i) ^ n) * 4) =
                    float4{acc[aa][0][i], acc[aa][1][i], acc[aa][2][i], acc[aa][3][i]};
    }
    __syncthreads();
    int bad = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) bad |= winv[w];
    const int hq0 = kvh * G;
    auto merged_m = [&](int hg) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, wm[w * G + hg]);
        return M;
    };
    if (n_parts > 1 && wave == 0) {
        auto merged_l = [&](int hg) {
            const float M = merged_m(hg);
            const float mu = M == -INFINITY ? 0.f : M;
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) L = fmaf(fast_exp2(wm[w * G + hg] - mu), wl[w * G + hg], L);
            return L;
        };
        // ordinary stores: 1.2% faster than non-temporal ones for the
        // records (long_fp8), the opposite of the acc rows below
        store_ml_record<G, false>(a.part_ml + ml_record(a, seq, kvh, part), lane, bad != 0, merged_m, merged_l);
    }
    // four consecutive dims per thread, so that each state row leaves in
    // 16-byte stores (granule x of head hg's row sits at x ^ hg)
    for (int o4 = threadIdx.x; o4 < G * D / 4; o4 += W * 64) {
        const int hg = o4 / (D / 4);
        const int d0 = 4 * (o4 - hg * (D / 4));
        const float M = merged_m(hg);
        const float mu = M == -INFINITY ? 0.f : M;
        float L = 0.f;
        f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = fast_exp2(wm[w * G + hg] - mu);
            L = fmaf(f, wl[w * G + hg], L);
            const f32x4 v = *(const f32x4*)(wacc + (w * G + hg) * D + (d0 ^ (hg << 2)));
#pragma unroll
            for (int e = 0; e < 4; ++e) A[e] = fmaf(f, v[e], A[e]);
        }
        const size_t row = (size_t)seq * a.num_heads + hq0 + hg;
        const float nan = __builtin_nanf("");
        if (n_parts == 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) store_out(a.out, a.out_dtype, row * D + d0 + e, bad ? nan : A[e] / L * vs);
        } else {
            const size_t pidx = row * a.max_partitions + part;
            f32x4 st;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[e] = bad ? nan : A[e] * vs;
            __builtin_nontemporal_store(st, (f32x4*)(a.part_acc + pidx * D + d0));
        }
    }
}

template <int D, int BS, int W, int S, bool COW>
int launch_partition_mfma8_as(const DecodeArgs& a, hipStream_t stream) {
    using Sh = MfmaShape<D, BS, W, S>;
    auto kernel = decode_partition_mfma8_kernel<D, BS, W, S, COW>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const size_t copies = COW ? 2 * (size_t)a.cow_num * cow_chunks<Fmt::FP8, D, BS, W * 64>(a.num_kv_heads) : 0;
    const dim3 grid((unsigned)(copies + (size_t)a.num_seqs * a.max_partitions * a.num_kv_heads));
    hipLaunchKernelGGL(kernel, grid, dim3(W * 64), Sh::LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// The copy-on-write instantiation when the launch carries pairs (never with
// new tokens: this kernel does not store them).
template <int D, int BS, int W, int S>
int launch_partition_mfma8(const DecodeArgs& a, hipStream_t stream) {
    if (a.new_k != nullptr) return PA_ERR_UNSUPPORTED;
    return a.cow_num > 0 ? launch_partition_mfma8_as<D, BS, W, S, true>(a, stream)
                         : launch_partition_mfma8_as<D, BS, W, S, false>(a, stream);
}

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 2
#endif
#ifndef PA_MFMA_STAGES
#define PA_MFMA_STAGES 2
#endif

// FP8 KV, bfloat16 queries, G = 8: head_dim 128 only (others use the vector
// kernel).  Returns PA_ERR_UNSUPPORTED for shapes it does not cover.
inline int dispatch_mfma8(const DecodeArgs& a, int head_dim, hipStream_t stream) {
    constexpr int W = PA_MFMA_WAVES, S = PA_MFMA_STAGES;
    if (head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (a.block_size == 16) return launch_partition_mfma8<128, 16, W, S>(a, stream);
    if (a.block_size == 32) return launch_partition_mfma8<128, 32, W, S>(a, stream);
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
