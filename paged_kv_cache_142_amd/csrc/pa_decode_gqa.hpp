// Partition kernel for query-head groups of G = 4 with 16-bit KV (bf16/fp16).
//
// Same decomposition, staging and merge as decode_partition_kernel (one
// workgroup per (sequence, kv head, KV partition); each wave streams its
// blocks' K/V tiles into a private LDS ring with asynchronous 16-byte
// copies), but the score step puts the G query heads into lanes instead of
// reducing every dot product across lanes:
//
//   score layout   lane = (head h, token tq, half), tq fastest:
//                  lane = h*16 + half*8 + tq.  The lane holds head h's query
//                  elements of its half of the row (64 dims) and computes the
//                  half dot product for token tq of the pass; one DPP
//                  rotate-add joins the two halves.  Two passes of 8 tokens
//                  cover a 16-token chunk.  The G heads read the same K rows
//                  (LDS broadcast), so each staged tile serves the whole group.
//   K tile in LDS  XOR-swizzled by 16-byte granule: row t's granule g lives
//                  at granule t*NG + (g ^ (t mod NG)).  The copy engine writes
//                  lane l's 16 bytes at granule l of each 1 KiB copy, so the
//                  swizzle is applied by choosing each lane's source address;
//                  reads of 8 different rows at one logical granule then hit
//                  8 different bank groups.
//   softmax        the running max m and sum l are per head and uniform over
//                  the wave: per chunk a 3-step DPP max and sum over the 8
//                  token lanes of the head, one exp2 per score and one for the
//                  rescale factor alpha = 2^(m - m').
//   value layout   as in decode_partition_kernel (lane = token row r, column
//                  c of 8 elements, all G heads per lane); p[t][h] and alpha[h]
//                  reach it through a 272-byte per-wave LDS scratch.  acc is
//                  rescaled only when some head's max moved (wave-uniform test).
//
// At the end the R row subsets and W waves are summed through LDS (the row
// subsets share the wave's per-head max; waves are merged with the
// log-sum-exp rule).
#pragma once

#include "pa_decode_kernel.hpp"

namespace pa {

template <Fmt KV, int D, int BS, int W, int S>
struct GqaShape {
    static constexpr int G = 4;
    static constexpr int EB = 2;
    static constexpr int NG = D * EB / 16;   // 16-byte granules per token row
    static constexpr int ROWB = D * EB;
    static constexpr int TILE = BS * ROWB;
    static constexpr int DMA_PER_TILE = TILE / 1024;
    static constexpr int DMA_PER_BLOCK = 2 * DMA_PER_TILE;
    static constexpr int STAGE = 2 * TILE;
    static constexpr int TQ = 8;             // tokens per score pass
    static constexpr int HALF_G = NG / 2;    // granules per half row
    static constexpr int QW = HALF_G * 4;    // 32-bit query words per lane
    static constexpr int NPASS = 16 / TQ;
    static constexpr int R = 64 / NG;        // value-layout token rows per pass
    static constexpr int VPASS = 16 / R;
    static constexpr int SCRATCH = 512;      // p[16][G] + alpha[G], padded
    static constexpr int QBYTES = G * D * 2; // the group's query rows
    static constexpr int RING = S * STAGE + SCRATCH + QBYTES;
    static constexpr int MERGE_HEAD = ((2 * W * G + W) * 4 + 15) / 16 * 16;
    static constexpr int MERGE = MERGE_HEAD + W * R * G * D * 4;
    static constexpr int LDS = (W * RING > MERGE) ? W * RING : MERGE;
    static constexpr int NEWROW = 2 * ROWB;           // an appended token's K and V rows, per wave
    static constexpr int LDS_APPEND = LDS + W * NEWROW;  // after everything else
    static_assert(TILE % 1024 == 0, "a tile must be a whole number of 1 KiB wave copies");
    static_assert((S - 1) * DMA_PER_BLOCK <= 63, "vmcnt can count at most 63 copies");
    static_assert(LDS_APPEND <= 160 * 1024, "LDS budget of one CU");
    static_assert(G * 2 * TQ == 64, "lane decomposition");
};

template <Fmt KV>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float c) {
    if constexpr (KV == Fmt::BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                               false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true)));
}

#ifndef PA_GQA_WAVES_PER_SIMD
#define PA_GQA_WAVES_PER_SIMD 3
#endif

// At most this many waves per SIMD in the launch bound (3 caps registers at 168).
// Waves per SIMD that the LDS lets a CU hold for this shape, at most
// PA_GQA_WAVES_PER_SIMD: the register budget of the launch bound.  Asking for
// more than the LDS allows would only cap registers (and make the compiler
// spill) without adding a wave.
template <Fmt KV, int D, int BS, int W, int S>
constexpr int gqa_waves_per_simd() {
    constexpr int per_cu = (160 * 1024) / GqaShape<KV, D, 16, W, S>::LDS_APPEND * W / 4;
    return per_cu < 1 ? 1 : per_cu > PA_GQA_WAVES_PER_SIMD ? PA_GQA_WAVES_PER_SIMD : per_cu;
}

// The partition workgroup's work, for workgroup bid of the partition grid
// (the kernel below passes its block index; the shared-prefix launch runs it
// after its own workgroups).
template <Fmt KV, int D, int BS, int W, int S, bool APPEND>
__device__ __forceinline__ void gqa4_partition(const DecodeArgs& a, unsigned bid) {
    // Tiles are staged 16 rows at a time whatever the pool's block size BS:
    // a 32-token block is two 16-row halves, each a contiguous tile.
    using Sh = GqaShape<KV, D, 16, W, S>;
    constexpr int HALVES = BS / 16;
    constexpr size_t POOL_TILE = (size_t)BS * D * 2;  // one (block, kv head) tile of the pool
    using Row = LaneRow<KV, D>;
    constexpr int G = Sh::G, NG = Sh::NG, ROWB = Sh::ROWB, TILE = Sh::TILE, TQ = Sh::TQ, R = Sh::R;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // score layout
    const int tq = lane & (TQ - 1);
    const int half = (lane >> 3) & 1;
    const int hl = lane >> 4;
    // value layout
    const int r = lane / NG;
    const int c = lane % NG;

    int seq, kvh, part;
    if (!partition_work_item(a, bid, seq, kvh, part)) return;
    const int P = a.partition_size;
    const int lb0 = part * P / BS;  // first logical block of the partition
    // Block ids of the whole partition, fetched together with the sequence
    // length (one lane per block, up to 64).  The read is in bounds of the
    // table row: part < ceil(max_seq_len / P), so lb0 < max_blocks_per_seq;
    // entries past the sequence's last block are loaded but never used.
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq + lb0;
    const int id_lim = min(min(P / BS, 64), a.max_blocks_per_seq - lb0);
    int ids = lane < id_lim ? bt[lane] : 0;
    const int T = load_uniform(a.seq_lens + seq);
    // copy-on-write pairs of this launch (decode with append only), one per
    // lane; -1 for lanes past them and for pairs outside the pool, which are
    // skipped as by pa_copy_blocks
    const bool cow = APPEND && a.cow_num > 0;
    CowPair pair{{0u, 0u, 0u, 0u}};
    if constexpr (APPEND) pair = load_cow_pair(a, lane);
    // wait for the ids here, together with the length: the compiler does not
    // see the asynchronous copies below and would otherwise wait for them too
    asm volatile("" : "+v"(ids));
    if constexpr (APPEND) pin_cow_pair(pair);
    int cow_src = -1, cow_dst = -1;
    if constexpr (APPEND) cow_pair_ids(a, pair, lane, cow_src, cow_dst);
    // A block that a pair of this launch overwrites is read from the pair's
    // source, which holds the same content once copied (the copying
    // workgroups run beside this one).  Each block id is checked when its
    // copy is issued (one compare of the pair lanes against it), so that
    // nothing stands between the ids' arrival and the first copies.  When
    // the sequence's last block is a destination, its copying workgroup
    // writes the new token into it, and this workgroup stores nothing there.
    auto source_of = [&](int pb) { return cow ? cow_source(cow_src, cow_dst, pb) : pb; };
    if (T <= 0 || T > a.max_seq_len) return;
    if ((T + BS - 1) / BS > a.max_blocks_per_seq) return;
    const int n_parts = (T + P - 1) / P;
    if (part >= n_parts) return;
    const int tok0 = part * P;
    const int tok1 = min(tok0 + P, T);
    const int nblk = (tok1 - tok0 + 15) / 16;  // 16-row tiles of the partition (blocks when BS = 16)
    // this wave's blocks: a contiguous, balanced share of the partition
    const int kb0 = nblk * wave / W;
    const int nbw = nblk * (wave + 1) / W - kb0;
    const int hq0 = kvh * G;
    const float qk_scale = a.qk_scale_log2;

    // Decode with append: the wave that stages the sequence's last block
    // copies the newest token's K and V rows of this kv head to LDS with its
    // first copies, writes them over that row of the staged tile once the tile
    // has landed, and stores them into the pool.  The attention thus never
    // depends on when the store reaches memory.
    const bool appends = APPEND && part == n_parts - 1 && nbw > 0 && kb0 + nbw == nblk;
    const int new_row = (T - 1) % 16;  // row of the newest token in its staged tile

    // Source offset of this lane's 16 bytes in each 1 KiB copy of a K tile
    // (swizzled) and a V tile (natural order); the same for every block.
    uint32_t koff[Sh::DMA_PER_TILE];
#pragma unroll
    for (int j = 0; j < Sh::DMA_PER_TILE; ++j) {
        const int pos = 64 * j + lane;
        const int t = pos / NG;
        const int g = (pos % NG) ^ (t & (NG - 1));
        koff[j] = (uint32_t)(t * ROWB + g * 16);
    }

    const char* kc = (const char*)a.k_cache;
    const char* vc = (const char*)a.v_cache;
    char* ring = smem + wave * Sh::RING;
    float* p_lds = (float*)(ring + S * Sh::STAGE);  // [16][G]
    float* alpha_lds = p_lds + 16 * G;                   // [G]
    const char* q_lds = ring + S * Sh::STAGE + Sh::SCRATCH;  // [G][D] query elements
    const uint32_t ring_lds = lds_addr_of(smem) + (uint32_t)(wave * Sh::RING);
    int invalid = 0;

    // The group's query rows go to LDS with the same asynchronous copies, ahead
    // of the first block; they are read into registers once that block landed.
    if (nbw > 0 && lane * 16 < Sh::QBYTES)
        dma16_to_lds((const char*)a.q + ((size_t)seq * a.num_heads + hq0) * D * 2 + lane * 16,
                     ring_lds + (uint32_t)(S * Sh::STAGE + Sh::SCRATCH));
    const char* new_lds = smem + Sh::LDS + wave * Sh::NEWROW;  // [K row][V row]
    if (appends && lane < NG) {
        const size_t src = ((size_t)seq * a.num_kv_heads + kvh) * ROWB + lane * 16;
        const uint32_t at = lds_addr_of(smem) + (uint32_t)(Sh::LDS + wave * Sh::NEWROW);
        dma16_to_lds((const char*)a.new_k + src, at);
        dma16_to_lds((const char*)a.new_v + src, at + ROWB);
    }
    uint32_t qw[Sh::QW];
    auto load_q = [&]() {
        const char* qrow = q_lds + (hl * D + half * (D / 2)) * 2;
#pragma unroll
        for (int i = 0; i < Sh::HALF_G; ++i) {
            const u32x4 v = *(const u32x4*)(qrow + i * 16);
            qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
        }
    };

    auto issue = [&](int k, int stage) {
        const int vidx = kb0 + k;         // 16-row tile inside the partition
        const int idx = vidx / HALVES;    // its block inside the partition
        // a uniform id (kept in a scalar register: a vector register that a
        // pending table load may still write would make later copies wait)
        int pb = idx < 64 ? __builtin_amdgcn_readlane(ids, idx) : __builtin_amdgcn_readfirstlane(bt[idx]);
        if ((unsigned)pb >= (unsigned)a.num_blocks) { invalid = 1; pb = 0; }
        pb = source_of(pb);
        size_t tile = ((size_t)pb * a.num_kv_heads + kvh) * POOL_TILE;
        if constexpr (HALVES > 1) tile += (size_t)(vidx % HALVES) * TILE;
        const uint32_t dst = ring_lds + (uint32_t)(stage * Sh::STAGE);
#pragma unroll
        for (int j = 0; j < Sh::DMA_PER_TILE; ++j) dma16_to_lds_stream(kc + tile + koff[j], dst + j * 1024);
#pragma unroll
        for (int j = 0; j < Sh::DMA_PER_TILE; ++j)
            dma16_to_lds_stream(vc + tile + (size_t)j * 1024 + lane * 16, dst + TILE + j * 1024);
    };

    float m = -INFINITY, l = 0.f;  // per head hl (uniform over its 16 lanes)
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

    auto chunk = [&](const char* stage_ptr, int ch, int row_tok0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        // ---- scores: lane (hl, half, tq), passes of TQ tokens
        float s[Sh::NPASS];
#pragma unroll
        for (int p = 0; p < Sh::NPASS; ++p) {
            const int t = ch * 16 + p * TQ + tq;  // row inside the block
            const char* rowp = stage_ptr + t * ROWB;
            float c0 = 0.f, c1 = 0.f;
#pragma unroll
            for (int i = 0; i < Sh::HALF_G; ++i) {
                const int g = half * Sh::HALF_G + i;
                const u32x4 kv = *(const u32x4*)(rowp + ((g ^ (t & (NG - 1))) * 16));
                float& cc = (i & 1) ? c1 : c0;
                cc = dot2_acc<KV>(qw[4 * i], kv.x, cc);
                cc = dot2_acc<KV>(qw[4 * i + 1], kv.y, cc);
                cc = dot2_acc<KV>(qw[4 * i + 2], kv.z, cc);
                cc = dot2_acc<KV>(qw[4 * i + 3], kv.w, cc);
            }
            float sp = c0 + c1;
            sp += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sp), 0x128, 0xf, 0xf, true));  // row_ror:8
            sp = mul_rounded(sp, qk_scale);
            if constexpr (MASKED) sp = (row_tok0 + p * TQ + tq < T) ? sp : -INFINITY;
            s[p] = sp;
        }
        // ---- online softmax per head (the 8 token lanes of each half agree)
        float mx = s[0];
#pragma unroll
        for (int p = 1; p < Sh::NPASS; ++p) mx = fmaxf(mx, s[p]);
        mx = dpp_max<0xB1>(mx);
        mx = dpp_max<0x4E>(mx);
        mx = dpp_max<0x141>(mx);
        const float mn = fmaxf(m, mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        float psum = 0.f;
        float pv[Sh::NPASS];
#pragma unroll
        for (int p = 0; p < Sh::NPASS; ++p) { pv[p] = fast_exp2(s[p] - mu); psum += pv[p]; }
        psum = group_sum<8>(psum);
        l = fmaf(l, alpha, psum);
        const bool moved = mn != m;
        m = mn;
        if (half == 0) {
#pragma unroll
            for (int p = 0; p < Sh::NPASS; ++p) p_lds[(p * TQ + tq) * G + hl] = pv[p];
            if (tq == 0) alpha_lds[hl] = alpha;
        }
        const bool rescale = __builtin_amdgcn_ballot_w64(moved) != 0;
        // ---- values: lane (r, c), all heads
        const char* vb = stage_ptr + TILE + ch * 16 * ROWB;
        if (rescale) {
            const float4 al = *(const float4*)alpha_lds;
            const float alg[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] *= alg[g];
        }
#pragma unroll
        for (int j = 0; j < Sh::VPASS; ++j) {
            const int tr = j * R + r;
            const float4 pp = *(const float4*)(p_lds + tr * G);
            uint32_t vw[Row::NW];
            Row::load(vb + tr * ROWB, c, vw);
            float v[8];
            Row::to_f32(vw, v);
            if constexpr (MASKED) {
                const bool ok = row_tok0 + tr < T;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = ok ? v[e] : 0.f;
            }
            const float pg[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pg[g], v[e], acc[g][e]);
        }
    };

    // ---- main loop
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        if (k < nbw) issue(k, k);
    int stage = 0;
    for (int k = 0; k < nbw; ++k) {
        if (k + S - 1 < nbw) issue(k + S - 1, stage == 0 ? S - 1 : stage - 1);
        wait_blocks_in_flight<Sh::DMA_PER_BLOCK, S - 1>(min(S - 1, nbw - 1 - k));
        if (k == 0) load_q();
        if (appends && k == nbw - 1) {
            // the host appends here only when a partition has at most 64 blocks
            const int last = min((nblk - 1) / HALVES, 63);
            const int pb = __builtin_amdgcn_readlane(ids, last);
            const bool stores = source_of(pb) == pb;  // else the copying workgroup does
            if (lane < NG) {
                const u32x4 kg = *(const u32x4*)(new_lds + lane * 16);
                const u32x4 vg = *(const u32x4*)(new_lds + ROWB + lane * 16);
                char* row = ring + stage * Sh::STAGE + new_row * ROWB;
                *(u32x4*)(row + ((lane ^ (new_row & (NG - 1))) * 16)) = kg;  // K granules are swizzled
                *(u32x4*)(row + TILE + lane * 16) = vg;
                if (stores && (unsigned)pb < (unsigned)a.num_blocks) {
                    const size_t dst = ((size_t)pb * a.num_kv_heads + kvh) * POOL_TILE + ((T - 1) % BS) * ROWB + lane * 16;
                    *(u32x4*)((char*)a.k_cache + dst) = kg;
                    *(u32x4*)((char*)a.v_cache + dst) = vg;
                }
            }
        }
        const char* sp = ring + stage * Sh::STAGE;
        const int blk_tok0 = (lb0 * HALVES + kb0 + k) * 16;
        // one 16-row chunk per staged tile (kept as a loop: the same code as
        // the chunk loop of a full block, which the compiler schedules best)
        if (blk_tok0 + 16 <= T) {
#pragma unroll
            for (int ch = 0; ch < 16 / 16; ++ch) chunk(sp, ch, blk_tok0 + ch * 16, std::false_type{});
        } else {
#pragma unroll
            for (int ch = 0; ch < 16 / 16; ++ch) chunk(sp, ch, blk_tok0 + ch * 16, std::true_type{});
        }
        stage = stage + 1 == S ? 0 : stage + 1;
    }

    // ---- merge: rows of a wave share its per-head max; waves by log-sum-exp
    __syncthreads();
    float* wm = (float*)smem;
    float* wl = wm + W * G;
    int* winv = (int*)(wl + W * G);
    float* wacc = (float*)(smem + Sh::MERGE_HEAD);  // [W*R][G][D]
    if (lane == 0) winv[wave] = invalid;
    if (half == 0 && tq == 0) { wm[wave * G + hl] = m; wl[wave * G + hl] = l; }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float* row = wacc + ((wave * R + r) * G + g) * D;
        *(float4*)(row + merge_pos(Row::dim(c, 0))) = float4{acc[g][0], acc[g][1], acc[g][2], acc[g][3]};
        *(float4*)(row + merge_pos(Row::dim(c, 4))) = float4{acc[g][4], acc[g][5], acc[g][6], acc[g][7]};
    }
    __syncthreads();
    int bad = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) bad |= winv[w];
    // two consecutive dims per thread, so that each row leaves in 8-byte
    // stores (merge_pos keeps pairs of dims together)
    for (int o2 = threadIdx.x; o2 < G * D / 2; o2 += W * 64) {
        const int g = o2 / (D / 2);
        const int d0 = 2 * (o2 - g * (D / 2));
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, wm[w * G + g]);
        const float mu = M == -INFINITY ? 0.f : M;
        float L = 0.f;
        f32x2 A = {0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = fast_exp2(wm[w * G + g] - mu);
            f32x2 rows = {0.f, 0.f};
#pragma unroll
            for (int rr = 0; rr < R; ++rr) rows += *(const f32x2*)(wacc + ((w * R + rr) * G + g) * D + merge_pos(d0));
            L = fmaf(f, wl[w * G + g], L);
            A[0] = fmaf(f, rows[0], A[0]);
            A[1] = fmaf(f, rows[1], A[1]);
        }
        const int hq = hq0 + g;
        const size_t row = (size_t)seq * a.num_heads + hq;
        const float nan = __builtin_nanf("");
        if (n_parts == 1) {
            store_out(a.out, a.out_dtype, row * D + d0, bad ? nan : A[0] / L);
            store_out(a.out, a.out_dtype, row * D + d0 + 1, bad ? nan : A[1] / L);
        } else {
            const size_t pidx = row * a.max_partitions + part;
            if (d0 == 0) {
                store_state(&a.part_m[pidx], bad ? nan : M);
                store_state(&a.part_l[pidx], bad ? nan : L);
            }
            *(f32x2*)(a.part_acc + pidx * D + d0) = bad ? f32x2{nan, nan} : A;
        }
    }
}

template <Fmt KV, int D, int BS, int W, int S, bool APPEND>
__global__ void __launch_bounds__(W * 64, (gqa_waves_per_simd<KV, D, BS, W, S>()))
decode_partition_gqa4_kernel(const DecodeArgs a) {
    if constexpr (APPEND) {
        // decode with append: the copy-on-write pairs' workgroups come last,
        // where the tail of the partition work leaves slots idle (nothing here
        // reads their destinations)
        const unsigned parts = (unsigned)a.num_seqs * (unsigned)a.max_partitions * (unsigned)a.num_kv_heads;
        if (blockIdx.x >= parts) {
            cow_copy_block<KV, D, BS, W * 64>(a, blockIdx.x - parts);
            return;
        }
        gqa4_partition<KV, D, BS, W, S, APPEND>(a, blockIdx.x);
    } else {
        gqa4_partition<KV, D, BS, W, S, APPEND>(a, blockIdx.x);
    }
}

template <Fmt KV, int D, int BS, int W, int S, bool APPEND>
int launch_partition_gqa4_as(const DecodeArgs& a, hipStream_t stream) {
    using Sh = GqaShape<KV, D, 16, W, S>;  // staged 16 rows at a time
    constexpr int LDS = APPEND ? Sh::LDS_APPEND : Sh::LDS;
    auto kernel = decode_partition_gqa4_kernel<KV, D, BS, W, S, APPEND>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const size_t copies = APPEND ? 2 * (size_t)a.cow_num * cow_chunks<KV, D, BS, W * 64>(a.num_kv_heads) : 0;
    const dim3 grid((unsigned)(copies + (size_t)a.num_seqs * a.max_partitions * a.num_kv_heads));
    hipLaunchKernelGGL(kernel, grid, dim3(W * 64), LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// The plain kernel, or the one that also stores the new tokens (decode with
// append): separate instantiations, so that the plain one carries none of it.
template <Fmt KV, int D, int BS, int W, int S>
int launch_partition_gqa4(const DecodeArgs& a, hipStream_t stream) {
    return a.new_k != nullptr ? launch_partition_gqa4_as<KV, D, BS, W, S, true>(a, stream)
                              : launch_partition_gqa4_as<KV, D, BS, W, S, false>(a, stream);
}

#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 4
#endif
#ifndef PA_GQA_STAGES
#define PA_GQA_STAGES 2
#endif

template <Fmt KV>
int dispatch_gqa4(const DecodeArgs& a, int head_dim, hipStream_t stream) {
    constexpr int W = PA_GQA_WAVES, S = PA_GQA_STAGES;
    const int bs = a.block_size;
    if (head_dim == 128 && bs == 16) return launch_partition_gqa4<KV, 128, 16, W, S>(a, stream);
    if (head_dim == 128 && bs == 32) return launch_partition_gqa4<KV, 128, 32, W, S>(a, stream);
    if (head_dim == 64 && bs == 16) return launch_partition_gqa4<KV, 64, 16, W, S>(a, stream);
    if (head_dim == 64 && bs == 32) return launch_partition_gqa4<KV, 64, 32, W, S>(a, stream);
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
