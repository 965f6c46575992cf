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
// Work decomposition: the unit of work is one (sequence, kv head, KV
// partition), as in decode_partition_kernel, but the workgroups are
// persistent: the grid holds as many workgroups as the CUs keep resident, and
// workgroup b takes units b, 2N-1-b, 2N+b, ... of the largest-first order the
// plan kernel writes (a snake over rounds of N = gridDim.x units).  Each of
// the W waves streams a contiguous share of a unit's 32-token steps (two
// blocks of 16 or one of 32) through a private two-stage LDS ring with
// asynchronous 16-byte copies.  The copies run ahead across units: during the
// last step of a unit the wave already issues the first step of its next
// unit (and that unit's queries), and the block ids of the next unit are
// copied into LDS a whole unit ahead, so the stream does not stop while the
// waves merge a unit's results and write them out.
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

template <int D, int BS, int W>
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
    static constexpr int RING = 2 * STAGE;          // two stages per wave
    static constexpr int QBYTES = G * D * 2;        // the unit's query rows
    static constexpr int QOPS = QBYTES / 1024;      // their 1 KiB copies
    static constexpr int IDS = 2 * 64 * 4;          // block ids, two units
    static constexpr int WAVE_LDS = RING + QBYTES + IDS;
    static constexpr int STATE_ML = G * D * 4;      // offset of m, l in a state
    static constexpr int META = 2 * W * 4;          // free stage and invalid flag per wave
    static constexpr int LDS = W * WAVE_LDS + META;
    static_assert(D == 128, "the lane roles assume 128-byte rows");
    static_assert(BS == 16 || BS == 32, "block size");
    static_assert(TILE % 1024 == 0, "a tile must be a whole number of 1 KiB wave copies");
    static_assert(DMA_PER_UNIT + QOPS <= 63, "vmcnt can count at most 63 copies");
    static_assert(STATE_ML + 2 * G * 4 <= STAGE, "a wave's merge state fits in one ring stage");
    static_assert(QBYTES % 1024 == 0, "query rows are whole 1 KiB copies");
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

template <int D, int BS, int W>
__global__ void __launch_bounds__(W * 64, PA_MFMA_WAVES_PER_SIMD)
decode_partition_mfma8_kernel(const DecodeArgs a) {
    using Sh = MfmaShape<D, BS, W>;
    constexpr int G = Sh::G, ROWB = Sh::ROWB, TILE = Sh::TILE, BPU = Sh::BPU, NA = Sh::NA;
    constexpr int DPU = Sh::DMA_PER_UNIT;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;   // lane group
    const int n = lane & 15;   // query head of the lane (real for n < G)
    const int P = a.partition_size;
    const int H = a.num_kv_heads;
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;

    // ---- this workgroup's units: r-th is round r of the snake
    const int units = a.plan[0] * H;
    const int full = units / nwg;
    const int rem = units - full * nwg;
    const int R = full + ((((full & 1) ? nwg - 1 - wg : wg) < rem) ? 1 : 0);
    if (R == 0) return;
    auto unit_of = [&](int r) { return r * nwg + ((r & 1) ? nwg - 1 - wg : wg); };

    // Plan entries, lengths and kv-head scales of 64 consecutive units, one
    // per lane (reloaded every 64 units).  Everything a unit needs besides its
    // block ids and queries comes from here, so the loop below has no loads
    // the compiler would have to wait for.
    int tab_code = 0, tab_len = 0;
    float tab_ks = 0.f, tab_vs = 0.f;
    auto load_tables = [&](int r0) {
        const int r = r0 + lane;
        const int w = r < R ? unit_of(r) : 0;
        const int code = r < R ? a.plan[PLAN_ITEMS_OFFSET + w / H] : 0;
        tab_ks = r < R ? a.k_scale[w % H] : 0.f;
        tab_vs = r < R ? a.v_scale[w % H] : 0.f;
        tab_len = r < R ? a.seq_lens[code / a.max_partitions] : 0;
        tab_code = code;
    };

    struct Unit {
        int seq, kvh, part, n_parts, tok0, tok1, nblk, u0, nuw;
        float ks, vs;
    };
    auto make_unit = [&](int r) {
        Unit u;
        const int w = unit_of(r);
        const int item = w / H;
        u.kvh = w - item * H;
        const int code = __builtin_amdgcn_readlane(tab_code, r & 63);
        const int T = __builtin_amdgcn_readlane(tab_len, r & 63);
        u.ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_ks), r & 63));
        u.vs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_vs), r & 63));
        u.seq = code / a.max_partitions;
        u.part = code - u.seq * a.max_partitions;
        u.n_parts = (T + P - 1) / P;
        u.tok0 = u.part * P;
        u.tok1 = min(u.tok0 + P, T);
        u.nblk = (u.tok1 - u.tok0 + BS - 1) / BS;
        const int nunits = (u.nblk + BPU - 1) / BPU;
        // this wave's steps: a contiguous, balanced share of the unit
        u.u0 = nunits * wave / W;
        u.nuw = nunits * (wave + 1) / W - u.u0;
        return u;
    };

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
    char* wbase = smem + wave * Sh::WAVE_LDS;  // ring | queries | block ids
    const uint32_t wbase_lds = lds_addr_of(smem) + (uint32_t)(wave * Sh::WAVE_LDS);
    const char* q_lds = wbase + Sh::RING;
    const int* ids_lds = (const int*)(wbase + Sh::RING + Sh::QBYTES);
    int* meta = (int*)(smem + W * Sh::WAVE_LDS);  // free stage [W], invalid [W]

    // Copy the block ids of this wave's share of unit u (at most 64 blocks:
    // the dispatcher guarantees it) into id buffer `buf`, one per lane.
    // Entries past the sequence's last block are never used; lanes past the
    // table row copy the partition's first entry instead.
    auto copy_ids = [&](const Unit& u, int buf) {
        const int lb0 = u.part * P / BS;
        int e = lb0 + u.u0 * BPU + lane;
        if (e >= a.max_blocks_per_seq) e = lb0;
        const int32_t* bt = a.block_tables + (size_t)u.seq * a.max_blocks_per_seq + e;
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(bt),
                     "{m0}"(wbase_lds + (uint32_t)(Sh::RING + Sh::QBYTES + buf * 256))
                     : "memory");
    };
    // Copy unit u's query rows (G heads, contiguous) into the query area.
    auto copy_q = [&](const Unit& u) {
        const char* src = (const char*)a.q + ((size_t)u.seq * a.num_heads + (size_t)u.kvh * G) * D * 2 + lane * 16;
#pragma unroll
        for (int j = 0; j < Sh::QOPS; ++j)
            dma16_to_lds(src + j * 1024, wbase_lds + (uint32_t)(Sh::RING + j * 1024));
    };

    // Issue the copies of step k of unit u (this wave's share) into `stage`.
    // Every step queues the same number of copies (a block past the
    // partition's end re-copies the step's first block, whose rows the mask
    // then drops), so the in-flight counts stay exact.  ids: the block ids of
    // the wave's share, one per lane; `bad` is set when one is out of range.
    auto issue = [&](const Unit& u, int ids, int k, int stage, int& bad) {
        const uint32_t dst = wbase_lds + (uint32_t)(stage * Sh::STAGE);
        size_t first = 0;
#pragma unroll
        for (int b = 0; b < BPU; ++b) {
            const int idx = (u.u0 + k) * BPU + b;  // block index inside the partition
            size_t tile = first;
            if (b == 0 || idx < u.nblk) {
                int pb = __builtin_amdgcn_readlane(ids, k * BPU + b);
                if ((unsigned)pb >= (unsigned)a.num_blocks) { bad = 1; pb = 0; }
                tile = ((size_t)pb * H + u.kvh) * TILE;
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
    float m, l;
    f32x4 acc[NA][4];
    bf16x8 qop[Sh::NC];
    float qk_scale = 0.f;
    int tok1 = 0;

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
                s[h][i] = ok[h][i] ? sc[h][i] * qk_scale : -INFINITY;
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

    // ---- the unit loop
    load_tables(0);
    Unit cur = make_unit(0);
    Unit nxt = cur;
    copy_ids(cur, 0);
    bool started = false;  // step 0 of cur (and its queries) already issued
    int invalid = 0;       // an out-of-range block id was met in cur
    int invalid_nxt = 0;   // ... in the step of nxt issued ahead
    int ids_cur = 0;
    int istage = 0;        // ring stage of the next step to issue
    int cstage = 0;        // ring stage of the next step to consume
    int fstage = 1;        // a stage no copy in flight targets (the last consumed one)
    for (int r = 0; r < R; ++r) {
        const bool has_next = r + 1 < R;
        if (has_next) {
            if (((r + 1) & 63) == 0) load_tables(r + 1);
            nxt = make_unit(r + 1);
            copy_ids(nxt, (r + 1) & 1);  // lands before the next wait below
        }
        if (!started && cur.nuw > 0) {
            wait_vmcnt<0>();  // this unit's block ids (and any stores) are complete
            ids_cur = ids_lds[(r & 1) * 64 + lane];
            copy_q(cur);
            issue(cur, ids_cur, 0, istage, invalid);
            istage ^= 1;
        }
        // per-unit constants
        tok1 = cur.tok1;
        qk_scale = a.qk_scale_log2 * cur.ks;
        m = -INFINITY;
        l = 0.f;
        invalid_nxt = 0;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[aa][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        // The copies of the next unit's first step go out during this unit's
        // last step when the query area is already read (this unit has at
        // least two steps here) and the wave has work in the next unit.
        const bool ahead = has_next && cur.nuw >= 2 && nxt.nuw > 0;
        int ids_nxt = 0;
        for (int k = 0; k < cur.nuw; ++k) {
            if (k + 1 < cur.nuw) {
                issue(cur, ids_cur, k + 1, istage, invalid);
                istage ^= 1;
                wait_vmcnt<DPU>();
            } else if (ahead) {
                ids_nxt = ids_lds[((r + 1) & 1) * 64 + lane];  // landed: older than the last wait
                copy_q(nxt);
                issue(nxt, ids_nxt, 0, istage, invalid_nxt);
                istage ^= 1;
                wait_vmcnt<DPU + Sh::QOPS>();
            } else {
                wait_vmcnt<0>();
            }
            if (k == 0) {
                // queries of head n, elements 32 g .. 32 g + 31 (zero for n >= G)
#pragma unroll
                for (int c = 0; c < Sh::NC; ++c) {
                    const u32x4 v = *(const u32x4*)(q_lds + (n < G ? n : 0) * D * 2 + 64 * g + 16 * c);
                    qop[c] = __builtin_bit_cast(bf16x8, n < G ? v : u32x4{0, 0, 0, 0});
                }
            }
            const char* st = wbase + cstage * Sh::STAGE;
            const int utok0 = cur.tok0 + (cur.u0 + k) * Sh::UNIT;
            if (utok0 + Sh::UNIT <= tok1)
                step(st, utok0, std::false_type{});
            else
                step(st, utok0, std::true_type{});
            fstage = cstage;
            cstage ^= 1;
        }
        started = ahead;

        // ---- merge: the lane groups' partial sums, then the waves by
        // log-sum-exp, through each wave's free ring stage
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        {
            float* state = (float*)(wbase + fstage * Sh::STAGE);
            if (n < G) {
                if (g == 0) { state[Sh::STATE_ML / 4 + n] = m; state[Sh::STATE_ML / 4 + G + n] = l; }
                float* dst = state + n * D + 16 * g;
#pragma unroll
                for (int aa = 0; aa < NA; ++aa)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(float4*)(dst + 64 * aa + 4 * i) =
                            float4{acc[aa][0][i], acc[aa][1][i], acc[aa][2][i], acc[aa][3][i]};
            }
            if (lane == 0) { meta[wave] = fstage; meta[W + wave] = invalid; }
        }
        __syncthreads();
        {
            int bad = 0;
            const float* st[W];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                bad |= meta[W + w];
                st[w] = (const float*)(smem + w * Sh::WAVE_LDS + meta[w] * Sh::STAGE);
            }
            const float vs = cur.vs;
            const int hq0 = cur.kvh * G;
            for (int o = threadIdx.x; o < G * D; o += W * 64) {
                const int hg = o / D;
                const int d = o - hg * D;
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < W; ++w) M = fmaxf(M, st[w][Sh::STATE_ML / 4 + hg]);
                const float mu = M == -INFINITY ? 0.f : M;
                float L = 0.f, A = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const float f = fast_exp2(st[w][Sh::STATE_ML / 4 + hg] - mu);
                    L = fmaf(f, st[w][Sh::STATE_ML / 4 + G + hg], L);
                    A = fmaf(f, st[w][hg * D + d], A);
                }
                const size_t row = (size_t)cur.seq * a.num_heads + hq0 + hg;
                if (cur.n_parts == 1) {
                    store_out(a.out, a.out_dtype, row * D + d, bad ? __builtin_nanf("") : A / L * vs);
                } else {
                    const size_t pidx = row * a.max_partitions + cur.part;
                    if (d == 0) {
                        store_stream(&a.part_m[pidx], bad ? __builtin_nanf("") : M);
                        store_stream(&a.part_l[pidx], bad ? __builtin_nanf("") : L);
                    }
                    store_stream(&a.part_acc[pidx * D + d], bad ? __builtin_nanf("") : A * vs);
                }
            }
        }
        __syncthreads();  // the free stages may be refilled from here on
        cur = nxt;
        ids_cur = ids_nxt;
        invalid = invalid_nxt;
    }
}

// Workgroups of one launch: as many as the device keeps resident at once
// (queried once per device), never more than the largest possible number of
// work units.
template <int D, int BS, int W>
int launch_partition_mfma8(const DecodeArgs& a, hipStream_t stream) {
    using Sh = MfmaShape<D, BS, W>;
    auto kernel = decode_partition_mfma8_kernel<D, BS, W>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PA_ERR_LAUNCH;
    static int resident[64];  // workgroups the device keeps resident; 0 = not queried yet
    if (resident[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, W * 64, Sh::LDS) !=
                hipSuccess ||
            cus <= 0 || per_cu <= 0)
            return PA_ERR_LAUNCH;
        resident[dev] = cus * per_cu;
    }
    const size_t max_units = (size_t)a.num_seqs * a.max_partitions * a.num_kv_heads;
    const unsigned grid = (unsigned)(max_units < (size_t)resident[dev] ? max_units : (size_t)resident[dev]);
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(W * 64), Sh::LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif

// FP8 KV, bfloat16 queries, G = 8: head_dim 128, and partitions whose wave
// shares hold at most 64 blocks (others use the vector kernel).  Returns
// PA_ERR_UNSUPPORTED for shapes it does not cover.
inline bool mfma8_covers(int head_dim, int block_size, int partition_size) {
    constexpr int W = PA_MFMA_WAVES;
    if (head_dim != 128 || (block_size != 16 && block_size != 32)) return false;
    const int steps = (partition_size + 31) / 32;
    return (steps + W - 1) / W * (32 / block_size) <= 64;
}

inline int dispatch_mfma8(const DecodeArgs& a, int head_dim, hipStream_t stream) {
    constexpr int W = PA_MFMA_WAVES;
    if (!mfma8_covers(head_dim, a.block_size, a.partition_size)) return PA_ERR_UNSUPPORTED;
    if (a.block_size == 16) return launch_partition_mfma8<128, 16, W>(a, stream);
    if (a.block_size == 32) return launch_partition_mfma8<128, 32, W>(a, stream);
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
