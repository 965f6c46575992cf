// Multi-query (prefill / chunked prefill) attention over paged K/V on the
// gfx950 matrix cores: pa_prefill.
//
// Sequence i has T = seq_lens[i] cached tokens; its Q = query_start[i+1] -
// query_start[i] packed query rows are its last Q tokens (row j at position
// T - Q + j) and each attends to the cached tokens 0 .. its position.
//
// Work decomposition: one workgroup per (sequence, query tile, kv head).  A
// tile holds TQ = 64 / G query tokens, i.e. 64 (token, query head) columns
// for the G query heads of the kv head; each of the four waves owns 16 of
// them.  The workgroup walks the keys 0 .. (its last position) in steps of 32
// (two blocks of 16 or one of 32): the step's K and V rows are copied once
// into LDS (the four waves issue a quarter of the 16-byte asynchronous copies
// each) and serve all 64 columns.  Two stages alternate; one barrier per step
// separates "everyone finished step k-1" from "step k+1 may overwrite it".
//
// Per wave, with v_mfma_f32_16x16x32 (bf16 or f16 operands, f32
// accumulation) and lane = 16 g + n (g = 0..3, n = 0..15):
//   scores   S^T[key][column] = K Q^T: A = K rows (lane supplies row n of
//            the 16-key half, elements 32 g + 8 c .. + 7 for the c-th of four
//            products over head_dim 128), B = the wave's query columns.  The
//            lane receives column n's scores for keys 4 g + i, i = 0..3, of
//            each half.
//   softmax  per column: the lane's 8 scores, a max across the four lane
//            groups, the running max uniform over the column's lanes; the
//            causal mask (key position > column position) gives -inf.
//   values   O^T[dim][column] += V^T P^T: B = the lane's own p (split into
//            a 16-bit high part and the rounded remainder, two products, so
//            p keeps about 16 significant bits); A = V^T, the lane supplying
//            dims 64 a + 4 n + b of its 8 keys (eight 8-byte LDS reads
//            repacked by byte permutes, one product per (a, b)).  The lane
//            receives column n's dims 64 a + 16 g + 4 i + b.
// K rows sit in LDS XOR-swizzled by 16-byte granule (row t, granule x at
// slot x ^ (t mod 16)) and V rows by half row (x ^ 8 when bit 2 of t is
// set), both through the copies' source addresses, so that the reads above
// spread over the banks.
//
// The physical block ids of the workgroup's key range are loaded into LDS
// first (in windows of ID_CAP blocks for very long sequences).  An id
// outside the pool is never used as an address: block 0 is read instead and
// the tile's output rows become NaN.  Rows of keys at or beyond T (the tail
// of the last block) are dropped: their scores are masked and their values
// zeroed.
#include <type_traits>

#include "pa_decode_kernel.hpp"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PrefillArgs {
    void* out;
    int out_dtype;
    const void* q;
    const int32_t* query_start;
    int total_q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* seq_lens;
    int max_seq_len;
    int num_seqs;
    int num_heads;
    int num_kv_heads;
    int num_blocks;
    int tiles;            // query tiles per sequence in the grid
    float qk_scale_log2;  // scale * log2(e)
};

template <Fmt F> struct MfmaOps;
template <> struct MfmaOps<Fmt::BF16> {
    typedef bf16x8 vec;
    typedef __bf16 elem;
    __device__ static __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct MfmaOps<Fmt::F16> {
    typedef f16x8 vec;
    typedef _Float16 elem;
    __device__ static __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Maximum over the four 16-lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float prefill_max_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float prefill_sum_groups(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 4
#endif

template <int D, int BS, int G>
struct PrefillShape {
    static constexpr int S = PA_PREFILL_STAGES;   // LDS stages (S - 1 steps of copies in flight)
    static constexpr int W = 4;                   // waves per workgroup
    static constexpr int COLS = 16;               // query columns per wave
    static constexpr int TQ = W * COLS / G;       // query tokens per workgroup
    static constexpr int TOK_PER_WAVE = COLS / G;
    static constexpr int STEP = 32;               // keys per step
    static constexpr int BPS = STEP / BS;         // blocks per step
    static constexpr int ROWB = D * 2;            // bytes of one K or V row
    static constexpr int HALF = STEP * ROWB;      // K (or V) rows of one step
    static constexpr int STAGE = 2 * HALF;
    static constexpr int COPIES = STAGE / 1024;   // 1 KiB copies per step
    static constexpr int COPIES_PER_WAVE = COPIES / W;
    static constexpr int ID_CAP = 2048;           // block ids held in LDS
    static constexpr int IDS_AT = S * STAGE;
    static constexpr int LDS = IDS_AT + ID_CAP * 4 + 16;
    static_assert(D == 128, "the lane roles assume head_dim 128");
    static_assert(BS == 16 || BS == 32, "block size");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group");
    static_assert(COPIES % W == 0, "copies split evenly over the waves");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(ID_CAP % BPS == 0, "a step's blocks never straddle an id window");
    static_assert(S >= 2 && S <= 4, "the waits below cover two to four stages");
};

template <Fmt KV, int D, int BS, int G>
__global__ void __launch_bounds__(256, 2) prefill_mfma_kernel(const PrefillArgs a) {
    using Sh = PrefillShape<D, BS, G>;
    using Ops = MfmaOps<KV>;
    using vec = typename Ops::vec;
    constexpr int ROWB = Sh::ROWB, STEP = Sh::STEP, BPS = Sh::BPS;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int n = lane & 15;

    // ---- (sequence, tile, kv head) of this workgroup: the last tiles of the
    // chunks first, since they see the most keys
    const int H = a.num_kv_heads;
    const int per_tile = a.num_seqs * H;
    const int tile = a.tiles - 1 - (int)(blockIdx.x / per_tile);
    const int rem = blockIdx.x % per_tile;
    const int seq = rem / H;
    const int kvh = rem - seq * H;

    const int q0 = a.query_start[seq];
    const int q1 = a.query_start[seq + 1];
    const int T = a.seq_lens[seq];
    if (q0 < 0 || q1 < q0 || q1 > a.total_q) return;  // rows that cannot be addressed
    const int Q = q1 - q0;
    const int tok_lo = tile * Sh::TQ;
    if (tok_lo >= Q) return;
    const int tok_hi = min(tok_lo + Sh::TQ, Q);
    const bool bad_seq = T <= 0 || T > a.max_seq_len || Q > T ||
                         (T + BS - 1) / BS > a.max_blocks_per_seq;

    // this lane's column: token tok_lo + wave * (16 / G) + n / G, head n % G
    const int ctok = tok_lo + wave * Sh::TOK_PER_WAVE + n / G;
    const int chead = kvh * G + n % G;
    const bool cvalid = ctok < tok_hi;
    const int cpos = cvalid ? T - Q + ctok : -1;  // -1: every key masked
    // key range of the workgroup and of this wave
    const int pos_max = T - Q + tok_hi - 1;
    const int wtok_lo = tok_lo + wave * Sh::TOK_PER_WAVE;
    const int wtok_hi = min(wtok_lo + Sh::TOK_PER_WAVE, tok_hi);
    const bool wave_cols = wtok_lo < tok_hi;       // the wave has at least one column
    const int wpos_min = T - Q + wtok_lo;
    const int wpos_max = T - Q + wtok_hi - 1;

    auto write_rows = [&](float v) {
        for (int o = threadIdx.x; o < (tok_hi - tok_lo) * G * D; o += 256) {
            const int tk = o / (G * D);
            const int rr = o - tk * G * D;
            const size_t row = (size_t)(q0 + tok_lo + tk) * a.num_heads + kvh * G + rr / D;
            store_out(a.out, a.out_dtype, row * D + rr % D, v);
        }
    };
    if (bad_seq) {
        write_rows(__builtin_nanf(""));
        return;
    }

    // ---- queries of this lane's column, elements 32 g + 8 c .. + 7 (zero
    // for columns past the tile)
    vec qop[4];
    {
        const u32x4* qp = (const u32x4*)((const char*)a.q +
                                         (((size_t)(q0 + (cvalid ? ctok : tok_lo)) * a.num_heads + chead) * D +
                                          32 * g) * 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 v = qp[c];
            qop[c] = __builtin_bit_cast(vec, cvalid ? v : u32x4{0, 0, 0, 0});
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(qop[c]));  // resident before the copies start
    }

    // ---- block ids of the key range into LDS, in windows of ID_CAP
    int* ids = (int*)(smem + Sh::IDS_AT);
    int* bad_flag = ids + Sh::ID_CAP;
    const int nblk = pos_max / BS + 1;
    const int32_t* bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    auto load_ids = [&](int first) {
        const int cnt = min(Sh::ID_CAP, nblk - first);
        for (int j = threadIdx.x; j < cnt; j += 256) {
            int id = bt[first + j];
            if ((unsigned)id >= (unsigned)a.num_blocks) {
                *bad_flag = 1;
                id = 0;
            }
            ids[j] = id;
        }
    };
    if (threadIdx.x == 0) *bad_flag = 0;
    __syncthreads();
    int window = 0;  // first block held in `ids`
    load_ids(0);
    __syncthreads();

    // ---- copies of one step: wave w copies COPIES_PER_WAVE 1 KiB pieces;
    // piece p < COPIES/2 is K, the rest V; each covers 4 rows of 256 bytes
    const char* kc = (const char*)a.k_cache;
    const char* vc = (const char*)a.v_cache;
    const uint32_t lds0 = lds_addr_of(smem);
    auto issue = [&](int k, int stage) {
#pragma unroll
        for (int j = 0; j < Sh::COPIES_PER_WAVE; ++j) {
            const int piece = wave * Sh::COPIES_PER_WAVE + j;
            const bool is_v = piece >= Sh::COPIES / 2;
            const int pk = is_v ? piece - Sh::COPIES / 2 : piece;
            const int row = pk * 4 + lane / 16;                 // key row inside the step
            const int slot = lane % 16;                          // 16-byte slot in the LDS row
            const int gran = is_v ? (slot ^ (((row >> 2) & 1) << 3)) : (slot ^ (row & 15));
            const int blk = k * BPS + row / BS;                  // block index in the sequence
            const int b0 = k * BPS;                              // the step's first block
            const int use = blk < nblk ? blk : b0;               // past the last block: reread the first
            const int pb = ids[use - window];
            const size_t src = (((size_t)pb * H + kvh) * BS + row % BS) * ROWB + gran * 16;
            const uint32_t dst = lds0 + (uint32_t)(stage * Sh::STAGE + (is_v ? Sh::HALF : 0) + pk * 1024);
            dma16_to_lds_stream((is_v ? vc : kc) + src, dst);
        }
    };

    // per-lane state of column n
    float m = -INFINITY, l = 0.f;
    f32x4 acc[2][4];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[aa][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float qk_scale = a.qk_scale_log2;

    // LDS read offsets that do not depend on the step
    const int kslot[4] = {(4 * g + 0) ^ n, (4 * g + 1) ^ n, (4 * g + 2) ^ n, (4 * g + 3) ^ n};

    auto step = [&](const char* st, int k0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const char* kb = st;
        const char* vb = st + Sh::HALF;
        // scores of both 16-key halves: sc[h][i] is key k0 + 16 h + 4 g + i
        f32x4 sc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const char* rowp = kb + (16 * h + n) * ROWB;
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                c = Ops::mma(__builtin_bit_cast(vec, *(const u32x4*)(rowp + kslot[cc] * 16)), qop[cc], c);
            sc[h] = c;
        }
        float s[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = !MASKED || k0 + 16 * h + 4 * g + i <= cpos;
                s[h][i] = ok ? sc[h][i] * qk_scale : -INFINITY;
            }
        float mx = s[0][0];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[h][i]);
        mx = prefill_max_groups(mx);
        const float mn = fmaxf(m, mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        if (__builtin_amdgcn_ballot_w64(mn != m) != 0) {
            const float alpha = fast_exp2(m - mu);
            l *= alpha;
#pragma unroll
            for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[aa][b] *= alpha;
        }
        m = mn;
        vec phi, plo;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[h][i] - mu);
                l += p;
                const typename Ops::elem ph = (typename Ops::elem)p;
                phi[4 * h + i] = ph;
                plo[4 * h + i] = (typename Ops::elem)(p - (float)ph);
            }
        // values: dims 64 a + 4 n + b of keys 16 h + 4 g + i, one product per (a, b)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
            u32x2 w[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * h + 4 * g + i;
                    const int gran = (8 * aa + n / 2) ^ (((row >> 2) & 1) << 3);
                    w[h][i] = *(const u32x2*)(vb + row * ROWB + gran * 16 + (n & 1) * 8);
                    if constexpr (MASKED) {
                        if (k0 + row >= T) w[h][i] = u32x2{0u, 0u};  // rows past the sequence may hold anything
                    }
                }
            // operand b, element 4 h + i = element b of w[h][i]: pairs of keys
            // share a 32-bit word
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                u32x4 op;
                const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        const uint32_t lo = w[h][2 * ip][b >> 1];
                        const uint32_t hi = w[h][2 * ip + 1][b >> 1];
                        op[2 * h + ip] = __builtin_amdgcn_perm(hi, lo, sel);
                    }
                const vec A = __builtin_bit_cast(vec, op);
                acc[aa][b] = Ops::mma(A, phi, acc[aa][b]);
                acc[aa][b] = Ops::mma(A, plo, acc[aa][b]);
            }
        }
    };

    // ---- main loop over 32-key steps, S - 1 steps of copies ahead.  The
    // first S - 1 steps never need a new id window (S - 1 < ID_CAP / BPS).
    constexpr int S = Sh::S;
    const int nsteps = pos_max / STEP + 1;
    const int steps_per_window = Sh::ID_CAP / BPS;
#pragma unroll
    for (int k = 0; k < S - 1; ++k)
        if (k < nsteps) issue(k, k);
    for (int k = 0; k < nsteps; ++k) {
        // this wave's copies of step k are complete when at most those of the
        // later steps already issued (up to S - 2 of them) are in flight
        const int later = min(S - 2, nsteps - 1 - k);
        if constexpr (S >= 4) {
            if (later >= 2) wait_vmcnt<2 * Sh::COPIES_PER_WAVE>();
            else if (later == 1) wait_vmcnt<Sh::COPIES_PER_WAVE>();
            else wait_vmcnt<0>();
        } else if constexpr (S == 3) {
            if (later >= 1) wait_vmcnt<Sh::COPIES_PER_WAVE>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();  // everyone's copies of step k landed; step k-1 is finished everywhere
        const int kn = k + S - 1;  // the step whose copies go out now, into step k-1's stage
        if (kn < nsteps) {
            if (kn % steps_per_window == 0) {  // its ids are in the next window
                window = kn * BPS;
                load_ids(window);
                __syncthreads();
            }
            issue(kn, kn % S);
        }
        const int k0 = k * STEP;
        if (wave_cols && k0 <= wpos_max) {  // some column of this wave sees keys of this step
            const char* st = smem + (k % S) * Sh::STAGE;
            if (k0 + STEP - 1 <= wpos_min && k0 + STEP <= T)
                step(st, k0, std::false_type{});
            else
                step(st, k0, std::true_type{});
        }
    }

    // ---- output: column n, dims 64 a + 16 g + 4 i + b
    l = prefill_sum_groups(l);
    const bool bad = *bad_flag != 0;
    if (cvalid) {
        const float inv = 1.f / l;
        const size_t base = ((size_t)(q0 + ctok) * a.num_heads + chead) * D;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float v = bad ? __builtin_nanf("") : acc[aa][b][i] * inv;
                    store_out(a.out, a.out_dtype, base + 64 * aa + 16 * g + 4 * i + b, v);
                }
    }
}

template <Fmt KV, int D, int BS, int G>
static int launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    using Sh = PrefillShape<D, BS, G>;
    auto kernel = prefill_mfma_kernel<KV, D, BS, G>;
    static const hipError_t attr =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, Sh::LDS);
    if (attr != hipSuccess) return PA_ERR_LAUNCH;
    const size_t grid = (size_t)a.tiles * a.num_seqs * a.num_kv_heads;
    if (grid == 0) return PA_OK;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), Sh::LDS, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <Fmt KV, int D, int BS>
static int dispatch_prefill_group(PrefillArgs& a, int group, int max_query_len, hipStream_t stream) {
    auto tiles = [&](int tq) { return (max_query_len + tq - 1) / tq; };
    switch (group) {
        case 1: a.tiles = tiles(PrefillShape<D, BS, 1>::TQ); return launch_prefill<KV, D, BS, 1>(a, stream);
        case 2: a.tiles = tiles(PrefillShape<D, BS, 2>::TQ); return launch_prefill<KV, D, BS, 2>(a, stream);
        case 4: a.tiles = tiles(PrefillShape<D, BS, 4>::TQ); return launch_prefill<KV, D, BS, 4>(a, stream);
        case 8: a.tiles = tiles(PrefillShape<D, BS, 8>::TQ); return launch_prefill<KV, D, BS, 8>(a, stream);
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
    if ((((uintptr_t)q) | ((uintptr_t)k_cache) | ((uintptr_t)v_cache)) & 15u) return PA_ERR_SHAPE;
    const long long tiles_max = (max_query_len + 7) / 8;  // the smallest tile is 8 tokens
    if (tiles_max * num_seqs * num_kv_heads > 0x7fffffffLL) return PA_ERR_SHAPE;
    PrefillArgs a;
    a.out = out;
    a.out_dtype = out_dtype;
    a.q = q;
    a.query_start = query_start;
    a.total_q = total_q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.seq_lens = seq_lens;
    a.max_seq_len = max_seq_len;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    a.tiles = 0;
    a.qk_scale_log2 = scale * kLog2e;
    const hipStream_t s = (hipStream_t)stream;
    if (kv_dtype == PA_DTYPE_BF16)
        return block_size == 16 ? dispatch_prefill_group<Fmt::BF16, 128, 16>(a, group, max_query_len, s)
                                : dispatch_prefill_group<Fmt::BF16, 128, 32>(a, group, max_query_len, s);
    return block_size == 16 ? dispatch_prefill_group<Fmt::F16, 128, 16>(a, group, max_query_len, s)
                            : dispatch_prefill_group<Fmt::F16, 128, 32>(a, group, max_query_len, s);
}
