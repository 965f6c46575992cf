/*
 * pagedattn.h -- C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * The library implements the GPU side of PagedAttention: the KV cache is cut
 * into fixed-size physical blocks of B tokens, and each sequence reaches its
 * tokens through a block table that maps logical block k (tokens k*B ..
 * k*B+B-1) to a physical block id (0h-n0.github.io, "論文解説: Efficient
 * Memory Management for Large Language Model Serving with PagedAttention",
 * section "PagedAttentionのメモリ管理"; dihengye.cn, "PagedAttention",
 * section "核心思想").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_cache, key, value, q, out, slot_mapping, block_pairs,
 *   block_tables, seq_lens, k_scale, v_scale and workspace are DEVICE
 *   pointers.  All other arguments are host scalars.
 * - `stream` is a hipStream_t handle (NULL = the null stream).  Every call is
 *   asynchronous on that stream, never synchronises and never reads device
 *   memory on the host.
 * - The library owns no memory and allocates none: the caller owns every
 *   buffer, including the split-KV workspace of pa_decode.  It keeps no
 *   global state; concurrent calls on different streams are independent as
 *   long as their output buffers do not overlap.
 * - Physical KV pool layout (one array for K, one for V):
 *       cache[num_blocks][num_kv_heads][block_size][head_dim]
 *   in the element format `kv_dtype`, contiguous, 16-byte aligned.  One
 *   (block, kv head) tile of block_size*head_dim elements is contiguous.
 * - Return value: PA_OK (0) or a negative pa_status.  Argument errors are
 *   detected on the host before anything is launched; then nothing runs.
 *   PA_ERR_LAUNCH reports a failed kernel launch.
 * - Device contents are not validated on the host.  Kernels guard every
 *   device-supplied index that would address memory: an out-of-range slot or
 *   block pair is skipped, and a sequence whose length or block ids are out
 *   of range gets a row of NaN in `out` instead of a memory access.
 * - The checked build (libpagedattn_checked.so, compiled with
 *   PA_CHECK_CONTENTS=1; same ABI) copies the index arrays each call reads
 *   to the host before launching, synchronising `stream`, and returns
 *   PA_ERR_CONTENT without launching anything when they break a contract
 *   stated below: a slot past the pool or used twice in one call; a copy or
 *   swap pair outside its pools, a destination named twice, or (copy) a
 *   destination that is also a source; a length outside [0, max_seq_len] or
 *   needing more than max_blocks_per_seq blocks; a table entry a sequence
 *   reads that is outside the pool; group_start or query_start not
 *   non-decreasing over their stated range; a negative prefix or a member
 *   whose table differs from its group's first sequence's over the shared
 *   tokens; a query count above max_query_len or above the sequence's
 *   length.  It is a debugging aid: its calls synchronise and cannot be
 *   captured in a graph.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  PA_DTYPE_FP8_E4M3 is the OCP 8-bit float E4M3FN (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN =
 * 0x7F/0xFF, largest finite 448), stored one byte per element with a float32
 * scale per kv head: value = decoded_code * scale.  FP8 KV storage with a
 * scale is named on youngju.dev, "KVキャッシュとPagedAttention — 推論メモリの
 * すべて", section "KV量子化: FP8とINT8". */
typedef enum pa_dtype {
    PA_DTYPE_F32 = 0,
    PA_DTYPE_F16 = 1,
    PA_DTYPE_BF16 = 2,
    PA_DTYPE_FP8_E4M3 = 3
} pa_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                        */
    PA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or inconsistent */
    PA_ERR_DTYPE = -3,       /* unknown dtype code or unsupported dtype combination */
    PA_ERR_UNSUPPORTED = -4, /* valid but not built: head_dim, block_size, GQA group */
    PA_ERR_WORKSPACE = -5,   /* workspace smaller than pa_decode_workspace_size()   */
    PA_ERR_LAUNCH = -6,      /* the HIP runtime rejected a kernel launch           */
    PA_ERR_MEMORY = -7,      /* a pool the GPU cannot address (pa_swap_blocks)      */
    PA_ERR_CONTENT = -8,     /* checked build only: device contents break the contract */
    PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: the call needs more than its static scratch */
} pa_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_string(int status);

/*
 * pa_reshape_and_cache -- store the K and V rows of new tokens in their slots.
 *
 * Keeping each token's K and V once computed, for reuse by every later
 * decode step, is what the KV cache is for (youngju.dev, same page, section
 * "核心原理: KVキャッシュとは何か"); blocks are taken one at a time as a
 * sequence grows (section "PagedAttention: OS仮想メモリ式の管理").
 *
 * For every token t < num_tokens with s = slot_mapping[t]:
 *     k_cache[s / block_size][h][s % block_size][:] = key[t][h][:]
 *     v_cache[s / block_size][h][s % block_size][:] = value[t][h][:]
 * for all kv heads h.  The copy is bitwise (elements are moved as bytes).
 *   key, value   [num_tokens][num_kv_heads][head_dim], kv_dtype, 16-B aligned
 *   k_cache, v_cache   pool as described above, kv_dtype
 *   slot_mapping [num_tokens] int64.  s < 0 means "skip this token".  A slot
 *                at or beyond num_blocks*block_size is skipped as well.
 *                Two tokens with the same slot in one call: which one lands
 *                is unspecified.
 *   head_dim     64 or 128;  block_size 16 or 32.
 * num_tokens == 0 is a valid no-op.  key, value and the pools must be 16-byte
 * aligned (PA_ERR_SHAPE otherwise).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int kv_dtype,
                         void* stream);

/*
 * pa_reshape_and_cache_fp8 -- store new tokens into FP8 pools, quantizing.
 *
 * The same scatter as pa_reshape_and_cache, for pools in PA_DTYPE_FP8_E4M3
 * (one byte per element with a float32 scale per kv head; youngju.dev, same
 * page, section "KV量子化: FP8とINT8"), from new K/V rows in a wider format.
 * For every element x of key[t][h][:] (value[t][h][:] likewise):
 *     code = E4M3FN(x / k_scale[h])   (v_scale[h] for values)
 * where x is widened exactly to float32, the quotient is the IEEE float32
 * division (round to nearest even), a NaN quotient gives code 0x7F, and
 * magnitudes beyond 448 (infinities included) saturate to 448 before the
 * conversion rounds to the nearest code (ties to even).  The stored value
 * code * scale then reads back through pa_decode's FP8 path.
 *   key, value   [num_tokens][num_kv_heads][head_dim] in src_dtype (F32, F16
 *                or BF16), 16-byte aligned
 *   k_cache, v_cache   FP8 pools [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale   [num_kv_heads] float32, device
 *   slot_mapping, num_tokens, shapes: as for pa_reshape_and_cache (slots < 0
 *                or past the pool are skipped).
 * key, value and the pools must be 16-byte aligned (PA_ERR_SHAPE otherwise).
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, int src_dtype, void* k_cache,
                             void* v_cache, const float* k_scale, const float* v_scale,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, void* stream);

/*
 * pa_copy_blocks -- copy whole physical blocks for copy-on-write.
 *
 * When a sequence must write into a block whose reference count exceeds one,
 * a new block is allocated, the shared block's contents are copied into it,
 * the old block's count is decremented and the table entry remapped
 * (0h-n0.github.io explainer, section "Copy-on-Write（CoW）によるメモリ共有").
 * This call performs the copy step for a batch of such blocks; the host
 * block manager does the rest.
 *
 * For every pair p < num_pairs with (src, dst) = (block_pairs[2p], block_pairs[2p+1]):
 *     k_cache[dst][:][:][:] = k_cache[src][:][:][:]   (all kv heads, all rows)
 *     v_cache[dst][:][:][:] = v_cache[src][:][:][:]
 * bitwise.  Precondition: destinations are distinct and none is also a
 * source in the same call (then every pair reads the contents from before
 * the call).  Pairs with an id outside [0, num_blocks) are skipped.
 *   block_pairs  [num_pairs][2] int64, device memory.
 * num_pairs == 0 is a valid no-op.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int num_blocks, int kv_dtype,
                   void* stream);

/*
 * pa_swap_blocks -- move whole blocks between two pools: the device pool
 * and a pool in pinned host memory.
 *
 * When GPU memory runs short, a sequence can be preempted by evicting its
 * physical blocks to CPU memory and bringing them back later; the transfer
 * is bound by the host link (0h-n0.github.io explainer, section
 * "プリエンプション戦略", strategy 1).  This call performs such a transfer for
 * a batch of blocks, in either direction; the host block manager keeps the
 * mapping (BlockManager.swap_out / swap_in in the Python package).
 *
 * For every pair p < num_pairs with (s, d) = (block_pairs[2p], block_pairs[2p+1]):
 *     dst_k[d][:][:][:] = src_k[s][:][:][:]   (all kv heads, all rows)
 *     dst_v[d][:][:][:] = src_v[s][:][:][:]
 * bitwise.  Swap-out: src = device pool, dst = host pool; swap-in: the
 * reverse.  Pairs with s outside [0, src_num_blocks) or d outside
 * [0, dst_num_blocks) are skipped.  Destinations must be distinct.
 *   src_k, src_v, dst_k, dst_v   pools [blocks][num_kv_heads][block_size][head_dim]
 *                in kv_dtype, 16-byte aligned.  A host pool must be pinned
 *                memory that the device can address (hipHostMalloc; torch's
 *                pin_memory=True): the GPU reads or writes it directly over
 *                the host link, one kernel for the whole batch.
 *   block_pairs  [num_pairs][2] int64, device (or pinned host) memory.
 * num_pairs == 0 is a valid no-op.  Before launching, each pool pointer is
 * checked with hipPointerGetAttributes: memory that is neither device memory
 * nor pinned host memory mapped for the device returns PA_ERR_MEMORY.  The
 * call is asynchronous on `stream`; synchronise before the host reads a
 * swapped-out block.
 */
int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int64_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int src_num_blocks, int dst_num_blocks, int kv_dtype, void* stream);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs.
 *
 * Holds one partial state (m, l, acc[head_dim]) in float32 per (sequence,
 * query head, KV partition), with ceil(max_seq_len / partition_size)
 * partitions per sequence: acc in rows of head_dim; m and l in 64-byte
 * records of one kv head's group, each written whole (sized for one record
 * per query head, the most kv heads there can be), or in per-row arrays
 * inside the same space for groups of four query heads over 16-bit K/V.  Its
 * contents need no initialisation.  Returns 0 for invalid arguments.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim, int max_seq_len,
                                int partition_size);

/*
 * pa_decode -- single-query attention of every sequence over its paged K/V.
 *
 * For sequence i with T = seq_lens[i] cached tokens (the current token
 * included) and query head h, with G = num_heads / num_kv_heads and kv head
 * g = h / G (consecutive query heads share a kv head; youngju.dev, same
 * page, section "GQAとMQA"):
 *     K_i, V_i = rows 0..T-1 of the sequence, token t read from physical
 *                block block_tables[i][t / block_size], row t % block_size,
 *                kv head g (dequantised: code * k_scale[g] / * v_scale[g] for FP8)
 *     out[i][h][:] = softmax(scale * K_i q[i][h]) V_i
 * which is the attention of the current query against all cached tokens
 * (0h-n0.github.io explainer, section "Attention計算").  T == 0 gives a row
 * of zeros.
 *
 * Method: the tokens of a sequence are split into partitions of
 * partition_size tokens (a multiple of block_size; partition p covers
 * [p*P, min((p+1)P, T)), so no partition is empty).  One workgroup per
 * (sequence, kv head, partition) walks the partition's blocks with the
 * online-softmax recurrence of auturnal.com, "メモリ予算内での言語モデルのサー
 * ビング", equation (4): m' = max(m, max_j s_j), l' = e^{m-m'} l +
 * sum_j e^{s_j-m'}, and the value accumulator rescaled by the same factor,
 * for all G query heads of the kv head at once.  A second kernel merges the
 * partition states of each (sequence, query head) with the same rule in a
 * fixed partition order.  Sequences with a single partition are finished by
 * the first kernel.  Results are deterministic (bitwise identical between
 * calls and independent of which physical blocks hold the data).
 *
 *   out          [num_seqs][num_heads][head_dim], out_dtype (F32, F16 or BF16)
 *   q            [num_seqs][num_heads][head_dim], q_dtype
 *   k_cache, v_cache   pool, kv_dtype
 *   block_tables [num_seqs][max_blocks_per_seq] int32; entries at and beyond
 *                ceil(seq_lens[i]/block_size) are never read
 *   seq_lens     [num_seqs] int32, device; each must lie in [0, max_seq_len]
 *                and need at most max_blocks_per_seq blocks
 *   max_seq_len  host upper bound of seq_lens (sizes the grid and workspace)
 *   num_blocks   number of physical blocks in the pool (bounds block ids)
 *   scale        softmax scale, typically 1/sqrt(head_dim)
 *   k_scale, v_scale   [num_kv_heads] float32, device; required for FP8 KV,
 *                ignored (may be NULL) otherwise
 *   partition_size     tokens per KV partition, a positive multiple of block_size
 *   workspace    device scratch of at least pa_decode_workspace_size(num_seqs,
 *                num_heads, head_dim, max_seq_len, partition_size) bytes,
 *                256-byte aligned; its contents on entry do not matter
 *
 * Supported: head_dim 64 or 128; block_size 16 or 32; G in {1, 2, 4, 8};
 * (kv_dtype, q_dtype) in {(F32, F32), (F16, F16), (BF16, BF16),
 * (FP8_E4M3, BF16)}; out_dtype F32, F16 or BF16.  Accumulation is float32.
 */
int pa_decode(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
              const void* v_cache, int kv_dtype, const int32_t* block_tables,
              int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
              float scale, const float* k_scale, const float* v_scale, int partition_size,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and results as pa_decode,
 * with the split-KV workspace taken from a static device array of the
 * library instead of a caller's buffer.
 *
 * Arguments: those of pa_decode without workspace and workspace_bytes.
 * The library's static array holds PA_DECODE_NOALLOC_SCRATCH_BYTES bytes on
 * every GPU it runs on, from the first call on that GPU until the process
 * ends; the call looks up its device address once per device and then
 * calls no allocating routine.  A call whose pa_decode_workspace_size(...)
 * exceeds that size returns PA_ERR_SCRATCH before touching the device.
 * Every call on one GPU shares that GPU's array, whose contents on entry do
 * not matter: calls that overlap in time on one GPU (two streams, or two
 * host threads) race on it and give undefined results; calls ordered on one
 * stream are safe.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)

int pa_decode_noalloc(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                      const void* v_cache, int kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      float scale, const float* k_scale, const float* v_scale, int partition_size,
                      void* stream);

/*
 * pa_decode_partition, pa_decode_reduce -- the two launches of pa_decode,
 * exported separately so that a caller can time them individually.  Called
 * in this order on one stream with identical arguments they are exactly
 * pa_decode.  pa_decode_partition writes the workspace (and the rows of
 * single-partition sequences); pa_decode_reduce reads it and writes the
 * remaining rows.
 */
int pa_decode_partition(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                        const void* v_cache, int kv_dtype, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                        int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                        int block_size, int num_blocks, float scale, const float* k_scale,
                        const float* v_scale, int partition_size, void* workspace,
                        size_t workspace_bytes, void* stream);

int pa_decode_reduce(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                     const void* v_cache, int kv_dtype, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                     int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, float scale, const float* k_scale, const float* v_scale,
                     int partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- store each sequence's newest token, then pa_decode.
 *
 * A decode step first writes the K and V rows of the token it has just
 * computed into the cache, then attends over all cached tokens, that token
 * included (the explainer's section "Attention計算": K holds every token so
 * far).  This call does both: for every sequence i with T = seq_lens[i] > 0,
 * it stores key[i] and value[i] (all kv heads) at position T - 1, i.e. in
 * row (T-1) % block_size of block block_tables[i][(T-1) / block_size], as
 * pa_reshape_and_cache would with that slot; then it computes exactly what
 * pa_decode computes.  The result and the pool are bitwise those of
 * pa_reshape_and_cache followed by pa_decode.
 *
 * The store happens inside the partition kernel -- the wave that stages a
 * sequence's last block writes the new rows into the pool and into its
 * staged tile, saving the separate scatter launch -- for every shape but
 * two: the FP8 matrix-core shape (E4M3 K/V, eight query heads per kv head,
 * head_dim 128) and the GQA-4 shapes (bf16 or f16 K/V, four query heads per
 * kv head) with more than 64 blocks per partition.  Those launch a small
 * copy kernel first.
 *   key, value   [num_seqs][num_kv_heads][head_dim] in kv_dtype (for FP8
 *                pools, E4M3 codes), 16-byte aligned, device
 *   other arguments: as for pa_decode.  The block that holds position T - 1
 *                must not be shared with another sequence (copy-on-write is
 *                the caller's, through pa_copy_blocks, before this call).
 * Sequences with T == 0 or an invalid length store nothing; a block id
 * outside the pool stores nothing and gives a NaN row, as in pa_decode.
 */
int pa_decode_append(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                     const void* v_cache, int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* seq_lens, int max_seq_len, int num_seqs, int num_heads, int num_kv_heads,
                     int head_dim, int block_size, int num_blocks, float scale, const float* k_scale,
                     const float* v_scale, int partition_size, void* workspace, size_t workspace_bytes,
                     void* stream, const void* key, const void* value);

/*
 * pa_decode_append_cow -- pa_copy_blocks, then pa_decode_append, in one
 * launch where possible.
 *
 * A decode step of a batch with copy-on-write (the explainer's section
 * "Copy-on-Write（CoW）によるメモリ共有": a sequence about to write into a
 * shared block gets a private copy first) copies those blocks, stores each
 * sequence's new token and attends.  The result and the pool are bitwise
 * those of pa_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, ...)
 * followed by pa_decode_append with the same arguments.
 *
 * Where pa_decode_append stores the tokens inside the partition kernel
 * (above; head_dim 64 or 128, block size 16 or 32) and num_pairs <= 16, the
 * copies run in the same launch: its last workgroups copy the pairs (K and
 * V, each block split into chunks of at most 8 16-byte granules per
 * thread), the partition workgroups read a destination block from its
 * source (the same content once copied), and when a destination is a
 * sequence's last block its copying workgroups write that sequence's new
 * token in place of the copied row.  Other shapes and more pairs make the
 * two calls.
 * key and value may both be null: the call is then pa_copy_blocks followed
 * by pa_decode (no token is stored; a step that stores its tokens another
 * way, such as pa_reshape_and_cache_fp8, makes that call first).  For the
 * FP8 matrix-core shape this runs as one launch as well, the copies and
 * the per-block source check as above; other shapes make the two calls.
 *   block_pairs  int64 [num_pairs][2] (source, destination), device; pairs
 *                outside the pool are skipped, as by pa_copy_blocks
 *   num_pairs    >= 0; 0 makes this pa_decode_append (pa_decode without
 *                new rows)
 *   other arguments: as for pa_decode_append.  Preconditions of
 *                pa_copy_blocks: destinations are distinct and none is a
 *                source; a destination belongs to at most one sequence.
 *                And a source that is some sequence's last block (which
 *                receives that sequence's token in this call) is copied only
 *                to the last block of a sequence appending at the same row
 *                (the copy-on-write of a shared last block before an
 *                append): the one-launch path copies beside the tokens'
 *                stores, so such a source may be read with or without its
 *                token, and only then does the copy hold the right one (the
 *                appending sequence's own).
 * Errors: PA_ERR_SHAPE for num_pairs < 0, PA_ERR_NULL for a null block_pairs
 * with num_pairs > 0 or for exactly one of key and value null (before any
 * launch), otherwise those of the two calls.
 */
int pa_decode_append_cow(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                         const void* v_cache, int kv_dtype, const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens, int max_seq_len, int num_seqs, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                         const float* k_scale, const float* v_scale, int partition_size, void* workspace,
                         size_t workspace_bytes, void* stream, const void* key, const void* value,
                         const int64_t* block_pairs, int num_pairs);

/*
 * pa_decode_shared_prefix -- pa_decode for batches whose sequences share
 * prompt blocks (parallel samples and beams forked from one prompt), reading
 * each shared block once per group instead of once per sequence.
 *
 * Forked sequences share every block of their parent through reference
 * counts (dihengye.cn, "PagedAttention", section "KV Cache 共享机制"; the
 * explainer's section "Copy-on-Write（CoW）によるメモリ共有"), so their
 * attention reads the same prompt K/V several times.  Here sequences
 * group_start[g] .. group_start[g+1]-1 form group g, and the first
 * group_prefix[g] tokens of every member are held in the same physical
 * blocks (precondition: the members' tables name the same ids for those
 * blocks; the group's first sequence's table is read).  The first
 * floor(group_prefix[g] / partition_size) partitions of the members are
 * computed once for the whole group on the matrix cores, with all members'
 * queries together; the remaining partitions of every sequence run as in
 * pa_decode and the same log-sum-exp merge combines them.  The result equals
 * pa_decode's up to the order of floating-point operations.
 *
 *   group_start   [num_groups + 1] int32, device: non-decreasing, from 0 to
 *                 num_seqs (otherwise results are undefined, without access
 *                 outside the arguments)
 *   group_prefix  [num_groups] int32, device: shared tokens of each group
 *   max_group_size, max_prefix_len   host bounds that size the grid: members
 *                 past the first max_group_size of a group are computed alone,
 *                 and prefixes are shared up to max_prefix_len tokens
 *   key, value    optional (both NULL, or both set): each sequence's newest
 *                 token, stored first as by pa_decode_append; that token must
 *                 lie past its group's shared tokens (its block is the
 *                 sequence's own)
 *   other arguments: as for pa_decode (same workspace size).
 * A member holding fewer tokens than its group's shared partitions is
 * computed alone; so is a whole group whose first sequence is that short.
 * Shapes the matrix-core path does not cover (FP8 or F32 KV, head_dim 64,
 * G = 16), an `out` that is not 16-byte aligned and num_groups == 0 run
 * pa_decode unchanged.
 */
int pa_decode_shared_prefix(void* out, int out_dtype, const void* q, int q_dtype, const void* k_cache,
                            const void* v_cache, int kv_dtype, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_seqs,
                            int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            float scale, const float* k_scale, const float* v_scale, int partition_size,
                            void* workspace, size_t workspace_bytes, void* stream, const int32_t* group_start,
                            const int32_t* group_prefix, int num_groups, int max_group_size,
                            int max_prefix_len, const void* key, const void* value);

/*
 * pa_prefill -- multi-query (prefill or chunked prefill) attention over the
 * same paged K/V.
 *
 * A prefill step attends for many new tokens of a sequence at once; its
 * computational shape differs from a decode step's (auturnal.com, "メモリ予
 * 算内での言語モデルのサービング", section 7).  The new tokens' keys and values
 * are first written into the sequence's blocks (pa_reshape_and_cache); then
 * each new token's query attends to the cached tokens up to its own position.
 * For sequence i with T = seq_lens[i] and Q = query_start[i+1] -
 * query_start[i], packed query row r = query_start[i] + j (j < Q) sits at
 * position p = T - Q + j, and for query head h (kv head h / G):
 *     out[r][h][:] = softmax(scale * K_i[0..p] q[r][h]) V_i[0..p]
 * (0h-n0.github.io explainer, section "Attention計算", restricted to the keys
 * up to p).  Q == T is a full prefill, Q < T a chunk appended to a context.
 *
 * Method: one workgroup per (tile of 128/G query tokens of one sequence, kv
 * head); the tile's 128 (token, head) columns share each staged 32-key K/V
 * step, and
 * the score and value products run on the matrix cores (v_mfma_f32_16x16x32,
 * fp32 accumulation; softmax weights enter the value product as a 16-bit
 * high part plus remainder) with the online-softmax recurrence of equation
 * (4) of the same review per column.
 *
 *   out          [total_q][num_heads][head_dim], out_dtype (F32, F16 or BF16),
 *                16-byte aligned
 *   q            [total_q][num_heads][head_dim], q_dtype, 16-byte aligned
 *   query_start  [num_seqs + 1] int32, device; non-decreasing, last = total_q
 *   max_query_len  host upper bound of the per-sequence query counts (sizes
 *                the grid); at most max_seq_len
 *   k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
 *   max_seq_len, num_blocks, scale: as for pa_decode.
 * Rows of a sequence whose length is invalid (0, above max_seq_len, needing
 * more than max_blocks_per_seq blocks, or shorter than its query count), or
 * whose table names a block outside the pool, are NaN.
 *
 * Supported: head_dim 128; block_size 16 or 32; G in {1, 2, 4, 8};
 * (kv_dtype, q_dtype) = (BF16, BF16) or (F16, F16); other valid formats return
 * PA_ERR_UNSUPPORTED.  total_q == 0 is a valid no-op.
 */
int pa_prefill(void* out, int out_dtype, const void* q, int q_dtype, const int32_t* query_start,
               int total_q, int max_query_len, const void* k_cache, const void* v_cache, int kv_dtype,
               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
               int max_seq_len, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
               int block_size, int num_blocks, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
