// Host-side checks of device contents for the checked build of the library
// (compiled with PA_CHECK_CONTENTS=1; the release build contains none of
// this).  Each check copies the index arrays that a call is about to read to
// the host, synchronising the call's stream, and returns PA_ERR_CONTENT when
// they break the call's contract, before anything is launched:
//   - slots: inside the pool (or negative: skipped) and distinct;
//   - copy and swap pairs: ids inside their pools, destinations distinct, and
//     for a copy inside one pool no destination that is also a source;
//   - sequences: lengths in [0, max_seq_len] needing at most
//     max_blocks_per_seq blocks, and every table entry a sequence reads
//     naming a block of the pool;
//   - groups: group_start non-decreasing from 0 to num_seqs, prefixes not
//     negative, every member's table naming its group's first sequence's
//     blocks for the tokens they share, and (when the call appends) every
//     member's newest token past the shared tokens;
//   - prefill queries: query_start non-decreasing from 0 to total_q, and
//     each sequence's query count at most max_query_len and its length.
// The copies make these calls synchronous, so the checked build is for
// debugging, not for graph capture or timing.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "pagedattn.h"

namespace pa {
namespace check {

// n elements of a device (or pinned host) array, on the host.
template <class T>
inline int fetch(std::vector<T>& v, const T* src, size_t n, hipStream_t stream) {
    v.assign(n, T());
    if (n == 0) return PA_OK;
    if (hipMemcpyAsync(v.data(), src, n * sizeof(T), hipMemcpyDefault, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return PA_ERR_LAUNCH;
    }
    return PA_OK;
}

inline bool all_distinct(std::vector<int64_t> v) {
    std::sort(v.begin(), v.end());
    return std::adjacent_find(v.begin(), v.end()) == v.end();
}

inline int slots(const int64_t* slot_mapping, int num_tokens, int num_blocks, int block_size, hipStream_t stream) {
    std::vector<int64_t> s;
    const int st = fetch(s, slot_mapping, (size_t)num_tokens, stream);
    if (st != PA_OK) return st;
    const int64_t limit = (int64_t)num_blocks * block_size;
    std::vector<int64_t> used;
    for (int64_t x : s) {
        if (x >= limit) return PA_ERR_CONTENT;
        if (x >= 0) used.push_back(x);
    }
    return all_distinct(used) ? PA_OK : PA_ERR_CONTENT;
}

// same_pool: a copy inside one pool (destinations may not also be sources)
inline int pairs(const int64_t* block_pairs, int num_pairs, int src_blocks, int dst_blocks, bool same_pool,
                 hipStream_t stream) {
    std::vector<int64_t> p;
    const int st = fetch(p, block_pairs, 2 * (size_t)num_pairs, stream);
    if (st != PA_OK) return st;
    std::vector<int64_t> src, dst;
    for (int i = 0; i < num_pairs; ++i) {
        if (p[2 * i] < 0 || p[2 * i] >= src_blocks || p[2 * i + 1] < 0 || p[2 * i + 1] >= dst_blocks)
            return PA_ERR_CONTENT;
        src.push_back(p[2 * i]);
        dst.push_back(p[2 * i + 1]);
    }
    if (!all_distinct(dst)) return PA_ERR_CONTENT;
    if (same_pool) {
        std::sort(src.begin(), src.end());
        for (int64_t d : dst)
            if (std::binary_search(src.begin(), src.end(), d)) return PA_ERR_CONTENT;
    }
    return PA_OK;
}

// The sequences' lengths and tables; on success `lens` and `tables` hold them.
inline int sequences(const int32_t* seq_lens, const int32_t* block_tables, int num_seqs, int max_blocks_per_seq,
                     int max_seq_len, int block_size, int num_blocks, std::vector<int32_t>& lens,
                     std::vector<int32_t>& tables, hipStream_t stream) {
    int st = fetch(lens, seq_lens, (size_t)num_seqs, stream);
    if (st != PA_OK) return st;
    st = fetch(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq, stream);
    if (st != PA_OK) return st;
    for (int i = 0; i < num_seqs; ++i) {
        const int T = lens[i];
        if (T < 0 || T > max_seq_len) return PA_ERR_CONTENT;
        const int nb = (T + block_size - 1) / block_size;
        if (nb > max_blocks_per_seq) return PA_ERR_CONTENT;
        for (int k = 0; k < nb; ++k) {
            const int32_t b = tables[(size_t)i * max_blocks_per_seq + k];
            if (b < 0 || b >= num_blocks) return PA_ERR_CONTENT;
        }
    }
    return PA_OK;
}

inline int sequences(const int32_t* seq_lens, const int32_t* block_tables, int num_seqs, int max_blocks_per_seq,
                     int max_seq_len, int block_size, int num_blocks, hipStream_t stream) {
    std::vector<int32_t> lens, tables;
    return sequences(seq_lens, block_tables, num_seqs, max_blocks_per_seq, max_seq_len, block_size, num_blocks, lens,
                     tables, stream);
}

// `lens` and `tables` as returned by sequences().
// appending: the call also stores each sequence's newest token, which must
// then lie past its group's shared tokens.
inline int groups(const int32_t* group_start, const int32_t* group_prefix, int num_groups, int num_seqs,
                  int max_blocks_per_seq, int block_size, const std::vector<int32_t>& lens,
                  const std::vector<int32_t>& tables, bool appending, hipStream_t stream) {
    std::vector<int32_t> start, prefix;
    int st = fetch(start, group_start, (size_t)num_groups + 1, stream);
    if (st != PA_OK) return st;
    st = fetch(prefix, group_prefix, (size_t)num_groups, stream);
    if (st != PA_OK) return st;
    if (start[0] != 0 || start[num_groups] != num_seqs) return PA_ERR_CONTENT;
    for (int g = 0; g < num_groups; ++g) {
        if (start[g + 1] < start[g] || prefix[g] < 0) return PA_ERR_CONTENT;
        if (start[g + 1] == start[g]) continue;
        const int lead = start[g];
        if (appending)
            for (int i = lead; i < start[g + 1]; ++i)
                if (lens[i] > 0 && lens[i] - 1 < prefix[g]) return PA_ERR_CONTENT;
        for (int i = lead + 1; i < start[g + 1]; ++i) {
            // the blocks holding the tokens both sequences have of the shared prefix
            const int shared = std::min(prefix[g], std::min(lens[i], lens[lead]));
            const int nb = (shared + block_size - 1) / block_size;
            for (int k = 0; k < nb; ++k)
                if (tables[(size_t)i * max_blocks_per_seq + k] != tables[(size_t)lead * max_blocks_per_seq + k])
                    return PA_ERR_CONTENT;
        }
    }
    return PA_OK;
}

inline int queries(const int32_t* query_start, int num_seqs, int total_q, int max_query_len,
                   const std::vector<int32_t>& lens, hipStream_t stream) {
    std::vector<int32_t> qs;
    const int st = fetch(qs, query_start, (size_t)num_seqs + 1, stream);
    if (st != PA_OK) return st;
    if (qs[0] != 0 || qs[num_seqs] != total_q) return PA_ERR_CONTENT;
    for (int i = 0; i < num_seqs; ++i) {
        const int Q = qs[i + 1] - qs[i];
        if (Q < 0 || Q > max_query_len || Q > lens[i]) return PA_ERR_CONTENT;
    }
    return PA_OK;
}

}  // namespace check
}  // namespace pa
