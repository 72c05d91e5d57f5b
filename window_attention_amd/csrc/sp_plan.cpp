// Host tables of window-aligned sequence parallelism (page "Window-Aligned
// Sequence Parallelism (SeedVR2)", sections "Planner" and "Plan A
// redistribution"): the deterministic LPT assignment of windows to ranks, and
// the redistribution tables between two assignments.  Plain host integer
// work; every input is validated before any output is written.
#include <algorithm>
#include <queue>
#include <vector>

#include "../../include/winattn.h"

namespace {

bool valid_cu(const int32_t* cu, int32_t n, int64_t L) {
    if (cu[0] != 0 || cu[n] != L) return false;
    for (int32_t i = 0; i < n; ++i)
        if (cu[i + 1] < cu[i]) return false;
    return true;
}

// order / rank_offsets describe a partition of 0..n-1 into `ranks` lists.
bool valid_assignment(const int32_t* order, const int32_t* rank_offsets, int32_t n, int32_t ranks) {
    if (rank_offsets[0] != 0 || rank_offsets[ranks] != n) return false;
    for (int32_t r = 0; r < ranks; ++r)
        if (rank_offsets[r + 1] < rank_offsets[r]) return false;
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        if (order[i] < 0 || order[i] >= n || seen[order[i]]) return false;
        seen[order[i]] = 1;
    }
    return true;
}

// Rank and local row of every canonical token of one layout under one
// assignment: rank r holds its windows in listed order, tokens in plan order.
bool locate(int64_t L, const int32_t* perm, const int32_t* cu, const int32_t* order, const int32_t* rank_offsets,
            int32_t ranks, std::vector<int32_t>& rank_of, std::vector<int32_t>& local_of,
            std::vector<int64_t>& held) {
    rank_of.assign(L, -1);
    local_of.assign(L, -1);
    held.assign(ranks, 0);
    for (int32_t r = 0; r < ranks; ++r) {
        int64_t k = 0;
        for (int32_t i = rank_offsets[r]; i < rank_offsets[r + 1]; ++i) {
            const int32_t w = order[i];
            for (int32_t j = cu[w]; j < cu[w + 1]; ++j) {
                const int32_t c = perm[j];
                if (c < 0 || c >= L || rank_of[c] >= 0) return false;  // not a permutation
                rank_of[c] = r;
                local_of[c] = (int32_t)k++;
            }
        }
        held[r] = k;
    }
    return true;
}

}  // namespace

extern "C" int win_lpt(int32_t num_windows, const int32_t* cu_seqlens, int32_t ranks, int32_t* owner, int32_t* order,
                       int32_t* rank_offsets, int64_t* rank_tokens) {
    if (num_windows < 0 || ranks <= 0 || !cu_seqlens || !owner || !order || !rank_offsets || !rank_tokens)
        return WIN_EINVAL;
    if (!valid_cu(cu_seqlens, num_windows, cu_seqlens[num_windows])) return WIN_EINVAL;
    // windows by (-tokens, window id)
    std::vector<int32_t> byload(num_windows);
    for (int32_t w = 0; w < num_windows; ++w) byload[w] = w;
    auto size = [&](int32_t w) { return cu_seqlens[w + 1] - cu_seqlens[w]; };
    std::sort(byload.begin(), byload.end(), [&](int32_t a, int32_t b) {
        return size(a) != size(b) ? size(a) > size(b) : a < b;
    });
    // each to the rank with the smallest (assigned tokens, rank id)
    typedef std::pair<int64_t, int32_t> Load;
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int32_t r = 0; r < ranks; ++r) heap.push(Load(0, r));
    std::vector<int32_t> own(num_windows);
    std::vector<int64_t> tokens(ranks, 0);
    for (int32_t w : byload) {
        const Load top = heap.top();
        heap.pop();
        own[w] = top.second;
        tokens[top.second] = top.first + size(w);
        heap.push(Load(tokens[top.second], top.second));
    }
    // each rank lists its windows in ascending id
    std::vector<int32_t> count(ranks + 1, 0);
    for (int32_t w = 0; w < num_windows; ++w) ++count[own[w] + 1];
    for (int32_t r = 0; r < ranks; ++r) count[r + 1] += count[r];
    for (int32_t r = 0; r <= ranks; ++r) rank_offsets[r] = count[r];
    for (int32_t w = 0; w < num_windows; ++w) {
        owner[w] = own[w];
        order[count[own[w]]++] = w;
    }
    for (int32_t r = 0; r < ranks; ++r) rank_tokens[r] = tokens[r];
    return WIN_OK;
}

extern "C" int win_plan_a(int64_t L, int32_t ranks, const int32_t* src_perm, const int32_t* src_cu,
                          int32_t src_windows, const int32_t* src_order, const int32_t* src_rank_offsets,
                          const int32_t* dst_perm, const int32_t* dst_cu, int32_t dst_windows,
                          const int32_t* dst_order, const int32_t* dst_rank_offsets, int64_t* counts,
                          int32_t* send_rows, int32_t* recv_pos, int32_t* exchange_required) {
    if (L <= 0 || ranks <= 0 || src_windows <= 0 || dst_windows <= 0) return WIN_EINVAL;
    if (L >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if (!src_perm || !src_cu || !src_order || !src_rank_offsets || !dst_perm || !dst_cu || !dst_order ||
        !dst_rank_offsets || !counts || !send_rows || !recv_pos || !exchange_required)
        return WIN_EINVAL;
    if (!valid_cu(src_cu, src_windows, L) || !valid_cu(dst_cu, dst_windows, L)) return WIN_EINVAL;
    if (!valid_assignment(src_order, src_rank_offsets, src_windows, ranks) ||
        !valid_assignment(dst_order, dst_rank_offsets, dst_windows, ranks))
        return WIN_EINVAL;
    std::vector<int32_t> src_rank, src_local, dst_rank, dst_local;
    std::vector<int64_t> src_held, dst_held;
    if (!locate(L, src_perm, src_cu, src_order, src_rank_offsets, ranks, src_rank, src_local, src_held) ||
        !locate(L, dst_perm, dst_cu, dst_order, dst_rank_offsets, ranks, dst_rank, dst_local, dst_held))
        return WIN_EINVAL;

    const int64_t P = ranks;
    std::vector<int64_t> C(P * P, 0);
    // destination tokens in (destination rank, destination-local position) order
    std::vector<int32_t> dst_tokens(L);
    {
        std::vector<int64_t> base(P + 1, 0);
        for (int64_t d = 0; d < P; ++d) base[d + 1] = base[d] + dst_held[d];
        for (int64_t c = 0; c < L; ++c) dst_tokens[base[dst_rank[c]] + dst_local[c]] = (int32_t)c;
    }
    for (int64_t t = 0; t < L; ++t) {
        const int32_t c = dst_tokens[t];
        ++C[(int64_t)src_rank[c] * P + dst_rank[c]];
    }
    // send rows: source rank r's block (at its first row in source-rank order)
    // takes its rows as the destinations need them, destination by
    // destination, each in destination-local order
    std::vector<int64_t> send_cur(P, 0), recv_cur(P * P, 0);
    for (int64_t r = 1; r < P; ++r) send_cur[r] = send_cur[r - 1] + src_held[r - 1];
    // receive positions: destination d's block takes, source rank by source
    // rank, the destination-local positions of the rows that rank sends
    {
        int64_t start = 0;
        for (int64_t d = 0; d < P; ++d) {
            int64_t k = start;
            for (int64_t r = 0; r < P; ++r) {
                recv_cur[d * P + r] = k;
                k += C[r * P + d];
            }
            start += dst_held[d];
        }
    }
    for (int64_t t = 0; t < L; ++t) {
        const int32_t c = dst_tokens[t];
        const int64_t r = src_rank[c], d = dst_rank[c];
        send_rows[send_cur[r]++] = src_local[c];
        recv_pos[recv_cur[d * P + r]++] = dst_local[c];
    }
    int32_t ex = 0;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t d = 0; d < P; ++d) {
            counts[r * P + d] = C[r * P + d];
            if (r != d && C[r * P + d]) ex = 1;
        }
    *exchange_required = ex;
    return WIN_OK;
}
