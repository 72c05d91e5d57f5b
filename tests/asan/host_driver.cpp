// Host entry points of libwinattn under AddressSanitizer.  Every table is a
// heap buffer of exactly the size include/winattn.h documents, so a read or
// write one element past it aborts the run.  Sweeps grids, window counts,
// both methods, rank counts and packing alignments; prints "ok <calls>".
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "winattn.h"

namespace {
int calls = 0;

int32_t* ialloc(size_t n) { return static_cast<int32_t*>(std::malloc((n ? n : 1) * sizeof(int32_t))); }
int64_t* lalloc(size_t n) { return static_cast<int64_t*>(std::malloc((n ? n : 1) * sizeof(int64_t))); }

bool check(int st, const char* what) {
    ++calls;
    if (st != WIN_OK) std::fprintf(stderr, "%s failed: %d (%s)\n", what, st, win_strerror(st));
    return st == WIN_OK;
}

struct HostPlan {
    win_plan_info info;
    int32_t *perm = nullptr, *inv = nullptr, *cu = nullptr, *boxes = nullptr;
    ~HostPlan() {
        std::free(perm);
        std::free(inv);
        std::free(cu);
        std::free(boxes);
    }
};

bool make_plan(int T, int H, int W, int nt, int nh, int nw, int method, HostPlan& p) {
    if (!check(win_plan(T, H, W, nt, nh, nw, method, &p.info, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
               "win_plan (size query)"))
        return false;
    const size_t L = (size_t)p.info.num_tokens, N = (size_t)p.info.num_windows;
    p.perm = ialloc(L);
    p.inv = ialloc(L);
    p.cu = ialloc(N + 1);
    p.boxes = ialloc(6 * N);
    return check(win_plan(T, H, W, nt, nh, nw, method, &p.info, p.perm, p.inv, p.cu, p.boxes, 0, nullptr),
                 "win_plan (fill)");
}

bool sweep_one(const int g[3], const int c[3]) {
    HostPlan pr, ps;
    if (!make_plan(g[0], g[1], g[2], c[0], c[1], c[2], 0, pr) || !make_plan(g[0], g[1], g[2], c[0], c[1], c[2], 1, ps))
        return false;
    const int64_t L = pr.info.num_tokens;

    // window-local coordinates, both layouts
    for (int method = 0; method < 2; ++method) {
        int32_t* local = ialloc(3 * (size_t)L);
        const bool ok = check(win_plan_local(g[0], g[1], g[2], c[0], c[1], c[2], method, local, 0, nullptr),
                              "win_plan_local");
        std::free(local);
        if (!ok) return false;
    }

    // rotary tables for the window extents
    for (int rope_dim : {6, 60, 126}) {
        const size_t rows = (size_t)ps.info.wt + ps.info.wh + ps.info.ww;
        float* table = static_cast<float*>(std::malloc(rows * (rope_dim / 3) * sizeof(float)));
        const bool ok = check(win_rope_table(ps.info.wt, ps.info.wh, ps.info.ww, 58, rope_dim, 10000.0, table),
                              "win_rope_table");
        std::free(table);
        if (!ok) return false;
    }

    // LPT assignments and Plan A tables from the regular to the shifted layout
    for (int ranks : {1, 2, 3, 8, 64}) {
        const int NR = pr.info.num_windows, NS = ps.info.num_windows;
        int32_t *own_r = ialloc(NR), *ord_r = ialloc(NR), *off_r = ialloc(ranks + 1);
        int32_t *own_s = ialloc(NS), *ord_s = ialloc(NS), *off_s = ialloc(ranks + 1);
        int64_t* tok = lalloc(ranks);
        int64_t* cnt = lalloc((size_t)ranks * ranks);
        int32_t *send = ialloc(L), *recv = ialloc(L);
        int32_t xreq = 0;
        const bool ok = check(win_lpt(NR, pr.cu, ranks, own_r, ord_r, off_r, tok), "win_lpt (regular)") &&
                        check(win_lpt(NS, ps.cu, ranks, own_s, ord_s, off_s, tok), "win_lpt (shifted)") &&
                        check(win_plan_a(L, ranks, pr.perm, pr.cu, NR, ord_r, off_r, ps.perm, ps.cu, NS, ord_s, off_s,
                                         cnt, send, recv, &xreq),
                              "win_plan_a");
        for (void* x : {(void*)own_r, (void*)ord_r, (void*)off_r, (void*)own_s, (void*)ord_s, (void*)off_s, (void*)tok,
                        (void*)cnt, (void*)send, (void*)recv})
            std::free(x);
        if (!ok) return false;
    }

    // the two layouts and the regular one again, packed as one call
    for (int align : {1, 7, 64, 1000}) {
        const HostPlan* ps3[3] = {&pr, &ps, &pr};
        int64_t nt[3];
        int32_t nw[3];
        std::vector<int32_t> perms, cus;
        int64_t total = 0;
        size_t segs = 1;
        for (int r = 0; r < 3; ++r) {
            nt[r] = L;
            nw[r] = ps3[r]->info.num_windows;
            perms.insert(perms.end(), ps3[r]->perm, ps3[r]->perm + L);
            cus.insert(cus.end(), ps3[r]->cu, ps3[r]->cu + nw[r] + 1);
            total += L + (align - L % align) % align;
            segs += (size_t)nw[r] + 1;
        }
        int32_t* perms_h = ialloc(perms.size());
        int32_t* cus_h = ialloc(cus.size());
        std::memcpy(perms_h, perms.data(), perms.size() * sizeof(int32_t));
        std::memcpy(cus_h, cus.data(), cus.size() * sizeof(int32_t));
        int64_t* off = lalloc(4);
        int32_t* perm_out = ialloc((size_t)total);
        int32_t* cu_out = ialloc(segs);
        int32_t mx = 0;
        const bool ok = check(win_pack(3, nt, nw, perms_h, cus_h, align, off, perm_out, cu_out, &mx), "win_pack");
        for (void* x : {(void*)perms_h, (void*)cus_h, (void*)off, (void*)perm_out, (void*)cu_out}) std::free(x);
        if (!ok) return false;
    }
    return true;
}
}  // namespace

int main() {
    const int grids[][3] = {{1, 3, 4}, {2, 5, 7}, {3, 6, 6}, {5, 9, 16}, {6, 11, 5}, {7, 4, 13}, {31, 3, 2}, {4, 45, 80}};
    const int counts[][3] = {{1, 1, 1}, {2, 3, 3}, {4, 3, 3}, {1, 26, 35}, {3, 17, 9}, {8, 2, 5}};
    for (const auto& g : grids)
        for (const auto& c : counts)
            if (!sweep_one(g, c)) return 1;
    // rejected arguments touch no buffer
    win_plan_info info;
    if (win_plan(0, 3, 4, 1, 1, 1, 0, &info, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != WIN_EINVAL) return 1;
    int32_t cu_bad[3] = {0, 5, 3};
    int32_t owner[2], order[2], offs[3];
    int64_t tok[2];
    if (win_lpt(2, cu_bad, 2, owner, order, offs, tok) != WIN_EINVAL) return 1;
    std::printf("ok %d\n", calls);
    return 0;
}
