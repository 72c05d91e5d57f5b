// win_plan: window sizes, axis segmentation and the integer tables of one
// layout (page "Window-Aligned Sequence Parallelism (SeedVR2)", section
// "Window layouts").  Built with -ffp-contract=off: the three double
// operations of the size formula must round exactly as written.
#include <cmath>

#include "common.h"
#include "plan_geometry.h"

namespace winattn {
namespace {

constexpr int32_t kReferenceArea = 45 * 80;  // 720p post-patch token grid
constexpr int32_t kMaxTemporalWindow = 30;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// scale = sqrt(45*80 / (H*W)); extent = round-half-even(n * scale).
int64_t rescaled_extent(int32_t n, int32_t H, int32_t W) {
    const double scale = std::sqrt((double)kReferenceArea / ((double)H * (double)W));
    const double x = (double)n * scale;
    return (int64_t)std::nearbyint(x);  // default rounding mode: to nearest, ties to even
}

__global__ void fill_tokens_kernel(GridGeom g, int64_t L, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= L) return;
    const int64_t j = window_position(g, c);
    if (perm) perm[j] = (int32_t)c;
    if (inv) inv[c] = (int32_t)j;
}

__global__ void fill_local_kernel(GridGeom g, int64_t L, int32_t* __restrict__ local) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= L) return;
    const int64_t j = window_position(g, c);
    const LocalPos p = window_local(g, c);
    local[3 * j] = p.t;
    local[3 * j + 1] = p.h;
    local[3 * j + 2] = p.w;
}

__global__ void fill_windows_kernel(GridGeom g, int32_t N, int64_t L, int32_t* __restrict__ cu,
                                    int32_t* __restrict__ boxes) {
    const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i > N) return;
    if (i == N) {
        if (cu) cu[N] = (int32_t)L;
        return;
    }
    const int32_t st = i % g.t.nseg;
    const int32_t sh = (i / g.t.nseg) % g.h.nseg;
    const int32_t sw = i / (g.t.nseg * g.h.nseg);
    if (cu) cu[i] = (int32_t)window_offset(g, st, sh, sw);
    if (boxes) {
        int32_t* bx = boxes + 6 * (int64_t)i;
        bx[0] = axis_start(g.t, st);
        bx[1] = axis_end(g.t, st);
        bx[2] = axis_start(g.h, sh);
        bx[3] = axis_end(g.h, sh);
        bx[4] = axis_start(g.w, sw);
        bx[5] = axis_end(g.w, sw);
    }
}

}  // namespace
}  // namespace winattn

using namespace winattn;

extern "C" int win_plan(int32_t T, int32_t H, int32_t W, int32_t nt, int32_t nh, int32_t nw, int32_t method,
                        win_plan_info* info, int32_t* perm, int32_t* inv, int32_t* cu_seqlens, int32_t* boxes,
                        int32_t on_device, void* stream) {
    if (!info) return WIN_EINVAL;
    if (T <= 0 || H <= 0 || W <= 0 || nt <= 0 || nh <= 0 || nw <= 0) return WIN_EINVAL;
    if (method != WIN_METHOD_REGULAR && method != WIN_METHOD_SHIFTED) return WIN_EINVAL;
    if (on_device != 0 && on_device != 1) return WIN_EINVAL;
    const int64_t L = (int64_t)T * H * W;
    if (L >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;

    const int64_t rh = rescaled_extent(H, H, W), rw = rescaled_extent(W, H, W);
    if (rh <= 0 || rw <= 0) return WIN_EINVAL;
    const int64_t wh = ceil_div(rh, nh), ww = ceil_div(rw, nw);
    const int64_t wt = ceil_div(T < kMaxTemporalWindow ? T : kMaxTemporalWindow, nt);
    if (wh >= ((int64_t)1 << 31) || ww >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;

    const bool shifted = method == WIN_METHOD_SHIFTED;
    GridGeom g;
    g.T = T;
    g.H = H;
    g.W = W;
    g.t = make_axis(T, (int32_t)wt, shifted);
    g.h = make_axis(H, (int32_t)wh, shifted);
    g.w = make_axis(W, (int32_t)ww, shifted);
    const int64_t N = (int64_t)g.t.nseg * g.h.nseg * g.w.nseg;  // <= L

    info->wt = (int32_t)wt;
    info->wh = (int32_t)wh;
    info->ww = (int32_t)ww;
    info->segs_t = g.t.nseg;
    info->segs_h = g.h.nseg;
    info->segs_w = g.w.nseg;
    info->num_windows = (int32_t)N;
    info->max_seqlen = axis_max_len(g.t) * axis_max_len(g.h) * axis_max_len(g.w);
    info->num_tokens = L;

    if (!on_device) {
        for (int64_t c = 0; c < L; ++c) {
            const int64_t j = window_position(g, c);
            if (perm) perm[j] = (int32_t)c;
            if (inv) inv[c] = (int32_t)j;
        }
        for (int32_t sw = 0; sw < g.w.nseg; ++sw)
            for (int32_t sh = 0; sh < g.h.nseg; ++sh)
                for (int32_t st = 0; st < g.t.nseg; ++st) {
                    const int32_t i = window_index(g, st, sh, sw);
                    if (cu_seqlens) cu_seqlens[i] = (int32_t)window_offset(g, st, sh, sw);
                    if (boxes) {
                        int32_t* bx = boxes + 6 * (int64_t)i;
                        bx[0] = axis_start(g.t, st);
                        bx[1] = axis_end(g.t, st);
                        bx[2] = axis_start(g.h, sh);
                        bx[3] = axis_end(g.h, sh);
                        bx[4] = axis_start(g.w, sw);
                        bx[5] = axis_end(g.w, sw);
                    }
                }
        if (cu_seqlens) cu_seqlens[N] = (int32_t)L;
        return WIN_OK;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr int kThreads = 256;
    if (perm || inv) {
        const int64_t blocks = ceil_div(L, kThreads);
        fill_tokens_kernel<<<dim3((uint32_t)blocks), dim3(kThreads), 0, s>>>(g, L, perm, inv);
        if (launch_status() != WIN_OK) return WIN_EDEVICE;
    }
    if (cu_seqlens || boxes) {
        const int64_t blocks = ceil_div(N + 1, kThreads);
        fill_windows_kernel<<<dim3((uint32_t)blocks), dim3(kThreads), 0, s>>>(g, (int32_t)N, L, cu_seqlens, boxes);
        if (launch_status() != WIN_OK) return WIN_EDEVICE;
    }
    return WIN_OK;
}

// win_pack: several requests' window plans packed into one varlen call (page
// "vLLM-Omni diffusion runtime", section 4.2 on packing): request r's rows
// follow those of the requests before it, padded by an alignment tail; its
// windows, moved by its row offset, and then its tail are segments of their
// own (a zero-length tail keeps its repeated boundary); the gather index of a
// row gets the request's offset added, and tail rows stay in place.  Host
// integer work: everything is validated before anything is written.
extern "C" int win_pack(int32_t num_requests, const int64_t* num_tokens, const int32_t* num_windows,
                        const int32_t* perms, const int32_t* cu_seqlens, int32_t align, int64_t* offsets,
                        int32_t* perm_out, int32_t* cu_out, int32_t* max_seqlen) {
    if (num_requests <= 0 || !num_tokens || !num_windows || !cu_seqlens || align <= 0) return WIN_EINVAL;
    if (!offsets || !cu_out || !max_seqlen || (perm_out && !perms)) return WIN_EINVAL;
    int64_t total = 0, longest = 0;
    const int32_t* c = cu_seqlens;
    const int32_t* p = perms;
    for (int32_t r = 0; r < num_requests; ++r) {
        const int64_t L = num_tokens[r];
        const int32_t N = num_windows[r];
        if (L <= 0 || N <= 0 || L >= ((int64_t)1 << 31)) return L >= ((int64_t)1 << 31) ? WIN_EOVERFLOW : WIN_EINVAL;
        if (c[0] != 0 || c[N] != L) return WIN_EINVAL;
        for (int32_t i = 0; i < N; ++i) {
            if (c[i + 1] < c[i]) return WIN_EINVAL;
            longest = c[i + 1] - c[i] > longest ? c[i + 1] - c[i] : longest;
        }
        if (perm_out) {
            for (int64_t j = 0; j < L; ++j)
                if (p[j] < 0 || p[j] >= L) return WIN_EINVAL;
            p += L;
        }
        const int64_t pad = (align - L % align) % align;
        longest = pad > longest ? pad : longest;
        total += L + pad;
        if (total >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
        c += N + 1;
    }
    c = cu_seqlens;
    p = perms;
    int64_t k = 0, o = 0;
    cu_out[k++] = 0;
    for (int32_t r = 0; r < num_requests; ++r) {
        const int64_t L = num_tokens[r];
        const int32_t N = num_windows[r];
        const int64_t end = o + L + (align - L % align) % align;
        offsets[r] = o;
        for (int32_t i = 1; i <= N; ++i) cu_out[k++] = (int32_t)(o + c[i]);
        cu_out[k++] = (int32_t)end;
        if (perm_out) {
            for (int64_t j = 0; j < L; ++j) perm_out[o + j] = (int32_t)(o + p[j]);
            for (int64_t t = o + L; t < end; ++t) perm_out[t] = (int32_t)t;
            p += L;
        }
        c += N + 1;
        o = end;
    }
    offsets[num_requests] = o;
    *max_seqlen = (int32_t)longest;
    return WIN_OK;
}

// win_plan_local: window-local coordinates of every row of a layout's window
// order (page "Window-Aligned Sequence Parallelism (SeedVR2)", section
// "Reference quirks reproduced on purpose": rotary positions restart at 0 in
// every window).  Row j holds canonical token perm[j]; local[3j .. 3j+2] are
// its (t, h, w) minus its window's first (t, h, w).
extern "C" int win_plan_local(int32_t T, int32_t H, int32_t W, int32_t nt, int32_t nh, int32_t nw, int32_t method,
                              int32_t* local, int32_t on_device, void* stream) {
    if (!local) return WIN_EINVAL;
    win_plan_info info;
    const int st = win_plan(T, H, W, nt, nh, nw, method, &info, nullptr, nullptr, nullptr, nullptr, 0, nullptr);
    if (st != WIN_OK) return st;
    if (on_device != 0 && on_device != 1) return WIN_EINVAL;
    const bool shifted = method == WIN_METHOD_SHIFTED;
    GridGeom g;
    g.T = T;
    g.H = H;
    g.W = W;
    g.t = make_axis(T, info.wt, shifted);
    g.h = make_axis(H, info.wh, shifted);
    g.w = make_axis(W, info.ww, shifted);
    const int64_t L = info.num_tokens;
    if (!on_device) {
        for (int64_t c = 0; c < L; ++c) {
            const int64_t j = window_position(g, c);
            const LocalPos p = window_local(g, c);
            local[3 * j] = p.t;
            local[3 * j + 1] = p.h;
            local[3 * j + 2] = p.w;
        }
        return WIN_OK;
    }
    constexpr int kThreads = 256;
    const int64_t blocks = ceil_div(L, kThreads);
    fill_local_kernel<<<dim3((uint32_t)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(g, L, local);
    return launch_status() == WIN_OK ? WIN_OK : WIN_EDEVICE;
}
