// Closed-form window geometry shared by the host planner and the device
// table-fill kernel.
//
// Page "Window-Aligned Sequence Parallelism (SeedVR2)", section "Window
// layouts".  One axis of extent n with window w is cut into segments:
//   regular: [k*w, min((k+1)*w, n))
//   shifted: every regular cut moved back by half a window, the windows
//            clipped to [0, n]; for odd w the moved cut is the truncated slice
//            index, so the cuts are floor(w/2), floor(w/2) + w, ...  An axis
//            one window already covers (w >= n) keeps the single segment
//            [0, n); with w == 1 the empty first segment disappears and the
//            layout equals the regular one.
// Both cases are "a first segment of length `first`, then full windows of w,
// the last one clipped at n", which is what AxisGeom stores.  Windows are the
// products of axis segments, enumerated w outermost, then h, then t, and
// tokens inside a window are row-major in (t, h, w), so the window-order
// position of a token and the start of every window have closed forms.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define WIN_HD __host__ __device__ inline
#else
#define WIN_HD inline
#endif

namespace winattn {

struct AxisGeom {
    int32_t n;      // extent
    int32_t w;      // window extent
    int32_t first;  // length of segment 0 (1 <= first <= n)
    int32_t nseg;   // number of segments
};

WIN_HD AxisGeom make_axis(int32_t n, int32_t w, bool shifted) {
    AxisGeom a;
    a.n = n;
    a.w = w;
    if (w >= n) {
        a.first = n;
    } else if (shifted && w / 2 > 0) {
        a.first = w / 2;
    } else {
        a.first = w;
    }
    a.nseg = a.first >= n ? 1 : 1 + (n - a.first + w - 1) / w;
    return a;
}

// Segment index of coordinate x (0 <= x < n).
WIN_HD int32_t axis_seg(const AxisGeom& a, int32_t x) { return x < a.first ? 0 : 1 + (x - a.first) / a.w; }

WIN_HD int32_t axis_start(const AxisGeom& a, int32_t s) { return s == 0 ? 0 : a.first + (s - 1) * a.w; }

WIN_HD int32_t axis_end(const AxisGeom& a, int32_t s) {
    const int64_t e = (int64_t)a.first + (int64_t)s * a.w;
    return e < a.n ? (int32_t)e : a.n;
}

// Longest segment: segment 0, or segment 1 (a full window, or the clipped
// tail when it is also the last); later segments are never longer.
WIN_HD int32_t axis_max_len(const AxisGeom& a) {
    if (a.nseg == 1) return a.first;
    const int32_t rest = a.n - a.first;
    const int32_t s1 = rest < a.w ? rest : a.w;
    return s1 > a.first ? s1 : a.first;
}

struct GridGeom {
    AxisGeom t, h, w;
    int32_t T, H, W;
};

// Window-order offset of the first token of window (st, sh, sw): all windows
// of earlier w-segments cover the full (t, h) extent, earlier h-segments of
// the same w-segment cover the full t extent.
WIN_HD int64_t window_offset(const GridGeom& g, int32_t st, int32_t sh, int32_t sw) {
    const int64_t ws = axis_start(g.w, sw), wl = axis_end(g.w, sw) - ws;
    const int64_t hs = axis_start(g.h, sh), hl = axis_end(g.h, sh) - hs;
    const int64_t ts = axis_start(g.t, st);
    return ws * g.H * g.T + hs * wl * g.T + ts * hl * wl;
}

// Window index of (st, sh, sw) in enumeration order.
WIN_HD int32_t window_index(const GridGeom& g, int32_t st, int32_t sh, int32_t sw) {
    return (sw * g.h.nseg + sh) * g.t.nseg + st;
}

// Window-order position of canonical token c.
WIN_HD int64_t window_position(const GridGeom& g, int64_t c) {
    const int32_t t = (int32_t)(c / ((int64_t)g.H * g.W));
    const int32_t rem = (int32_t)(c - (int64_t)t * g.H * g.W);
    const int32_t h = rem / g.W, w = rem - h * g.W;
    const int32_t st = axis_seg(g.t, t), sh = axis_seg(g.h, h), sw = axis_seg(g.w, w);
    const int64_t ts = axis_start(g.t, st);
    const int64_t hs = axis_start(g.h, sh), hl = axis_end(g.h, sh) - hs;
    const int64_t ws = axis_start(g.w, sw), wl = axis_end(g.w, sw) - ws;
    return window_offset(g, st, sh, sw) + ((t - ts) * hl + (h - hs)) * wl + (w - ws);
}

// Window-local coordinates of canonical token c: its (t, h, w) minus the first
// coordinate of its window on each axis.
struct LocalPos {
    int32_t t, h, w;
};

WIN_HD LocalPos window_local(const GridGeom& g, int64_t c) {
    const int32_t t = (int32_t)(c / ((int64_t)g.H * g.W));
    const int32_t rem = (int32_t)(c - (int64_t)t * g.H * g.W);
    const int32_t h = rem / g.W, w = rem - h * g.W;
    LocalPos p;
    p.t = t - axis_start(g.t, axis_seg(g.t, t));
    p.h = h - axis_start(g.h, axis_seg(g.h, h));
    p.w = w - axis_start(g.w, axis_seg(g.w, w));
    return p;
}

}  // namespace winattn
