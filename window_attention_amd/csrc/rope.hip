// win_permute_rope / win_rope_table: window-local 3D rotary position
// embedding of query and key rows, fused into the gather into a window layout
// or the transition between two layouts.
//
// Page "Window-Aligned Sequence Parallelism (SeedVR2)", section "Reference
// quirks reproduced on purpose": a video token at window-local (dt, dh, dw)
// rotates with axial indices (text_len + dt, dh, dw), every window restarting
// at 0; the rotary span is 3 * (rope_dim / 3) channels and the channels after
// it pass through.  Inside the span, three consecutive blocks of
// d = rope_dim / 3 channels hold the t, h and w axes, and channel pair
// (2i, 2i+1) of a block turns by position * base^(-2i/d) (the rotation of Su
// et al., RoFormer).  The row index of the permute and the position of the
// row are distinct: positions come from the destination layout's
// window-local table, never from the row index.
//
// The kernel is the permute's: one wave per row, 16-byte lanes, one read and
// one write of every byte, so the rotation rides on the same HBM traffic.  A
// lane's 16-byte chunks are 8 channels of successive heads; with 64 lanes and
// a head of a multiple of 8 channels dividing 512, every chunk of a lane
// holds the same 8 channels, so a lane fetches its four (cos, sin) pairs once
// per row from a small table and applies them to every head.
#include <cmath>

#include "common.h"

namespace winattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte chunks in flight per lane: 8 holds a whole 6 KiB row (24 heads x
// 128) in one pass; measured ~1-2 % above 4 and 6 on the 21x45x80 gather.
constexpr int kUnroll = 8;

__device__ __forceinline__ int32_t clamp_to(int32_t x, int32_t n) { return x < 0 ? 0 : (x >= n ? n - 1 : x); }

// One bf16 pair (x0 in the low half of w, x1 in the high half) turned by
// (c, s); pass-through pairs keep their bits.
__device__ __forceinline__ uint32_t turn(uint32_t w, f32x2 cs, bool rotate) {
    const float x0 = __builtin_bit_cast(float, w << 16);
    const float x1 = __builtin_bit_cast(float, w & 0xffff0000u);
    const f32x2 y = {fmaf(x0, cs[0], -x1 * cs[1]), fmaf(x0, cs[1], x1 * cs[0])};
    const uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
    return rotate ? r : w;
}

struct RopeArgs {
    const u32x4* src;
    u32x4* dst;
    const int32_t* idx;       // gather index (window order -> source row), or inv_src of a transition
    const int32_t* perm_dst;  // null for a gather
    const int32_t* local;     // [L * 3] window-local (dt, dh, dw) of the destination rows
    const f32x2* table;       // (cos, sin) per (axis row, pair)
    int32_t L;
    uint32_t rows;
    uint32_t cpr;             // 16-byte chunks per row
    int32_t head_chunks;      // head_dim / 8
    int32_t span_pairs;       // rotated pairs per head: 3 * (rope_dim / 3) / 2
    int32_t axis_pairs;       // pairs per axis block: (rope_dim / 3) / 2
    int32_t ext[3];           // window extents on t, h, w (rows of the table per axis)
};

// This lane's four (cos, sin) pairs, the same in every head of the row.  The
// row's three window-local coordinates are wave-uniform (scalar loads); a
// lane picks the one of its pairs' axis.
__device__ __forceinline__ void row_rotation(const RopeArgs& a, int32_t j, uint32_t lane, f32x2 (&cs)[4],
                                             bool (&rot)[4]) {
    const int32_t* lj = a.local + 3 * (int64_t)j;  // 3 j passes 2^31 before j does
    const int32_t loc[3] = {clamp_to(lj[0], a.ext[0]), clamp_to(lj[1], a.ext[1]), clamp_to(lj[2], a.ext[2])};
    const int32_t cb = (int32_t)lane % a.head_chunks;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int32_t p = cb * 4 + q;
        rot[q] = p < a.span_pairs;
        const int32_t axis = rot[q] ? p / a.axis_pairs : 0;
        const int32_t i = rot[q] ? p - axis * a.axis_pairs : 0;
        const int32_t row = axis == 0 ? loc[0] : (axis == 1 ? a.ext[0] + loc[1] : a.ext[0] + a.ext[1] + loc[2]);
        cs[q] = a.table[row * a.axis_pairs + i];
    }
}

__global__ __launch_bounds__(64) void rope_rows_kernel(RopeArgs a) {
    const uint32_t lane = threadIdx.x;
    const uint32_t r = blockIdx.x;
    if (r >= a.rows) return;
    const uint32_t b = r / (uint32_t)a.L;
    const int32_t j = (int32_t)(r - b * (uint32_t)a.L);
    const int32_t jj = a.perm_dst ? clamp_to(a.idx[clamp_to(a.perm_dst[j], a.L)], a.L) : clamp_to(a.idx[j], a.L);
    const u32x4* s = a.src + ((uint64_t)b * a.L + jj) * a.cpr;
    u32x4* d = a.dst + (uint64_t)r * a.cpr;
    f32x2 cs[4];
    bool rot[4];
    for (uint32_t c0 = 0; c0 < a.cpr; c0 += 64 * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t c = c0 + u * 64 + lane;
            if (c < a.cpr) v[u] = __builtin_nontemporal_load(s + c);
        }
        // the rotation's table reads go out behind the row's first loads
        if (c0 == 0) row_rotation(a, j, lane, cs, rot);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t c = c0 + u * 64 + lane;
            if (c < a.cpr) {
                u32x4 y;
#pragma unroll
                for (int q = 0; q < 4; ++q) y[q] = turn(v[u][q], cs[q], rot[q]);
                __builtin_nontemporal_store(y, d + c);
            }
        }
    }
}

}  // namespace
}  // namespace winattn

using namespace winattn;

extern "C" int win_rope_table(int32_t wt, int32_t wh, int32_t ww, int32_t text_len, int32_t rope_dim, double base,
                              float* table) {
    if (wt <= 0 || wh <= 0 || ww <= 0 || text_len < 0 || rope_dim < 6 || !table) return WIN_EINVAL;
    if (!(base > 1.0) || !std::isfinite(base)) return WIN_EINVAL;
    const int32_t d = rope_dim / 3;
    if (d % 2) return WIN_EUNSUPPORTED;
    const int32_t np = d / 2;
    const int32_t ext[3] = {wt, wh, ww};
    int64_t row = 0;
    for (int axis = 0; axis < 3; ++axis)
        for (int32_t p = 0; p < ext[axis]; ++p, ++row) {
            const double pos = (double)(axis == 0 ? text_len + p : p);
            for (int32_t i = 0; i < np; ++i) {
                const double ang = pos * std::pow(base, -2.0 * i / d);
                table[2 * (row * np + i)] = (float)std::cos(ang);
                table[2 * (row * np + i) + 1] = (float)std::sin(ang);
            }
        }
    return WIN_OK;
}

extern "C" int win_permute_rope(const void* src, void* dst, const int32_t* idx, const int32_t* perm_dst,
                                const int32_t* local, const float* table, int32_t wt, int32_t wh, int32_t ww,
                                int64_t L, int32_t batch, int32_t heads, int32_t head_dim, int32_t rope_dim,
                                void* stream) {
    if (L < 0 || batch <= 0 || heads <= 0 || wt <= 0 || wh <= 0 || ww <= 0) return WIN_EINVAL;
    if (head_dim != 64 && head_dim != 128) return WIN_EUNSUPPORTED;
    if (rope_dim < 6 || rope_dim > head_dim || (rope_dim / 3) % 2) return WIN_EUNSUPPORTED;
    if (L == 0) return WIN_OK;
    if (!src || !dst || !idx || !local || !table) return WIN_EINVAL;
    if (!aligned16(src) || !aligned16(dst) || (reinterpret_cast<uintptr_t>(table) & 7u)) return WIN_EUNSUPPORTED;
    if (L >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    const int64_t row_bytes = (int64_t)heads * head_dim * 2;
    const int64_t nrows = L * batch;
    if (nrows >= ((int64_t)1 << 31) || row_bytes / 16 >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if (row_bytes > ((int64_t)1 << 62) / nrows) return WIN_EOVERFLOW;  // tensor bytes stay below 2^62
    if (overlaps(src, (uint64_t)(nrows * row_bytes), dst, (uint64_t)(nrows * row_bytes))) return WIN_EINVAL;
    RopeArgs a;
    a.src = static_cast<const u32x4*>(src);
    a.dst = static_cast<u32x4*>(dst);
    a.idx = idx;
    a.perm_dst = perm_dst;
    a.local = local;
    a.table = reinterpret_cast<const f32x2*>(table);
    a.L = (int32_t)L;
    a.rows = (uint32_t)nrows;
    a.cpr = (uint32_t)(row_bytes / 16);
    a.head_chunks = head_dim / 8;
    a.span_pairs = 3 * (rope_dim / 3) / 2;
    a.axis_pairs = (rope_dim / 3) / 2;
    a.ext[0] = wt;
    a.ext[1] = wh;
    a.ext[2] = ww;
    rope_rows_kernel<<<dim3(a.rows), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(a);
    return launch_status();
}
