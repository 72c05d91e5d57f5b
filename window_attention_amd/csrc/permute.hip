// win_permute / win_transition: whole-row copies between token orders.
//
// Page "Window-Aligned Sequence Parallelism (SeedVR2)": the entry
// distribution and final reconstruction of section "SeedVR2 integration", and
// the layout change of sections "Motivation" / "Plan A redistribution", which
// on one device is a local permutation of rows.  A transition is done in one
// pass with the composed index inv_src[perm_dst[j]] instead of a scatter to
// canonical order followed by a gather.
//
// These kernels are pure HBM traffic: one read and one write of every row.
// Each wave copies one row per step with 16-byte lanes, so a wave moves a
// contiguous 1 KiB per instruction; the row index is wave-uniform and comes
// from a scalar load.  Loads and stores are marked non-temporal: every byte is
// touched exactly once.
#include "common.h"

namespace winattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Measured on the 21x45x80 regular-layout gather of 6 KiB rows: 4 chunks in
// flight per lane (a row in two passes) with one wave per block moves
// ~5.9 TB/s; 8 per lane with 4 waves per block ~5.5 TB/s (more registers,
// fewer waves resident).
constexpr int kWavesPerBlock = 1;
constexpr int kUnroll = 4;  // 16-byte chunks in flight per lane

enum PermuteMode { kGather = 0, kScatter = 1, kTransition = 2 };

__device__ __forceinline__ int32_t clamp_index(int32_t x, int32_t L) { return x < 0 ? 0 : (x >= L ? L - 1 : x); }

template <int MODE>
__global__ __launch_bounds__(kWavesPerBlock * 64) void permute_rows_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, const int32_t* __restrict__ idx_a,
    const int32_t* __restrict__ idx_b, int32_t L, uint32_t rows, uint32_t cpr) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t r = blockIdx.x * kWavesPerBlock + wave;
    if (r >= rows) return;
    const uint32_t b = r / (uint32_t)L;
    const uint32_t l = r - b * (uint32_t)L;
    uint64_t src_row, dst_row;
    if (MODE == kGather) {
        src_row = (uint64_t)b * L + clamp_index(idx_a[l], L);
        dst_row = r;
    } else if (MODE == kScatter) {
        src_row = r;
        dst_row = (uint64_t)b * L + clamp_index(idx_a[l], L);
    } else {
        src_row = (uint64_t)b * L + clamp_index(idx_a[clamp_index(idx_b[l], L)], L);
        dst_row = r;
    }
    const u32x4* s = src + src_row * cpr;
    u32x4* d = dst + dst_row * cpr;
    for (uint32_t c0 = 0; c0 < cpr; c0 += 64 * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t c = c0 + u * 64 + lane;
            if (c < cpr) v[u] = __builtin_nontemporal_load(s + c);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t c = c0 + u * 64 + lane;
            if (c < cpr) __builtin_nontemporal_store(v[u], d + c);
        }
    }
}

int check_rows(const void* src, void* dst, int64_t L, int32_t batch, int64_t row_elems, int32_t dtype,
               uint32_t* rows, uint32_t* cpr) {
    if (L < 0 || batch <= 0 || row_elems <= 0) return WIN_EINVAL;
    const int eb = element_bytes(dtype);
    if (!eb) return WIN_EUNSUPPORTED;
    if (L == 0) {  // nothing to copy; pointers are not used
        *rows = 0;
        *cpr = 0;
        return WIN_OK;
    }
    if (!src || !dst) return WIN_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return WIN_EUNSUPPORTED;
    if (L >= ((int64_t)1 << 31) || row_elems >= ((int64_t)1 << 33)) return WIN_EOVERFLOW;
    const int64_t row_bytes = row_elems * eb;
    if (row_bytes % 16) return WIN_EUNSUPPORTED;
    if (row_bytes / 16 >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    const int64_t nrows = L * batch;
    if (nrows >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if (row_bytes > ((int64_t)1 << 62) / nrows) return WIN_EOVERFLOW;  // tensor bytes stay below 2^62
    if (overlaps(src, (uint64_t)(nrows * row_bytes), dst, (uint64_t)(nrows * row_bytes))) return WIN_EINVAL;
    *rows = (uint32_t)nrows;
    *cpr = (uint32_t)(row_bytes / 16);
    return WIN_OK;
}

template <int MODE>
int launch(const void* src, void* dst, const int32_t* a, const int32_t* b, int64_t L, uint32_t rows, uint32_t cpr,
           void* stream) {
    if (rows == 0) return WIN_OK;
    const uint32_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    permute_rows_kernel<MODE><<<dim3(blocks), dim3(kWavesPerBlock * 64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), a, b, (int32_t)L, rows, cpr);
    return launch_status();
}

}  // namespace
}  // namespace winattn

using namespace winattn;

extern "C" int win_permute(const void* src, void* dst, const int32_t* idx, int64_t L, int32_t batch,
                           int64_t row_elems, int32_t dtype, int32_t mode, void* stream) {
    uint32_t rows = 0, cpr = 0;
    const int st = check_rows(src, dst, L, batch, row_elems, dtype, &rows, &cpr);
    if (st != WIN_OK) return st;
    if (!idx && L > 0) return WIN_EINVAL;
    if (mode == WIN_GATHER) return launch<kGather>(src, dst, idx, nullptr, L, rows, cpr, stream);
    if (mode == WIN_SCATTER) return launch<kScatter>(src, dst, idx, nullptr, L, rows, cpr, stream);
    return WIN_EINVAL;
}

extern "C" int win_transition(const void* src, void* dst, const int32_t* inv_src, const int32_t* perm_dst, int64_t L,
                              int32_t batch, int64_t row_elems, int32_t dtype, void* stream) {
    uint32_t rows = 0, cpr = 0;
    const int st = check_rows(src, dst, L, batch, row_elems, dtype, &rows, &cpr);
    if (st != WIN_OK) return st;
    if ((!inv_src || !perm_dst) && L > 0) return WIN_EINVAL;
    return launch<kTransition>(src, dst, inv_src, perm_dst, L, rows, cpr, stream);
}
