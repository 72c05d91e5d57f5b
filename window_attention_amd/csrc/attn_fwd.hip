// win_attn_fwd: variable-length window attention, forward, for gfx950.
//
// Page "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Motivation"
// (attention only inside each 3D window) and "SeedVR2 integration" (one packed
// variable-length call over cu_seqlens segments).  For each (batch, window,
// head) the kernel computes softmax(Q K^T * scale) V with a flash-style online
// softmax over key tiles, so the n x n score matrix never leaves registers.
//
// Mapping to CDNA4
//   * One workgroup = NW waves = a tile of 32*NW query rows of one (batch,
//     window, head).  Each wave owns 32 query rows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane holds
//     16 keys of ONE query column (lane % 32), so the softmax row max and row
//     sum are in-lane reductions plus one exchange with lane ^ 32.
//   * O^T = V^T P^T with the same instruction.  P^T is used straight from the
//     score registers as the B operand: the 8 keys a lane supplies for a
//     16-key step are the ones its accumulator already holds (keys
//     16j+4h+{0..3} and 16j+8+4h+{0..3}, h = lane / 32).  The V^T operand is
//     read with ds_read_b64_tr_b16, which returns four rows of one column per
//     lane, so V needs no transpose pass.  The O^T accumulator column is again
//     the lane's own query, so the online-softmax rescale is per lane.
//   * K and V tiles (64 keys) are copied HBM -> LDS with
//     global_load_lds_dwordx4 (no VGPR staging), double buffered.  Rows are
//     stored with an XOR swizzle of their 16-byte chunks so that the K reads
//     (32 rows, same chunk) and the transposed V reads (4 rows x 4 columns per
//     16 lanes) are spread over the LDS banks.
//   * Grid: blockIdx % 8 selects the XCD; all query tiles of one (batch,
//     window, head) go to the same XCD, consecutively, so they share its L2
//     while they stream the same K/V tiles.
//   * Rows past the end of a window are clamped to its last row on load and
//     masked to -inf as keys, so no access leaves the window's tensors.
#include <cmath>

#include "common.h"

namespace winattn {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;          // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* cu;
    int32_t num_windows;
    int32_t L;
    int32_t heads;
    int32_t qtiles;      // query tiles per (batch, window, head) in the grid
    int32_t pairs;       // batch * num_windows * heads
    float scale;         // softmax scale
    float scale_log2;    // softmax scale * log2(e)
};

template <int D>
struct Layout {
    static constexpr int kCPR = D / 8;                 // 16-byte chunks per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kSegs = kTileBytes / 1024;    // wave-wide 1 KiB copies per tile
    static constexpr int kRowsPerSeg = 1024 / kRowBytes;
    static constexpr int kVSwz = kCPR >= 16 ? 4 : 2;   // V chunk swizzle stride
    // physical 16-byte chunk of logical chunk c in row r
    __device__ static int k_chunk(int r, int c) { return c ^ (r & (kCPR - 1)); }
    __device__ static int v_chunk(int r, int c) { return c ^ (kVSwz * (r & 3)); }
};

// Value of x held by lane l ^ 32 (the other lane of this query column).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.  Swapping x against 0 twice moves each half of x
// to the other half and leaves 0 where the data did not come from, so the OR
// of the two results is the partner value.  (A single swap of x with itself
// would do, but the compiler treats the two results of swap(x, x) as equal.)
__device__ __forceinline__ float partner32(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto lo = __builtin_amdgcn_permlane32_swap(u, 0u, false, false);  // lanes 0-31 of [1] <- x[32..63]
    const auto hi = __builtin_amdgcn_permlane32_swap(0u, u, false, false);  // lanes 32-63 of [0] <- x[0..31]
    return __builtin_bit_cast(float, lo[1] | hi[0]);
}
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, partner32(x)); }
__device__ __forceinline__ float pair_sum(float x) { return x + partner32(x); }

// HBM -> LDS copy of one K or V tile (kBN rows of D bf16 starting at key kv0),
// each wave moving kSegs / NW wave-wide 1 KiB segments.  Row r of the tile
// lives at LDS byte r * kRowBytes with its chunks permuted by the swizzle.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void load_tile(const bf16* __restrict__ base, size_t row_stride, int kv0, int n,
                                          LDS_AS char* __restrict__ tile, int wave, int lane) {
    using Ly = Layout<D>;
    static_assert(Ly::kSegs % NW == 0, "tile copy must split evenly over waves");
#pragma unroll
    for (int i = 0; i < Ly::kSegs / NW; ++i) {
        const int seg = wave * (Ly::kSegs / NW) + i;
        const int row = seg * Ly::kRowsPerSeg + lane / Ly::kCPR;
        const int pc = lane % Ly::kCPR;
        const int lc = IS_V ? Ly::v_chunk(row, pc) : Ly::k_chunk(row, pc);  // xor swizzles are involutions
        int key = kv0 + row;
        key = key < n ? key : n - 1;
        const bf16* g = base + (size_t)key * row_stride + lc * 8;
        __builtin_amdgcn_global_load_lds((const void*)g, (LDS_AS void*)(tile + seg * 1024), 16, 0, 0);
    }
}

// Running state of one wave: 32 query rows, online softmax in base 2.
template <int D>
struct WaveState {
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    bf16x8 qf[KSTEPS];  // Q fragment (B operand of S^T = K Q^T)
    f32x16 oacc[DBLK];  // O^T accumulator: column = this lane's query
    float m_run;        // reference max of raw scores (equal in lanes l, l^32)
    float l_run;        // sum of the bf16 probabilities this lane contributed
    int koff[KSTEPS];   // LDS byte offsets of the K operand per k step
    int voff[DBLK];     // LDS byte offsets of the transposed V reads per O^T block
};

// Rescaling is deferred until a tile's max exceeds the reference max by this
// many powers of two, so probabilities stay below 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.f;

// One key tile: issue the copies of the next tile, then S^T, softmax and O^T
// update from the current tile.  The buffers are restrict-qualified so that
// the compiler knows the copies into *_next never alias the reads of *_cur.
template <int D, int NW>
__device__ __forceinline__ void attend_tile(WaveState<D>& st, const LDS_AS char* __restrict__ kcur,
                                            const LDS_AS char* __restrict__ vcur, LDS_AS char* __restrict__ knext,
                                            LDS_AS char* __restrict__ vnext, bool load_next, const bf16* kbase,
                                            const bf16* vbase, size_t row_stride, int kv_next, int n, int lim,
                                            float c, int wave, int lane) {
    using Ly = Layout<D>;
    constexpr int KSTEPS = WaveState<D>::KSTEPS;
    constexpr int DBLK = WaveState<D>::DBLK;
    const int h = lane >> 5;
    if (load_next) {
        load_tile<D, NW, false>(kbase, row_stride, kv_next, n, knext, wave, lane);
        load_tile<D, NW, true>(vbase, row_stride, kv_next, n, vnext, wave, lane);
    }
    // S^T block kb: rows = keys kb*32 .. +31, columns = this wave's queries
    f32x16 s[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const bf16x8 kf = *reinterpret_cast<const LDS_AS bf16x8*>(kcur + kb * 32 * Ly::kRowBytes + st.koff[t]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.qf[t], s[kb], 0, 0, 0);
        }
    }
    if (lim < kBN) {  // keys past the window end (last tile only)
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                s[kb][r] = key < lim ? s[kb][r] : -INFINITY;
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
    mx = pair_max(mx);
    const bool grow = (mx - st.m_run) * c > kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : st.m_run;
        const float alpha = __builtin_amdgcn_exp2f((st.m_run - m_new) * c);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    }
    const float mc = st.m_run * c;
    // P^T as bf16 B operands, one per 16-key step; the row sum adds the
    // rounded bf16 values, i.e. exactly the weights the P V product uses
    bf16x8 pb[kBN / 16];
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < kBN / 16; ++jj) {
        const int kb = jj >> 1, r0 = 8 * (jj & 1);
        f32x8 x;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i], c, -mc));
        pb[jj] = __builtin_convertvector(x, bf16x8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 pr = {pb[jj][2 * i], pb[jj][2 * i + 1]};
            rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
        }
    }
    st.l_run += rs;
    // O^T += V^T P^T
#pragma unroll
    for (int jj = 0; jj < kBN / 16; ++jj) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const LDS_AS char* a0 = vcur + st.voff[db] + (16 * jj) * Ly::kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * Ly::kRowBytes));
            const i16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[jj],
                                                                  st.oacc[db], 0, 0, 0);
        }
    }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(AttnParams p) {
    using Ly = Layout<D>;
    constexpr int BM = 32 * NW;
    constexpr int KSTEPS = WaveState<D>::KSTEPS;
    constexpr int DBLK = WaveState<D>::DBLK;
    __shared__ __attribute__((aligned(1024))) char smem[4 * Ly::kTileBytes];
    LDS_AS char* lds = (LDS_AS char*)smem;
    LDS_AS char* kbuf[2] = {lds, lds + Ly::kTileBytes};
    LDS_AS char* vbuf[2] = {lds + 2 * Ly::kTileBytes, lds + 3 * Ly::kTileBytes};

    // ---- work item: XCD-aware decomposition of blockIdx ------------------
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int pair = (slot / p.qtiles) * 8 + xcd;
    const int qt = slot % p.qtiles;
    if (pair >= p.pairs) return;
    const int head = pair % p.heads;
    const int bw = pair / p.heads;
    const int win = bw % p.num_windows;
    const int b = bw / p.num_windows;
    int start = p.cu[win], end = p.cu[win + 1];
    start = start < 0 ? 0 : (start > p.L ? p.L : start);
    end = end < start ? start : (end > p.L ? p.L : end);
    const int n = end - start;
    const int q0 = qt * BM;
    if (q0 >= n) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const size_t row_stride = (size_t)p.heads * D;
    const size_t base_off = ((size_t)b * p.L + start) * row_stride + (size_t)head * D;
    const bf16* kbase = p.k + base_off;
    const bf16* vbase = p.v + base_off;

    const int nkv = (n + kBN - 1) / kBN;
    load_tile<D, NW, false>(kbase, row_stride, 0, n, kbuf[0], wave, lane);
    load_tile<D, NW, true>(vbase, row_stride, 0, n, vbuf[0], wave, lane);

    WaveState<D> st;
    const int qrow = q0 + wave * 32 + (lane & 31);
    {
        const int qrow_c = qrow < n ? qrow : n - 1;
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(p.q + base_off + (size_t)qrow_c * row_stride);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) st.qf[t] = qp[2 * t + h];
    }
    // K (A operand of S^T): lane reads row (lane % 32) of a 32-key block,
    // logical chunk 2t + h.
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        const int r = lane & 31;
        st.koff[t] = r * Ly::kRowBytes + Ly::k_chunk(r, 2 * t + h) * 16;
    }
    // V (A operand of O^T, transposed read): address-supplying lane s of
    // 16-lane group g points at row 4*(g/2) + e, column 16*(g%2) + 4*c of a
    // 16-key x 32-column block (e = (s/4)%4, c = s%4); the transposed read
    // hands lane l the four rows 4*(l/32)+{0..3} of column l % 32.
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, c = lane & 3;
        const int r = 4 * (g >> 1) + e;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int lc = db * 4 + 2 * (g & 1) + (c >> 1);
            st.voff[db] = r * Ly::kRowBytes + Ly::v_chunk(r, lc) * 16 + (c & 1) * 8;
        }
    }
    st.m_run = -INFINITY;
    st.l_run = 0.f;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) st.oacc[db] = f32x16{};

    for (int j = 0; j < nkv; ++j) {
        const int cur = j & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile j have landed
        __syncthreads();                      // ... and every wave's; tile j-1 buffers are free
        const int lim = n - j * kBN;
        attend_tile<D, NW>(st, kbuf[cur], vbuf[cur], kbuf[cur ^ 1], vbuf[cur ^ 1], j + 1 < nkv, kbase, vbase,
                           row_stride, (j + 1) * kBN, n, lim, p.scale_log2, wave, lane);
    }

    // ---- epilogue ------------------------------------------------------------
    const float l_tot = pair_sum(st.l_run);
    const float inv = 1.f / l_tot;
    if (qrow < n) {
        bf16* orow = p.o + base_off + (size_t)qrow * row_stride;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = st.oacc[db][4 * a + i] * inv;
                const bf16x4 y = __builtin_convertvector(x, bf16x4);
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * a + 4 * h) = y;
            }
        if (p.lse && h == 0) {
            p.lse[((size_t)b * p.heads + head) * p.L + start + qrow] = st.m_run * p.scale + logf(l_tot);
        }
    }
}

template <int D, int NW>
int launch_attn(const AttnParams& prm, int32_t max_seqlen, hipStream_t stream) {
    constexpr int BM = 32 * NW;
    AttnParams p = prm;
    p.qtiles = (max_seqlen + BM - 1) / BM;
    if (p.qtiles == 0 || p.pairs == 0) return WIN_OK;
    const int64_t groups = ((int64_t)p.pairs + 7) / 8;
    const int64_t blocks = groups * 8 * p.qtiles;
    if (blocks >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    attn_fwd_kernel<D, NW><<<dim3((uint32_t)blocks), dim3(NW * 64), 0, stream>>>(p);
    return launch_status();
}

}  // namespace
}  // namespace winattn

using namespace winattn;

extern "C" int win_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int32_t num_windows, int32_t max_seqlen, int64_t L,
                            int32_t batch, int32_t heads, int32_t head_dim, float softmax_scale, void* stream) {
    if (!q || !k || !v || !o || !cu_seqlens) return WIN_EINVAL;
    if (num_windows < 0 || max_seqlen < 0 || L < 0 || batch <= 0 || heads <= 0) return WIN_EINVAL;
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return WIN_EINVAL;
    if (head_dim != 64 && head_dim != 128) return WIN_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return WIN_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return WIN_EUNSUPPORTED;
    if (L >= ((int64_t)1 << 31) || max_seqlen > L) return max_seqlen > L ? WIN_EINVAL : WIN_EOVERFLOW;
    const int64_t elems = (int64_t)batch * L * heads * head_dim;
    const uint64_t bytes = (uint64_t)elems * 2;
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
        return WIN_EINVAL;
    if (lse && overlaps(lse, (uint64_t)batch * heads * L * 4, o, bytes)) return WIN_EINVAL;
    const int64_t pairs = (int64_t)batch * num_windows * heads;
    if (pairs >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if (num_windows == 0 || L == 0 || max_seqlen == 0) return WIN_OK;

    AttnParams p;
    p.q = static_cast<const bf16*>(q);
    p.k = static_cast<const bf16*>(k);
    p.v = static_cast<const bf16*>(v);
    p.o = static_cast<bf16*>(o);
    p.lse = lse;
    p.cu = cu_seqlens;
    p.num_windows = num_windows;
    p.L = (int32_t)L;
    p.heads = heads;
    p.qtiles = 0;
    p.pairs = (int32_t)pairs;
    p.scale = softmax_scale;
    p.scale_log2 = softmax_scale * kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (head_dim == 128) return launch_attn<128, 4>(p, max_seqlen, s);
    return launch_attn<64, 4>(p, max_seqlen, s);
}
