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
constexpr float kLn2 = 0.6931471805599453f;

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

// HBM -> LDS copy of one K or V tile (kBN rows of D bf16 starting at key
// kv0), each wave moving kSegs / NW wave-wide 1 KiB segments.  Row r of the
// tile lives at LDS byte r * kRowBytes with its 16-byte chunks permuted by the
// swizzle.  Segment i of this lane copies tile row seg_row(i) (lane / kCPR
// within the segment), logical chunk seg_chunk(i).
template <int D, int NW, bool IS_V>
struct TileCopy {
    using Ly = Layout<D>;
    static constexpr int kPerWave = Ly::kSegs / NW;
    static_assert(Ly::kSegs % NW == 0, "tile copy must split evenly over waves");
    // chunk_xor relies on: rows per segment a power of two (so the segment
    // part and the lane part of a row index occupy disjoint bits) and every
    // wave's first row a multiple of the chunk count.
    static_assert((Ly::kRowsPerSeg & (Ly::kRowsPerSeg - 1)) == 0, "rows per segment must be a power of two");
    static_assert((kPerWave * Ly::kRowsPerSeg) % Ly::kCPR == 0, "wave segments must start at a swizzle period");
    __device__ static int seg_row(int wave, int lane, int i) {
        return (wave * kPerWave + i) * Ly::kRowsPerSeg + lane / Ly::kCPR;
    }
    __device__ static int seg_chunk(int wave, int lane, int i) {
        const int row = seg_row(wave, lane, i), pc = lane % Ly::kCPR;
        return IS_V ? Ly::v_chunk(row, pc) : Ly::k_chunk(row, pc);  // xor swizzles are involutions
    }
    // Byte offset of this lane's source for segment i, relative to tile row
    // 0.  The segments of one lane are kRowsPerSeg rows apart (a uniform
    // offset); their logical chunks differ by an XOR that only touches bits
    // of the chunk index: for K (swizzle r % kCPR, rows 4i + g for D = 128)
    // chunk(i) = chunk(0) ^ (kRowsPerSeg * i % kCPR), for V (swizzle of
    // r % 4, the same for every segment) chunk(i) = chunk(0).
    __device__ static uint32_t src_off0(size_t row_stride, int wave, int lane) {
        return (uint32_t)(((size_t)seg_row(wave, lane, 0) * row_stride + seg_chunk(wave, lane, 0) * 8) * 2);
    }
    __device__ static constexpr uint32_t chunk_xor(int i) {
        return IS_V ? 0u : (uint32_t)(((i * Ly::kRowsPerSeg) & (Ly::kCPR - 1)) * 16);
    }
    // every row of the tile inside the window: uniform base + fixed offsets
    __device__ static void full(const char* __restrict__ base, uint32_t off0, size_t row_stride,
                                LDS_AS char* __restrict__ tile, int wave) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const char* b = base + (size_t)i * Ly::kRowsPerSeg * row_stride * 2;
            __builtin_amdgcn_global_load_lds((const void*)(b + (off0 ^ chunk_xor(i))),
                                             (LDS_AS void*)(tile + (wave * kPerWave + i) * 1024), 16, 0, 0);
        }
    }
    // last tile: rows past the window end re-read its last row
    __device__ static void clamped(const bf16* __restrict__ base, size_t row_stride, int kv0, int n,
                                   LDS_AS char* __restrict__ tile, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            int key = kv0 + seg_row(wave, lane, i);
            key = key < n ? key : n - 1;
            const bf16* g = base + (size_t)key * row_stride + seg_chunk(wave, lane, i) * 8;
            __builtin_amdgcn_global_load_lds((const void*)g, (LDS_AS void*)(tile + (wave * kPerWave + i) * 1024), 16,
                                             0, 0);
        }
    }
};

// Running state of one wave: 32 query rows, online softmax in base 2.
// Scores are kept relative to a reference max m_ref (in log2 units of the
// scaled scores); the score MFMA chain starts from the splat -m_ref, so the
// probabilities are plain exp2 of the accumulator.
template <int D, int NW>
struct WaveState {
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    bf16x8 qf[KSTEPS];  // Q * scale * log2(e), B operand of S^T = K Q^T
    f32x16 oacc[DBLK];  // O^T accumulator: column = this lane's query
    f32x16 neg_ref;     // splat(-m_ref)
    float m_ref;        // reference max (equal in lanes l and l ^ 32)
    float l_run;        // sum of the bf16 probabilities this lane contributed
    int koff0;          // LDS byte offset of the K operand at k step 0 (step t: ^ 32 t)
    int voff[DBLK];     // LDS byte offsets of the transposed V reads per O^T block
    uint32_t kcopy;     // source offset of this lane's first K tile segment
    uint32_t vcopy;     // source offset of this lane's first V tile segment
};

// Rescaling is deferred until a tile's max exceeds the reference max by this
// many powers of two, so probabilities stay below 2^kRescaleLog2.
constexpr float kRescaleLog2 = 8.f;

// One key tile: issue the copies of the next tile, then S^T, softmax and O^T
// update from the current tile.  The buffers are restrict-qualified so that
// the compiler knows the copies into *_next never alias the reads of *_cur.
template <int D, int NW>
__device__ __forceinline__ void attend_tile(WaveState<D, NW>& st, const LDS_AS char* __restrict__ kcur,
                                            const LDS_AS char* __restrict__ vcur, LDS_AS char* __restrict__ knext,
                                            LDS_AS char* __restrict__ vnext, const bf16* kbase, const bf16* vbase,
                                            size_t row_stride, int kv, int n, bool first, int wave, int lane) {
    using Ly = Layout<D>;
    constexpr int KSTEPS = WaveState<D, NW>::KSTEPS;
    constexpr int DBLK = WaveState<D, NW>::DBLK;
    const int h = lane >> 5;
    const int kv_next = kv + kBN;
    // Keep the per-lane bases opaque to loop-invariant code motion: the
    // offsets derived from them by XOR / add with constants are cheaper to
    // recompute each tile than to hold in registers across the loop.
    asm volatile("" : "+v"(st.koff0), "+v"(st.kcopy), "+v"(st.vcopy));
    if (kv_next + kBN <= n) {
        const size_t adv = (size_t)kv_next * row_stride * 2;
        TileCopy<D, NW, false>::full(reinterpret_cast<const char*>(kbase) + adv, st.kcopy, row_stride, knext, wave);
        TileCopy<D, NW, true>::full(reinterpret_cast<const char*>(vbase) + adv, st.vcopy, row_stride, vnext, wave);
    } else if (kv_next < n) {
        TileCopy<D, NW, false>::clamped(kbase, row_stride, kv_next, n, knext, wave, lane);
        TileCopy<D, NW, true>::clamped(vbase, row_stride, kv_next, n, vnext, wave, lane);
    }
    // S'^T block kb = K Q'^T - m_ref: rows = keys kb*32 .. +31, columns = queries
    f32x16 s[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = st.neg_ref;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const bf16x8 kf =
                *reinterpret_cast<const LDS_AS bf16x8*>(kcur + kb * 32 * Ly::kRowBytes + (st.koff0 ^ (32 * t)));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.qf[t], s[kb], 0, 0, 0);
        }
    }
    const int lim = n - kv;
    if (lim < kBN) {  // keys past the window end (last tile only)
        // key of register r in block kb is kb*32 + 8*(r/4) + 4h + r%4:
        // compare the constant part against the limit less the lane part
        const int lim_h = lim - 4 * h;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) < lim_h ? s[kb][r] : -INFINITY;
    }
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        mx0 = fmaxf(fmaxf(mx0, s[0][r]), s[0][r + 1]);
        mx1 = fmaxf(fmaxf(mx1, s[1][r]), s[1][r + 1]);
    }
    const float mx = pair_max(fmaxf(mx0, mx1));
    const bool grow = first || mx > kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float delta = grow ? mx : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        st.m_ref += delta;
        st.l_run *= alpha;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) st.neg_ref[r] = -st.m_ref;
    }
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
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(s[kb][r0 + i]);
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
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(AttnParams p) {
    using Ly = Layout<D>;
    using St = WaveState<D, NW>;
    constexpr int BM = 32 * NW;
    constexpr int KSTEPS = St::KSTEPS;
    constexpr int DBLK = St::DBLK;
    __shared__ __attribute__((aligned(1024))) char smem[4 * Ly::kTileBytes];
    LDS_AS char* lds = (LDS_AS char*)smem;
    LDS_AS char* const k0 = lds;
    LDS_AS char* const k1 = lds + Ly::kTileBytes;
    LDS_AS char* const v0 = lds + 2 * Ly::kTileBytes;
    LDS_AS char* const v1 = lds + 3 * Ly::kTileBytes;

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

    St st;
    st.kcopy = TileCopy<D, NW, false>::src_off0(row_stride, wave, lane);
    st.vcopy = TileCopy<D, NW, true>::src_off0(row_stride, wave, lane);
    const int nkv = (n + kBN - 1) / kBN;
    if (kBN <= n) {
        TileCopy<D, NW, false>::full(reinterpret_cast<const char*>(kbase), st.kcopy, row_stride, k0, wave);
        TileCopy<D, NW, true>::full(reinterpret_cast<const char*>(vbase), st.vcopy, row_stride, v0, wave);
    } else {
        TileCopy<D, NW, false>::clamped(kbase, row_stride, 0, n, k0, wave, lane);
        TileCopy<D, NW, true>::clamped(vbase, row_stride, 0, n, v0, wave, lane);
    }

    const int qrow = q0 + wave * 32 + (lane & 31);
    {
        const int qrow_c = qrow < n ? qrow : n - 1;
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(p.q + base_off + (size_t)qrow_c * row_stride);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const bf16x8 x = qp[2 * t + h];
            f32x8 y;
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = (float)x[i] * p.scale_log2;
            st.qf[t] = __builtin_convertvector(y, bf16x8);
        }
    }
    // K (A operand of S^T): lane reads row r = lane % 32 of a 32-key block,
    // logical chunk 2t + h, stored at chunk (2t + h) ^ (r % kCPR).  The t
    // part only flips chunk bits above bit 0, so the offset of step t is the
    // step-0 offset XOR 32 t.
    {
        const int r = lane & 31;
        st.koff0 = r * Ly::kRowBytes + Ly::k_chunk(r, h) * 16;
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
    st.m_ref = 0.f;
    st.l_run = 0.f;
    st.neg_ref = f32x16{};
#pragma unroll
    for (int db = 0; db < DBLK; ++db) st.oacc[db] = f32x16{};

    // key tiles in pairs, so that the LDS buffers of each are compile-time
    int j = 0;
    for (; j + 1 < nkv; j += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile j have landed
        __syncthreads();                      // ... and every wave's; the other buffers are free
        attend_tile<D, NW>(st, k0, v0, k1, v1, kbase, vbase, row_stride, j * kBN, n, j == 0, wave, lane);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        attend_tile<D, NW>(st, k1, v1, k0, v0, kbase, vbase, row_stride, (j + 1) * kBN, n, false, wave, lane);
    }
    if (j < nkv) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        attend_tile<D, NW>(st, k0, v0, k1, v1, kbase, vbase, row_stride, j * kBN, n, j == 0, wave, lane);
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
            // sum_k exp(scale * s_k) = 2^m_ref * l_tot
            p.lse[((size_t)b * p.heads + head) * p.L + start + qrow] = st.m_ref * kLn2 + logf(l_tot);
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
