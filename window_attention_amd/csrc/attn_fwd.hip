// win_attn_fwd: variable-length window attention, forward, for gfx950.
//
// Page "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Motivation"
// (attention only inside each 3D window) and "SeedVR2 integration" (one packed
// variable-length call over cu_seqlens segments).  For each (batch, window,
// head) the kernel computes softmax(Q K^T * scale) V with a flash-style online
// softmax over key tiles, so the n x n score matrix never leaves registers.
//
// Mapping to CDNA4
//   * One workgroup = NW waves = a tile of 32*QB*NW query rows of one
//     (batch, window, head).  Each wave owns QB blocks of 32 query rows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 accumulator layout a lane holds
//     16 keys of ONE query column (lane % 32), so the softmax row max and row
//     sum are in-lane reductions plus one exchange with lane ^ 32.
//   * The softmax runs in base 2: a probability is exp2(c * s - mc) with
//     c = scale * log2(e), s the fp32 score from the MFMAs (bf16 products
//     are exact, sums in fp32) and mc a per-row reference, one fma and one
//     exp2 per score.
//   * O^T = V^T P^T with the same instruction.  P^T is used straight from the
//     score registers as the B operand: the 8 keys a lane supplies for a
//     16-key step are the ones its accumulator already holds (keys
//     16j+4h+{0..3} and 16j+8+4h+{0..3}, h = lane / 32).  The V^T operand is
//     read with ds_read_b64_tr_b16, which returns four rows of one column per
//     lane, so V needs no transpose pass.  The O^T accumulator column is again
//     the lane's own query, so the online-softmax rescale is per lane.
//   * Every K or V fragment read from LDS feeds QB MFMAs (one per query
//     block), so LDS read traffic per flop falls as 1 / QB.  The library
//     launches QB = 1: two blocks per wave need a SIMD's whole register file,
//     one wave per SIMD, and that ran slower than two waves of one block.
//   * K and V tiles (64 keys) are copied HBM -> LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging), double buffered.  Rows are
//     stored with an XOR swizzle of their 16-byte chunks so that the K reads
//     (32 rows, same chunk) and the transposed V reads (4 rows x 4 columns per
//     16 lanes) are spread over the LDS banks.
//   * The key loop is software pipelined: while the MFMAs of tile j+1's
//     scores run, the VALU packs tile j's probabilities; while the MFMAs of
//     tile j's P V product run, the VALU does tile j+1's exp2 and row sums.
//     No row max is taken on the common path: a tile's probabilities are
//     bounded by its row sum, and only a sum above kSumLimit = 2^8 sends the
//     tile down the rare path that moves the reference.
//     The loop is laid out by hand in slots of one MFMA each, with the LDS
//     reads of an operand issued a few MFMAs before its use and scheduling
//     fences between slots, so that an MFMA never waits for a read issued
//     just before it.  Two workgroups share a CU (one wave of each per
//     SIMD); a wave in its value half takes issue priority over one in its
//     score half.
//   * Grid: blockIdx % 8 selects the XCD; all query tiles of one (batch,
//     window, head) go to the same XCD, consecutively, so they share its L2
//     while they stream the same K/V tiles.
//   * Query rows past the end of a window are clamped to its last row; key
//     and value rows past it fail the copies' buffer range check and are
//     masked to -inf as keys, so no access leaves the window's rows.
#include <cmath>
#include <mutex>

#include "common.h"

namespace winattn {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

// The reference of a row moves (and O is rescaled) only when some lane's
// probabilities of one tile sum to more than kSumLimit; as long as none does,
// every probability is at most kSumLimit.
constexpr float kSumLimit = 256.f;

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
    int32_t qtiles;    // query tiles per (batch, window, head) in the grid
    int32_t pairs;     // batch * num_windows * heads
    float scale;       // softmax scale
    float scale_log2;  // softmax scale * log2(e)
    // text rows appended to every window's segment (none when text_len == 0)
    const bf16* tq;    // [batch, text_len, heads, head_dim]
    const bf16* tk;
    const bf16* tv;
    float* tpart;      // per-window text outputs [batch, num_windows, text_len, heads, head_dim]
    int32_t text_len;
    int32_t qtiles_v;  // video query tiles per (batch, window, head); the text's follow
};

template <int D>
struct Layout {
    static constexpr int kCPR = D / 8;  // 16-byte chunks per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBN * kRowBytes;
    static constexpr int kSegs = kTileBytes / 1024;  // wave-wide 1 KiB copies per tile
    static constexpr int kRowsPerSeg = 1024 / kRowBytes;
    static constexpr int kVSwz = kCPR >= 16 ? 4 : 2;  // V chunk swizzle stride
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
    // chunk_xor relies on the row index wave * kPerWave * kRowsPerSeg +
    // i * kRowsPerSeg + lane / kCPR having its three parts in disjoint bits,
    // so that adding them is XOR-ing them: both strides powers of two.
    static_assert((Ly::kRowsPerSeg & (Ly::kRowsPerSeg - 1)) == 0, "rows per segment must be a power of two");
    static_assert(((kPerWave * Ly::kRowsPerSeg) & (kPerWave * Ly::kRowsPerSeg - 1)) == 0,
                  "rows per wave must be a power of two");
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
    // of the chunk index: for K (swizzle r % kCPR) the row's segment part
    // i * kRowsPerSeg shares no bit with the rest of the row index, so
    // chunk(i) = chunk(0) ^ (i * kRowsPerSeg % kCPR); for V (swizzle of
    // r % 4, the same for every segment) chunk(i) = chunk(0).
    __device__ static uint32_t src_off0(size_t row_stride, int wave, int lane) {
        return (uint32_t)(((size_t)seg_row(wave, lane, 0) * row_stride + seg_chunk(wave, lane, 0) * 8) * 2);
    }
    __device__ static constexpr uint32_t chunk_xor(int i) {
        return IS_V ? 0u : (uint32_t)(((i * Ly::kRowsPerSeg) & (Ly::kCPR - 1)) * 16);
    }
    // segment i of this wave: per-lane offsets fixed for the whole loop,
    // segment i a uniform kRowsPerSeg rows further
    __device__ static void segment(__amdgpu_buffer_rsrc_t src, uint32_t off, uint32_t seg_bytes,
                                   LDS_AS char* __restrict__ tile, int wave, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (LDS_AS void*)(tile + (wave * kPerWave + i) * 1024), 16,
                                                 off, i * seg_bytes, 0, 0);
    }
};

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

// One pending HBM -> LDS tile copy, issued segment by segment.  The source is
// a buffer resource based at the tile's first row and sized to the tile's rows
// inside the window: offsets stay 32-bit, and rows past the window end fail
// the range check, so no other window's data reaches the LDS (the rows keep
// what the buffer held before: this window's earlier keys, or zeros).  A tile
// past the last one gets an empty range and loads nothing.  Buffer (not
// global) LDS-DMA loads also keep the compiler's LDS wait counts exact while
// copies are in flight.
template <int D, int NW, bool IS_V>
struct TileJob {
    using TC = TileCopy<D, NW, IS_V>;
    __amdgpu_buffer_rsrc_t src;
    const uint32_t* offs;  // per-lane source offsets of the segments
    uint32_t seg_bytes;    // source bytes between consecutive segments of a lane
    LDS_AS char* tile;

    __device__ TileJob(const uint32_t* offs_, const bf16* base, size_t row_stride, int kv, int n, LDS_AS char* tile_)
        : offs(offs_), tile(tile_) {
        const uint32_t row_bytes = (uint32_t)row_stride * 2;
        // (a select and a min, not a clamp: the clamp becomes a vector med3)
        const int rows = kv >= n ? 0 : (n - kv < kBN ? n - kv : kBN);
        seg_bytes = TC::Ly::kRowsPerSeg * row_bytes;
        // every input is wave-uniform; saying so keeps the resource in SGPRs
        // (the compiler would otherwise wrap each load in a readfirstlane loop)
        const uint64_t a = reinterpret_cast<uint64_t>(base + (size_t)kv * row_stride);
        const uint64_t a_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
        src = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a_u), 0,
                                                __builtin_amdgcn_readfirstlane(rows * (int)row_bytes), kBufferWord3);
    }
    __device__ void issue(int wave, int i) const { TC::segment(src, offs[i], seg_bytes, tile, wave, i); }
    __device__ void issue_all(int wave) const {
#pragma unroll
        for (int i = 0; i < TC::kPerWave; ++i) issue(wave, i);
    }
};

// The keys of one (batch, window, head): the window's rows, then the text
// rows (page "Window-Aligned Sequence Parallelism (SeedVR2)", section
// "SeedVR2 integration": segments [video window, replicated text]).  Key
// tile t holds window rows kBN t .. for t < tw, else text rows
// kBN (t - tw) ..: every tile draws from one source, so the text starts on a
// tile boundary and the window's last tile is masked past its end.
struct KeyRange {
    const bf16* kw;
    const bf16* vw;
    int32_t nw;  // window rows
    const bf16* kt;
    const bf16* vt;
    int32_t nt;  // text rows
    int32_t tw;  // window tiles
    // TEXT false: no text rows (the plain call); the selection compiles away
    template <bool TEXT>
    __device__ int32_t tiles() const {
        return TEXT ? tw + (nt + kBN - 1) / kBN : tw;
    }
    // keys of tile t inside its source (kBN or more: no mask)
    template <bool TEXT>
    __device__ int32_t limit(int32_t t) const {
        return !TEXT || t < tw ? nw - t * kBN : nt - (t - tw) * kBN;
    }
};

template <int D, int NW, bool IS_V, bool TEXT>
__device__ __forceinline__ TileJob<D, NW, IS_V> tile_job(const KeyRange& kr, const uint32_t* off0, size_t row_stride,
                                                         int32_t t, LDS_AS char* __restrict__ buf) {
    if constexpr (!TEXT) return TileJob<D, NW, IS_V>(off0, IS_V ? kr.vw : kr.kw, row_stride, t * kBN, kr.nw, buf);
    const bool win = t < kr.tw;
    const bf16* base = IS_V ? (win ? kr.vw : kr.vt) : (win ? kr.kw : kr.kt);
    return TileJob<D, NW, IS_V>(off0, base, row_stride, win ? t * kBN : (t - kr.tw) * kBN, win ? kr.nw : kr.nt, buf);
}

// Running state of one wave: QB blocks of 32 query rows, online softmax in
// base 2.  With c = softmax_scale * log2(e), the probability of score s is
// exp2(c s - mc), mc a reference that no tile's probabilities exceed by much
// (see kSumLimit).
template <int D, int QB>
struct WaveState {
    static constexpr int KSTEPS = D / 16;
    static constexpr int DBLK = D / 32;
    bf16x8 qf[QB][KSTEPS];  // Q fragments, B operands of S^T = K Q^T
    f32x16 oacc[QB][DBLK];  // O^T accumulators: column = this lane's query
    float mc[QB];           // reference, in units of c * s (equal in lanes l and l ^ 32)
    float l_run[QB];        // sum of the fp32 probabilities this lane contributed
    float alpha[QB];        // O rescale factor owed since the reference last moved
    bool pending;           // wave-uniform: alpha must be applied before the next P V
    int koff[KSTEPS];       // LDS byte offsets of the K operand per k step
    int voff[DBLK];         // LDS byte offsets of the transposed V reads per O^T block
    // source offsets of this lane's K and V tile segments (the first
    // TileCopy::kPerWave entries are used)
    uint32_t kcopy[Layout<D>::kSegs];
    uint32_t vcopy[Layout<D>::kSegs];
};

// K fragment (A operand of S^T) number i of a key tile: fragments alternate
// between the two 32-key blocks (independent accumulator chains), so
// fragment i is block i % 2, k step i / 2.
template <int D, int QB>
__device__ __forceinline__ bf16x8 k_fragment(const WaveState<D, QB>& st, const LDS_AS char* __restrict__ kt, int i) {
    using Ly = Layout<D>;
    return *reinterpret_cast<const LDS_AS bf16x8*>(kt + (i & 1) * 32 * Ly::kRowBytes + st.koff[i >> 1]);
}

// Instruction slots.  The key loop is laid out by hand as a sequence of
// slots, each one MFMA (per query block), the LDS reads of the operand a
// few MFMAs later and a share of the independent VALU work, closed by a
// scheduling fence so that nothing migrates between slots.  Operands are thus
// in flight kKAhead (K) or kVAhead (V) MFMAs ahead of their use, and the
// waits before an MFMA are for its own operand only.
constexpr int kKAhead = 3;
constexpr int kVAhead = 2;
__device__ __forceinline__ void slot_fence() { __builtin_amdgcn_sched_barrier(0); }
// A value computed in a slot is pinned there: without a use at this point the
// compiler would sink the arithmetic to its first real use, a later slot or
// the next step, past the fences (they only order machine scheduling).
template <typename T>
__device__ __forceinline__ void pin(const T& x) {
    asm volatile("" ::"v"(x));
}

// Keys past the window end (the last tile only) get score -inf.
__device__ __forceinline__ void mask_tail(f32x16 (&s)[kBN / 32], int lim, int h) {
    if (lim < kBN) {
        // key of register r in block kb is kb*32 + 8*(r/4) + 4h + r%4:
        // compare the constant part against the limit less the lane part
        const int lim_h = lim - 4 * h;
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) < lim_h ? s[kb][r] : -INFINITY;
    }
}

// Row max of one query block's score tile (equal in lanes l and l ^ 32).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[kBN / 32]) {
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        mx0 = fmaxf(fmaxf(mx0, s[0][r]), s[0][r + 1]);
        mx1 = fmaxf(fmaxf(mx1, s[1][r]), s[1][r + 1]);
    }
    return pair_max(fmaxf(mx0, mx1));
}

// Move the reference of query block qb up by delta (0 in lanes whose
// reference stays) and rebase the running sum.  Returns the factor O must be
// multiplied by once every earlier P V product is in it.
template <int D, int QB>
__device__ __forceinline__ float move_reference(WaveState<D, QB>& st, int qb, float delta) {
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    st.mc[qb] += delta;
    st.l_run[qb] *= alpha;
    return alpha;
}

// Sum of one query block's probabilities of a tile, in this lane.
__device__ __forceinline__ float tile_sum(const f32x16 (&s)[kBN / 32]) {
    float a = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) a += s[kb][r];
    return a;
}
// exp2 of one query block's raw scores against its reference, in place.
__device__ __forceinline__ void tile_exp(f32x16 (&s)[kBN / 32], float c, float mc) {
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
}

// bf16 probabilities (B operands of the P V product, one per 16 keys), split
// into kBN / 4 pieces of one pair each: piece i converts keys 2i, 2i+1 of
// fragment i / 4.  (The row sums add the fp32 probabilities when they are
// computed: plain fp32 adds co-issue with the MFMAs, while the packed bf16 dot
// product that would add the rounded values shares their pipe.  The two sums
// differ by at most 2^-8 relative per term.)
struct PackedP {
    uint32_t w[kBN / 16][4];  // bf16 pairs of the B operand of 16-key step jj
};

template <int QB>
__device__ __forceinline__ void pack_piece(const f32x16 (&pf)[QB][kBN / 32], PackedP (&pp)[QB], int i) {
    const int jj = i >> 2, m = i & 3;
    const int kb = jj >> 1, r = 8 * (jj & 1) + 2 * m;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const f32x2 x = {pf[qb][kb][r], pf[qb][kb][r + 1]};
        const bf16x2 pr = __builtin_convertvector(x, bf16x2);
        pp[qb].w[jj][m] = __builtin_bit_cast(uint32_t, pr);
        pin(pp[qb].w[jj][m]);
    }
}

__device__ __forceinline__ bf16x8 p_operand(const PackedP& pp, int jj) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v w = {pp.w[jj][0], pp.w[jj][1], pp.w[jj][2], pp.w[jj][3]};
    return __builtin_bit_cast(bf16x8, w);
}

// V^T fragment (A operand of O^T block `voff`) for 16-key step jj.
template <int D>
__device__ __forceinline__ bf16x8 v_fragment(const LDS_AS char* __restrict__ vt, int voff, int jj) {
    using Ly = Layout<D>;
    const LDS_AS char* a0 = vt + voff + (16 * jj) * Ly::kRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * Ly::kRowBytes));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Deferred rescale of O by alpha (a move of the reference max, applied once
// every P V product computed against the old reference is in O).
template <int D, int QB>
__device__ __forceinline__ void apply_pending_rescale(WaveState<D, QB>& st) {
    if (st.pending) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < WaveState<D, QB>::DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[qb][db][r] *= st.alpha[qb];
        st.pending = false;
    }
}

// K fragment i of a key tile, kept in a per-step array indexed by fragment
// (the compiler allocates the few that are live at once).
template <int D, int QB>
__device__ __forceinline__ void read_k(const WaveState<D, QB>& st, const LDS_AS char* __restrict__ kt,
                                       bf16x8* kf, int i) {
    kf[i] = k_fragment(st, kt, i);
}

// Score slots of one key tile: S^T = K Q^T, s[qb][kb] holding keys kb*32 ..
// +31 against query block qb.  Fragments alternate between the two 32-key
// blocks (independent accumulator chains).  Slot i issues MFMA i and the read
// of K fragment i + kKAhead.  Inside a pipeline step (PACK) it also packs
// its share of the previous tile's probabilities and issues one segment of the
// step's tile copies, and past the last K fragment it reads the first V
// fragments of the P V product that follows.
template <int D, int NW, int QB, bool PACK>
__device__ __forceinline__ void score_slots(WaveState<D, QB>& st, const LDS_AS char* __restrict__ kt,
                                            const LDS_AS char* __restrict__ vt, f32x16 (&s)[QB][kBN / 32],
                                            bf16x8 (&vf)[WaveState<D, QB>::DBLK * (kBN / 16)],
                                            const f32x16 (&pf)[QB][kBN / 32], PackedP (&pp)[QB],
                                            const TileJob<D, NW, false>& kjob, const TileJob<D, NW, true>& vjob,
                                            int wave) {
    constexpr int KSEG = TileCopy<D, NW, false>::kPerWave;
    constexpr int VSEG = TileCopy<D, NW, true>::kPerWave;
    constexpr int DBLK = WaveState<D, QB>::DBLK;
    constexpr int NS = (kBN / 32) * WaveState<D, QB>::KSTEPS;
    static_assert(kBN / 32 == 2, "fragment order alternates two score blocks");
    constexpr int PPS = (kBN / 4) / NS;  // pack pieces per slot
    static_assert(PPS * NS == kBN / 4, "pack pieces must split evenly over the score slots");
    static_assert(KSEG + VSEG <= NS, "one tile-copy segment per score slot");
    bf16x8 kf[NS];
#pragma unroll
    for (int i = 0; i < kKAhead; ++i) read_k(st, kt, kf, i);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        s[qb][0] = f32x16{};
        s[qb][1] = f32x16{};
    }
    slot_fence();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            s[qb][i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], st.qf[qb][i >> 1], s[qb][i & 1], 0, 0, 0);
        const int nx = i + kKAhead;
        if (nx < NS)
            read_k(st, kt, kf, nx);
        else if (PACK && nx - NS < kVAhead)
            vf[nx - NS] = v_fragment<D>(vt, st.voff[(nx - NS) % DBLK], (nx - NS) / DBLK);
        if constexpr (PACK) {
#pragma unroll
            for (int pc = 0; pc < PPS; ++pc) pack_piece<QB>(pf, pp, i * PPS + pc);
            // tile copies for the next step, one segment per slot so that the
            // vector-memory queue never holds up the wave
            if (i < KSEG)
                kjob.issue(wave, i);
            else if (i < KSEG + VSEG)
                vjob.issue(wave, i - KSEG);
        }
        slot_fence();
    }
}

// Value slot i of one key tile: O^T block i % DBLK += V^T P^T over 16-key
// step i / DBLK, and the read of V fragment i + kVAhead.  vf[0 .. kVAhead-1]
// are in flight on entry.
template <int D, int QB>
__device__ __forceinline__ void value_slot(WaveState<D, QB>& st, const LDS_AS char* __restrict__ vt,
                                           const PackedP (&pp)[QB], bf16x8 (&vf)[WaveState<D, QB>::DBLK * (kBN / 16)],
                                           int i) {
    constexpr int DBLK = WaveState<D, QB>::DBLK;
    constexpr int NV = DBLK * (kBN / 16);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        st.oacc[qb][i % DBLK] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], p_operand(pp[qb], i / DBLK), st.oacc[qb][i % DBLK], 0, 0, 0);
    if (i + kVAhead < NV) vf[i + kVAhead] = v_fragment<D>(vt, st.voff[(i + kVAhead) % DBLK], (i + kVAhead) / DBLK);
}

// One pipelined step j (j + 1 < number of key tiles).  On entry pf holds the
// fp32 probabilities of tile j (against the current references); on exit
// those of tile j+1.  Two MFMA streams, each with independent VALU work in
// its slots:
//   scores:  S(j+1) = K(j+1) Q^T          || bf16 P(j)
//   values:  O += V(j)^T P(j)^T            || exp2 of S(j+1) and its row sums
// plus the copies of K(j+2) and V(j+1) into the buffers read in step j-1.
template <int D, int NW, int QB, bool TEXT>
__device__ __forceinline__ void pipeline_step(WaveState<D, QB>& st, f32x16 (&pf)[QB][kBN / 32],
                                              const LDS_AS char* __restrict__ k_next,
                                              const LDS_AS char* __restrict__ v_cur, LDS_AS char* __restrict__ k_fill,
                                              LDS_AS char* __restrict__ v_fill, const KeyRange& kr, size_t row_stride,
                                              int j, float c, int wave, int lane) {
    constexpr int DBLK = WaveState<D, QB>::DBLK;
    constexpr int NV = DBLK * (kBN / 16);
    const int h = lane >> 5;
    apply_pending_rescale(st);
    const TileJob<D, NW, false> kjob = tile_job<D, NW, false, TEXT>(kr, st.kcopy, row_stride, j + 2, k_fill);
    const TileJob<D, NW, true> vjob = tile_job<D, NW, true, TEXT>(kr, st.vcopy, row_stride, j + 1, v_fill);
    slot_fence();
    // scores stream
    PackedP pp[QB];
    f32x16 s[QB][kBN / 32];
    bf16x8 vf[NV];
    // The two waves of a SIMD run independent workgroups.  The one in its
    // value half (MFMAs plus all the exp2 and row-sum work) gets issue
    // priority over one in its score half (MFMAs plus light VALU), which
    // fills the gaps: about 2.5 % on a regular layer.
    __builtin_amdgcn_s_setprio(0);
    score_slots<D, NW, QB, true>(st, k_next, v_cur, s, vf, pf, pp, kjob, vjob, wave);
    __builtin_amdgcn_s_setprio(1);
    const int lim = kr.limit<TEXT>(j + 1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mask_tail(s[qb], lim, h);
    slot_fence();
    // values stream: exp2 of S(j+1) against the current reference, EPS2
    // scores per slot, and their row sums
    float rsn[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rsn[qb] = 0.f;
    constexpr int EPS2 = QB * (kBN / 2) / NV;
    static_assert(EPS2 * NV == QB * (kBN / 2), "exp2 work must split evenly over the value slots");
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        value_slot(st, v_cur, pp, vf, i);
#pragma unroll
        for (int e = i * EPS2; e < (i + 1) * EPS2; ++e) {
            const int qb = e / (kBN / 2), kb = (e / 16) % 2, r = e % 16;
            s[qb][kb][r] = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], c, -st.mc[qb]));
            rsn[qb] += s[qb][kb][r];
            pin(s[qb][kb][r]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pin(rsn[qb]);
        slot_fence();
    }
    // A lane's probabilities are at most its tile sum: as long as no sum
    // exceeds kSumLimit, no probability does.  Otherwise (rare) the tile's
    // scores are computed again from K(j+1), still in the LDS, and the
    // reference moves to their exact pair maximum.
    bool big = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) big |= rsn[qb] > kSumLimit;
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
        bf16x8 vf_unused[NV];
        PackedP pp_unused[QB];
        const TileJob<D, NW, false> kj_unused(st.kcopy, kr.kw, row_stride, 0, 0, k_fill);
        const TileJob<D, NW, true> vj_unused(st.vcopy, kr.vw, row_stride, 0, 0, v_fill);
        score_slots<D, NW, QB, false>(st, k_next, k_next, s, vf_unused, s, pp_unused, kj_unused, vj_unused, wave);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mask_tail(s[qb], lim, h);
            const float mxp = fmaf(tile_max(s[qb]), c, -st.mc[qb]);
            const float delta = mxp > 0.f ? mxp : 0.f;  // equal in both lanes of the pair
            st.alpha[qb] = move_reference(st, qb, delta);
            tile_exp(s[qb], c, st.mc[qb]);
            rsn[qb] = tile_sum(s[qb]);
        }
        st.pending = true;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st.l_run[qb] += rsn[qb];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb) pf[qb][kb] = s[qb][kb];
}

// Step j of a wave with no query row inside the window: only its share of
// the tile copies (the LDS tiles are shared by the workgroup).
template <int D, int NW, int QB, bool TEXT>
__device__ __forceinline__ void copy_step(const WaveState<D, QB>& st, LDS_AS char* __restrict__ k_fill,
                                          LDS_AS char* __restrict__ v_fill, const KeyRange& kr, size_t row_stride,
                                          int j, int wave) {
    tile_job<D, NW, false, TEXT>(kr, st.kcopy, row_stride, j + 2, k_fill).issue_all(wave);
    tile_job<D, NW, true, TEXT>(kr, st.vcopy, row_stride, j + 1, v_fill).issue_all(wave);
}

// P V product of the last tile, whose probabilities are in pf.
template <int D, int QB>
__device__ __forceinline__ void final_pv(WaveState<D, QB>& st, const f32x16 (&pf)[QB][kBN / 32],
                                         const LDS_AS char* __restrict__ v_cur) {
    constexpr int DBLK = WaveState<D, QB>::DBLK;
    constexpr int NV = DBLK * (kBN / 16);
    apply_pending_rescale(st);
    PackedP pp[QB];
    bf16x8 vf[NV];
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) vf[i] = v_fragment<D>(v_cur, st.voff[i % DBLK], i / DBLK);
#pragma unroll
    for (int i = 0; i < kBN / 4; ++i) pack_piece<QB>(pf, pp, i);
    slot_fence();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        value_slot(st, v_cur, pp, vf, i);
        slot_fence();
    }
}

// Waves per SIMD the register budget is sized for: one query block per wave
// fits two waves per SIMD, two blocks need the whole register file of one.
template <int QB>
constexpr int waves_per_simd() {
    return QB == 1 ? 2 : 1;
}

template <int D, int NW, int QB, bool TEXT>
__global__ __launch_bounds__(NW * 64, waves_per_simd<QB>()) void attn_fwd_kernel(AttnParams p) {
    using Ly = Layout<D>;
    using St = WaveState<D, QB>;
    constexpr int BM = 32 * QB * NW;
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
    const int qt_all = slot % p.qtiles;
    if (pair >= p.pairs) return;
    // video query tiles first, then the text's (rows of the text appended to
    // this window's segment)
    const bool text_rows = TEXT && qt_all >= p.qtiles_v;
    const int qt = text_rows ? qt_all - p.qtiles_v : qt_all;
    const int head = pair % p.heads;
    const int bw = pair / p.heads;
    const int win = bw % p.num_windows;
    const int b = bw / p.num_windows;
    int start = p.cu[win], end = p.cu[win + 1];
    start = start < 0 ? 0 : (start > p.L ? p.L : start);
    end = end < start ? start : (end > p.L ? p.L : end);
    const int n = end - start;
    const int nq = text_rows ? p.text_len : n;  // query rows of this work item
    const int q0 = qt * BM;
    if (q0 >= nq) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const size_t row_stride = (size_t)p.heads * D;
    const size_t base_off = ((size_t)b * p.L + start) * row_stride + (size_t)head * D;
    const size_t text_off = (size_t)b * p.text_len * row_stride + (size_t)head * D;
    KeyRange kr;
    kr.kw = p.k + base_off;
    kr.vw = p.v + base_off;
    kr.nw = n;
    kr.kt = p.text_len ? p.tk + text_off : kr.kw;
    kr.vt = p.text_len ? p.tv + text_off : kr.vw;
    kr.nt = p.text_len;
    kr.tw = (n + kBN - 1) / kBN;
    const bf16* qsrc = text_rows ? p.tq + text_off : p.q + base_off;
    const float c = p.scale_log2;

    St st;
    {
        const uint32_t k0off = TileCopy<D, NW, false>::src_off0(row_stride, wave, lane);
        const uint32_t v0off = TileCopy<D, NW, true>::src_off0(row_stride, wave, lane);
#pragma unroll
        for (int i = 0; i < TileCopy<D, NW, false>::kPerWave; ++i) {
            st.kcopy[i] = k0off ^ TileCopy<D, NW, false>::chunk_xor(i);
            asm volatile("" : "+v"(st.kcopy[i]));
        }
#pragma unroll
        for (int i = 0; i < TileCopy<D, NW, true>::kPerWave; ++i) st.vcopy[i] = v0off ^ TileCopy<D, NW, true>::chunk_xor(i);
    }
    const int nkv = kr.tiles<TEXT>();
    // V rows past the window end are never loaded: the V buffers start as
    // zeros (each wave clears the segments its own copies write, and waits for
    // that before they are issued)
    {
        constexpr int VSEG = TileCopy<D, NW, true>::kPerWave;
        typedef uint32_t u32x4z __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < VSEG; ++i) {
            *(LDS_AS u32x4z*)(v0 + (wave * VSEG + i) * 1024 + lane * 16) = u32x4z{0, 0, 0, 0};
            *(LDS_AS u32x4z*)(v1 + (wave * VSEG + i) * 1024 + lane * 16) = u32x4z{0, 0, 0, 0};
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    tile_job<D, NW, false, TEXT>(kr, st.kcopy, row_stride, 0, k0).issue_all(wave);
    tile_job<D, NW, true, TEXT>(kr, st.vcopy, row_stride, 0, v0).issue_all(wave);

    // query row of this lane in block qb: q0 + (wave * QB + qb) * 32 + lane % 32
    const int qrow0 = q0 + wave * 32 * QB + (lane & 31);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qr = qrow0 + qb * 32;
        const int qr_c = qr < nq ? qr : nq - 1;
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(qsrc + (size_t)qr_c * row_stride);
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) st.qf[qb][t] = qp[2 * t + h];
    }
    // K (A operand of S^T): lane reads row r = lane % 32 of a 32-key block,
    // logical chunk 2t + h, stored at chunk (2t + h) ^ (r % kCPR).  The t
    // part only flips chunk bits above bit 0, so the offset of step t is the
    // step-0 offset XOR 32 t.  (Kept opaque so that the compiler holds them
    // rather than recomputing them in the loop.)
    {
        const int r = lane & 31;
        const int koff0 = r * Ly::kRowBytes + Ly::k_chunk(r, h) * 16;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            st.koff[t] = koff0 ^ (32 * t);
            asm volatile("" : "+v"(st.koff[t]));
        }
    }
    // V (A operand of O^T, transposed read): address-supplying lane s of
    // 16-lane group g points at row 4*(g/2) + e, column 16*(g%2) + 4*c of a
    // 16-key x 32-column block (e = (s/4)%4, c = s%4); the transposed read
    // hands lane l the four rows 4*(l/32)+{0..3} of column l % 32.
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, cc = lane & 3;
        const int r = 4 * (g >> 1) + e;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int lc = db * 4 + 2 * (g & 1) + (cc >> 1);
            st.voff[db] = r * Ly::kRowBytes + Ly::v_chunk(r, lc) * 16 + (cc & 1) * 8;
        }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        st.mc[qb] = 0.f;
        st.l_run[qb] = 0.f;
        st.alpha[qb] = 1.f;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) st.oacc[qb][db] = f32x16{};
    }
    st.pending = false;

    // ---- prologue: tile 0 scores and probabilities ---------------------------
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of tile 0 have landed
    __syncthreads();                      // ... and every wave's
    tile_job<D, NW, false, TEXT>(kr, st.kcopy, row_stride, 1, k1).issue_all(wave);
    // A wave whose query rows all lie past the window end (the last query
    // tile of a window) computes nothing; it still copies its share of every
    // tile and meets every barrier.
    const bool active = q0 + wave * 32 * QB < nq;
    f32x16 pf[QB][kBN / 32];
    if (active) {
        bf16x8 vf_unused[DBLK * (kBN / 16)];
        PackedP pp_unused[QB];
        const TileJob<D, NW, false> kj_unused(st.kcopy, kr.kw, row_stride, 0, 0, k1);
        const TileJob<D, NW, true> vj_unused(st.vcopy, kr.vw, row_stride, 0, 0, v1);
        score_slots<D, NW, QB, false>(st, k0, k0, pf, vf_unused, pf, pp_unused, kj_unused, vj_unused, wave);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mask_tail(pf[qb], kr.limit<TEXT>(0), h);
            move_reference(st, qb, tile_max(pf[qb]) * c);  // first reference: the tile max (O is still zero)
            tile_exp(pf[qb], c, st.mc[qb]);
            st.l_run[qb] = tile_sum(pf[qb]);
        }
    }

    // ---- pipelined key loop, steps in pairs so that LDS buffers are static ----
    // step j reads K(j+1) from k[(j+1)%2] and V(j) from v[j%2]; it refills
    // k[j%2] with K(j+2) and v[(j+1)%2] with V(j+1).  The last tile's P V runs
    // after the loop.
    int j = 0;
    for (; j + 2 < nkv; j += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (active)
            pipeline_step<D, NW, QB, TEXT>(st, pf, k1, v0, k0, v1, kr, row_stride, j, c, wave, lane);
        else
            copy_step<D, NW, QB, TEXT>(st, k0, v1, kr, row_stride, j, wave);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (active)
            pipeline_step<D, NW, QB, TEXT>(st, pf, k0, v1, k1, v0, kr, row_stride, j + 1, c, wave, lane);
        else
            copy_step<D, NW, QB, TEXT>(st, k1, v0, kr, row_stride, j + 1, wave);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (j + 1 < nkv) {  // one more full step (tiles j, j+1), then the P V of tile j+1
        if (active)
            pipeline_step<D, NW, QB, TEXT>(st, pf, k1, v0, k0, v1, kr, row_stride, j, c, wave, lane);
        else
            copy_step<D, NW, QB, TEXT>(st, k0, v1, kr, row_stride, j, wave);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (active) final_pv(st, pf, v1);
    } else if (active) {  // the P V of tile j
        final_pv(st, pf, v0);
    }
    if (!active) return;

    // ---- epilogue ------------------------------------------------------------
    // O^T holds one query row per lane, so stores straight from the
    // accumulators would put 16 bytes into each of 32 rows per instruction.
    // The rows go through this wave's own 32-row region of the K buffers
    // instead (idle since the last step barrier), so that every store writes
    // whole rows: bf16 video rows in one pass, fp32 text rows in two passes of
    // half a row.  The region keeps the tiles' chunk swizzle.  One wave's LDS
    // accesses complete in order; the waits also keep the compiler from moving
    // reads above the writes they depend on, or writes above earlier reads.
    static_assert(NW * 32 * Ly::kRowBytes <= 2 * Ly::kTileBytes, "O staging must fit the K buffers");
    LDS_AS char* const stage = k0 + wave * 32 * Ly::kRowBytes;
    const int r0 = lane & 31;
    const int sw0 = r0 & (Ly::kCPR - 1);
    constexpr int kRowsPerStore = 1024 / Ly::kRowBytes;
    const int sc = lane % Ly::kCPR;  // chunk of a row this lane stores
    const int row0 = q0 + wave * 32 * QB;  // first query row of this wave
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qr = qrow0 + qb * 32;
        const float l_tot = pair_sum(st.l_run[qb]);
        const float inv = 1.f / l_tot;
        if (text_rows) {
            // this window's text output, normalized, kept in fp32 for the mean
            // over windows
            float* const tbase = p.tpart + ((size_t)b * p.num_windows + win) * p.text_len * row_stride + head * D;
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
#pragma unroll
                for (int db = hr * DBLK / 2; db < (hr + 1) * DBLK / 2; ++db)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        f32x4 x;
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] = st.oacc[qb][db][4 * a + i] * inv;
                        const int chunk = ((db - hr * DBLK / 2) * 8 + 2 * a + h) ^ sw0;
                        *(LDS_AS f32x4*)(stage + r0 * Ly::kRowBytes + chunk * 16) = x;
                    }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int t = 0; t < 32 / kRowsPerStore; ++t) {
                    const int r = t * kRowsPerStore + lane / Ly::kCPR;
                    const f32x4 y = *(const LDS_AS f32x4*)(stage + r * Ly::kRowBytes + (sc ^ (r & (Ly::kCPR - 1))) * 16);
                    const int row = row0 + qb * 32 + r;
                    if (row < nq) *reinterpret_cast<f32x4*>(tbase + (size_t)row * row_stride + hr * (D / 2) + sc * 4) = y;
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        } else {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = st.oacc[qb][db][4 * a + i] * inv;
                    *(LDS_AS bf16x4*)(stage + r0 * Ly::kRowBytes + ((db * 4 + a) ^ sw0) * 16 + h * 8) =
                        __builtin_convertvector(x, bf16x4);
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t = 0; t < 32 / kRowsPerStore; ++t) {
                const int r = t * kRowsPerStore + lane / Ly::kCPR;
                const bf16x8 y = *(const LDS_AS bf16x8*)(stage + r * Ly::kRowBytes + (sc ^ (r & (Ly::kCPR - 1))) * 16);
                const int row = row0 + qb * 32 + r;
                if (row < nq) *reinterpret_cast<bf16x8*>(p.o + base_off + (size_t)row * row_stride + sc * 8) = y;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (p.lse && h == 0 && qr < nq) {
                // sum_k exp(scale * s_k) = exp(scale * m_ref) * l_tot
                p.lse[((size_t)b * p.heads + head) * p.L + start + qr] = st.mc[qb] * 0.6931471805599453f + logf(l_tot);
            }
        }
    }
}

// Text stream of the window page (section "Text stream"): the text passed
// on is the sum of the per-window text outputs over the window count,
// summed in window order in fp32 and rounded once to bf16.  Thread i owns
// four consecutive elements of one batch's text rows.
__global__ __launch_bounds__(256) void text_mean_kernel(const float* __restrict__ part, bf16* __restrict__ out,
                                                        int32_t num_windows, int64_t per_batch, int64_t total) {
    const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e >= total) return;
    const int64_t b = e / per_batch, r = e - b * per_batch;
    const float* src = part + (size_t)b * num_windows * per_batch + r;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // unrolled so that several windows' loads are in flight; the adds keep
    // window order
#pragma unroll 8
    for (int32_t i = 0; i < num_windows; ++i) acc += *reinterpret_cast<const f32x4*>(src + (size_t)i * per_batch);
    const float w = (float)num_windows;
    const f32x4 m = {acc[0] / w, acc[1] / w, acc[2] / w, acc[3] / w};
    *reinterpret_cast<bf16x4*>(out + e) = __builtin_convertvector(m, bf16x4);
}

template <int D, int NW, int QB>
int launch_attn(const AttnParams& prm, int32_t max_seqlen, hipStream_t stream) {
    constexpr int BM = 32 * QB * NW;
    AttnParams p = prm;
    p.qtiles_v = (max_seqlen + BM - 1) / BM;
    p.qtiles = p.qtiles_v + (p.text_len + BM - 1) / BM;
    if (p.qtiles == 0 || p.pairs == 0) return WIN_OK;
    const int64_t groups = ((int64_t)p.pairs + 7) / 8;
    const int64_t blocks = groups * 8 * p.qtiles;
    if (blocks >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if (p.text_len > 0)
        attn_fwd_kernel<D, NW, QB, true><<<dim3((uint32_t)blocks), dim3(NW * 64), 0, stream>>>(p);
    else
        attn_fwd_kernel<D, NW, QB, false><<<dim3((uint32_t)blocks), dim3(NW * 64), 0, stream>>>(p);
    return launch_status();
}

// Launch configuration: (waves per workgroup, query blocks per wave).
#ifndef WINATTN_NW
#define WINATTN_NW 4
#endif
#ifndef WINATTN_QB
#define WINATTN_QB 1
#endif

}  // namespace
}  // namespace winattn

using namespace winattn;

namespace {

int attn_impl(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
              int32_t num_windows, int32_t max_seqlen, int64_t L, int32_t batch, int32_t heads, int32_t head_dim,
              float softmax_scale, const void* tq, const void* tk, const void* tv, int32_t text_len, void* text_o,
              float* text_partial, void* stream) {
    if (!q || !k || !v || !o || !cu_seqlens) return WIN_EINVAL;
    if (num_windows < 0 || max_seqlen < 0 || L < 0 || batch <= 0 || heads <= 0 || text_len < 0) return WIN_EINVAL;
    if (head_dim != 64 && head_dim != 128) return WIN_EUNSUPPORTED;
    // 0 selects the scaled-dot-product default 1/sqrt(head_dim)
    if (softmax_scale == 0.f) softmax_scale = (float)(1.0 / std::sqrt((double)head_dim));
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return WIN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return WIN_EUNSUPPORTED;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return WIN_EUNSUPPORTED;
    if (L >= ((int64_t)1 << 31) || max_seqlen > L) return max_seqlen > L ? WIN_EINVAL : WIN_EOVERFLOW;
    // a key tile's rows are addressed with 32-bit buffer offsets; with that,
    // batch * L < 2^38 keeps every byte count below 2^63
    if ((int64_t)kBN * heads * head_dim * 2 >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    if ((int64_t)batch * L >= ((int64_t)1 << 38)) return WIN_EOVERFLOW;
    const int64_t elems = (int64_t)batch * L * heads * head_dim;
    const uint64_t bytes = (uint64_t)elems * 2;
    if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
        return WIN_EINVAL;
    if (lse && overlaps(lse, (uint64_t)batch * heads * L * 4, o, bytes)) return WIN_EINVAL;
    const int64_t pairs = (int64_t)batch * num_windows * heads;
    if (pairs >= ((int64_t)1 << 31)) return WIN_EOVERFLOW;
    // batch * text_len < 2^38 and heads * head_dim < 2^24 keep t_elems below
    // 2^62; the per-window text outputs are bounded by 2^40 elements before
    // their count is formed
    if (text_len >= ((int64_t)1 << 31) / 64 || (int64_t)batch * text_len >= ((int64_t)1 << 38))
        return WIN_EOVERFLOW;
    const int64_t t_elems = (int64_t)batch * text_len * heads * head_dim;
    if (text_len > 0 && num_windows > (((int64_t)1 << 40) - 1) / t_elems) return WIN_EOVERFLOW;
    const int64_t p_elems = t_elems * num_windows;
    if (text_len > 0) {
        if (!tq || !tk || !tv || !text_o || !text_partial || num_windows == 0) return WIN_EINVAL;
        if (!aligned16(tq) || !aligned16(tk) || !aligned16(tv) || !aligned16(text_o) || !aligned16(text_partial))
            return WIN_EUNSUPPORTED;
        const uint64_t tb = (uint64_t)t_elems * 2, pb = (uint64_t)p_elems * 4;
        const void* ins[6] = {q, k, v, tq, tk, tv};
        for (const void* x : ins) {
            const uint64_t xb = (x == q || x == k || x == v) ? bytes : tb;
            if (overlaps(text_o, tb, x, xb) || overlaps(text_partial, pb, x, xb)) return WIN_EINVAL;
        }
        if (overlaps(text_o, tb, o, bytes) || overlaps(text_partial, pb, o, bytes) ||
            overlaps(text_partial, pb, text_o, tb) || (lse && overlaps(lse, (uint64_t)batch * heads * L * 4,
                                                                        text_partial, pb)))
            return WIN_EINVAL;
    }
    if (num_windows == 0 || (text_len == 0 && (L == 0 || max_seqlen == 0))) return WIN_OK;

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
    p.tq = static_cast<const bf16*>(tq);
    p.tk = static_cast<const bf16*>(tk);
    p.tv = static_cast<const bf16*>(tv);
    p.tpart = text_partial;
    p.text_len = text_len;
    p.qtiles_v = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int st = head_dim == 128 ? launch_attn<128, WINATTN_NW, WINATTN_QB>(p, max_seqlen, s)
                                   : launch_attn<64, WINATTN_NW, WINATTN_QB>(p, max_seqlen, s);
    if (st != WIN_OK || text_len == 0) return st;
    const int64_t per_batch = (int64_t)text_len * heads * head_dim;
    const int64_t threads = t_elems / 4;
    text_mean_kernel<<<dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, s>>>(
        text_partial, static_cast<bf16*>(text_o), num_windows, per_batch, t_elems);
    return launch_status();
}

}  // namespace

// Per-window text outputs of win_attn_fwd_text_noalloc: a static device array
// (each device holds its own copy from module load until the process ends).
// Host code never names it as an address: the device address comes from
// hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) float scratch[WIN_TEXT_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WIN_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return WIN_EDEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return WIN_OK;
}

}  // namespace

extern "C" int win_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int32_t num_windows, int32_t max_seqlen, int64_t L,
                            int32_t batch, int32_t heads, int32_t head_dim, float softmax_scale, void* stream) {
    return attn_impl(q, k, v, o, lse, cu_seqlens, num_windows, max_seqlen, L, batch, heads, head_dim, softmax_scale,
                     nullptr, nullptr, nullptr, 0, nullptr, nullptr, stream);
}

extern "C" int win_attn_fwd_text(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int32_t* cu_seqlens, int32_t num_windows, int32_t max_seqlen, int64_t L,
                                 int32_t batch, int32_t heads, int32_t head_dim, float softmax_scale,
                                 const void* text_q, const void* text_k, const void* text_v, int32_t text_len,
                                 void* text_o, float* text_partial, void* stream) {
    return attn_impl(q, k, v, o, lse, cu_seqlens, num_windows, max_seqlen, L, batch, heads, head_dim, softmax_scale,
                     text_q, text_k, text_v, text_len, text_o, text_partial, stream);
}

extern "C" int win_attn_fwd_text_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                         const int32_t* cu_seqlens, int32_t num_windows, int32_t max_seqlen,
                                         int64_t L, int32_t batch, int32_t heads, int32_t head_dim,
                                         float softmax_scale, const void* text_q, const void* text_k,
                                         const void* text_v, int32_t text_len, void* text_o, void* stream) {
    void* ws = nullptr;
    if (text_len > 0) {
        if (num_windows < 0 || batch <= 0 || heads <= 0 || head_dim <= 0) return WIN_EINVAL;
        // the per-window text outputs (batch * num_windows * text_len * heads
        // rows of head_dim floats) must fit the static array; checked factor
        // by factor, so no product leaves int64
        const int64_t limit = WIN_TEXT_SCRATCH_BYTES / 4 / head_dim;
        int64_t rows = 1;
        for (const int64_t f : {(int64_t)batch, (int64_t)num_windows, (int64_t)text_len, (int64_t)heads}) {
            rows *= f;
            if (rows > limit) return WIN_ESCRATCH;
        }
        const int st = scratch_address(&ws);
        if (st != WIN_OK) return st;
    }
    return attn_impl(q, k, v, o, lse, cu_seqlens, num_windows, max_seqlen, L, batch, heads, head_dim, softmax_scale,
                     text_q, text_k, text_v, text_len, text_o, static_cast<float*>(ws), stream);
}
