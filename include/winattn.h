/*
 * winattn.h -- C ABI of the MI355X (gfx950) 3D window-attention library.
 *
 * The operations follow the page "Window-Aligned Sequence Parallelism
 * (SeedVR2)" (vLLM-Omni design notes):
 *   - win_plan        section "Window layouts": 720p-normalised window sizes,
 *                     regular and half-window-shifted clipped windows,
 *                     w-outermost / t-innermost enumeration, row-major tokens
 *                     inside a window, canonical id (t*H + h)*W + w, ragged
 *                     windows described by cu_seqlens.
 *   - win_permute     section "SeedVR2 integration": entry distribution of
 *                     canonical rows into window order and final
 *                     reconstruction back to canonical order.
 *   - win_transition  sections "Motivation" and "Plan A redistribution": the
 *                     layout change between consecutive layers, a local
 *                     permutation of rows on one device, done in one pass.
 *   - win_attn_fwd    sections "Motivation" and "SeedVR2 integration":
 *                     attention only inside each window, one packed
 *                     variable-length call over cu_seqlens segments.
 *   - win_attn_fwd_text  sections "SeedVR2 integration" and "Text stream":
 *                     [video window, replicated text] segments and the text
 *                     output averaged over windows.
 *   - win_plan_local, section "Reference quirks reproduced on purpose":
 *     win_rope_table, window-local 3D rotary position embedding of queries
 *     win_permute_rope and keys, fused into the gather / transition.
 *   - win_lpt,        sections "Planner" and "Plan A redistribution": the
 *     win_plan_a      single-GPU tables of window-aligned sequence
 *                     parallelism (window assignment, exchange tables).
 * and the page "vLLM-Omni diffusion runtime" (blog post):
 *   - win_pack        section 4.2: several requests' plans packed into one
 *                     varlen call with alignment tails.
 *
 * Conventions shared by every entry point
 *   - Every function returns WIN_OK (0) or a negative status; win_strerror()
 *     names it.  Arguments are validated on the host before anything is
 *     launched; on a non-zero status nothing has been enqueued.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no pointer after a call returns.
 *   - "device" pointers are HIP device allocations of the current device;
 *     "host" pointers are ordinary process memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *     enqueued on it asynchronously; no function synchronises the device.
 *     Device work is kernel launches only (no allocation, no memset, no
 *     copy), so every call may be recorded into a stream-captured HIP graph
 *     and replayed with new data in the same buffers.
 *   - Token tensors are contiguous [B, L, row] with a 16-byte aligned base;
 *     the same plan applies to every batch element.  Attention tensors are
 *     [B, L, heads, head_dim] bf16.
 *   - Sources and destinations must not overlap (WIN_EINVAL if src == dst).
 */
#ifndef WINATTN_H
#define WINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define WIN_OK            0
#define WIN_EINVAL       (-1) /* bad argument, geometry, null/aliased pointer */
#define WIN_EUNSUPPORTED (-2) /* dtype, head_dim, row size or alignment not handled */
#define WIN_EOVERFLOW    (-3) /* a size or index exceeds the 32-bit index range */
#define WIN_EDEVICE      (-4) /* the HIP runtime reported an error */
#define WIN_ESCRATCH     (-5) /* the work needs more than the library's static scratch */

/* ---- enumerations -------------------------------------------------------- */
#define WIN_METHOD_REGULAR 0 /* slice(k*w, min((k+1)*w, n)) on every axis */
#define WIN_METHOD_SHIFTED 1 /* every cut moved by half a window, clipped to [0, n] */

#define WIN_DTYPE_BF16 0 /* 2-byte elements */
#define WIN_DTYPE_FP16 1 /* 2-byte elements */
#define WIN_DTYPE_FP32 2 /* 4-byte elements */

#define WIN_GATHER  0 /* dst[b, j] = src[b, idx[j]]   canonical -> window order */
#define WIN_SCATTER 1 /* dst[b, idx[j]] = src[b, j]   window -> canonical order */

/* ---- win_plan ------------------------------------------------------------ */
typedef struct win_plan_info {
    int32_t wt, wh, ww;             /* window extent on t, h, w */
    int32_t segs_t, segs_h, segs_w; /* number of window segments on each axis */
    int32_t num_windows;            /* N = segs_t * segs_h * segs_w */
    int32_t max_seqlen;             /* tokens in the largest window */
    int64_t num_tokens;             /* L = T * H * W */
} win_plan_info;

/*
 * Window layout of a post-patch (T, H, W) token grid (page section "Window
 * layouts").
 *
 * Sizes: scale = sqrt(45*80 / (H*W)) in IEEE double, wh = ceil(round(H*scale)
 * / nh), ww = ceil(round(W*scale) / nw), wt = ceil(min(T, 30) / nt), with
 * round-half-to-even on the double product.
 * Axis segments (extent n, window w): regular [k*w, min((k+1)*w, n));
 * shifted: if w >= n the single segment [0, n), otherwise the cuts are 0,
 * floor(w/2), floor(w/2) + w, ... clipped to n, empty segments dropped.
 * Windows are the products of axis segments, enumerated w outermost, then h,
 * then t; tokens inside a window are row-major in (t, h, w).
 *
 * Arguments
 *   T, H, W, nt, nh, nw  > 0; T*H*W must be < 2^31.
 *   method               WIN_METHOD_REGULAR or WIN_METHOD_SHIFTED.
 *   info                 host, required: receives sizes and counts.
 *   perm                 [L] int32: perm[j] = canonical id at window position j.
 *   inv                  [L] int32: inv[perm[j]] = j.
 *   cu_seqlens           [N+1] int32 prefix sums of window sizes (cu[0] = 0).
 *   boxes                [N*6] int32: (t0, t1, h0, h1, w0, w1) per window.
 *   Any of perm / inv / cu_seqlens / boxes may be NULL (not written), so a
 *   first call with all four NULL is a size query.
 *   on_device            0: the four tables are host memory, filled on the
 *                        host before return.  1: they are device memory,
 *                        filled by a kernel enqueued on `stream`.
 * Errors: WIN_EINVAL (non-positive input, rescaled extent of zero, bad
 * method, info NULL), WIN_EOVERFLOW (L >= 2^31), WIN_EDEVICE.
 */
int win_plan(int32_t T, int32_t H, int32_t W, int32_t nt, int32_t nh, int32_t nw, int32_t method,
             win_plan_info* info, int32_t* perm, int32_t* inv, int32_t* cu_seqlens, int32_t* boxes,
             int32_t on_device, void* stream);

/*
 * Entry gather / exit scatter of whole token rows (page section "SeedVR2
 * integration": entry distribution and final reconstruction).
 *   mode WIN_GATHER:  dst[b, j, :] = src[b, idx[j], :]
 *   mode WIN_SCATTER: dst[b, idx[j], :] = src[b, j, :]
 *   src, dst   device, [batch, L, row_elems] of `dtype`, 16-byte aligned, no overlap.
 *   idx        device, [L] int32, a permutation of 0..L-1 (win_plan's perm).
 *              Entries outside [0, L) are clamped into range, so no access
 *              leaves the tensors; the rows they touch are then unspecified.
 *   row_elems * element size must be a multiple of 16 bytes.  With L == 0
 *   nothing is read or written and the pointers may be NULL.
 * Bit-exact copy.  Errors: WIN_EINVAL, WIN_EUNSUPPORTED (dtype, row size,
 * alignment), WIN_EOVERFLOW (L or batch * L >= 2^31, row_elems >= 2^33, or
 * batch * L rows of more than 2^62 bytes), WIN_EDEVICE.
 */
int win_permute(const void* src, void* dst, const int32_t* idx, int64_t L, int32_t batch, int64_t row_elems,
                int32_t dtype, int32_t mode, void* stream);

/*
 * Layout transition A -> B in one pass (page sections "Motivation" and "Plan A
 * redistribution": on one device a local permutation of rows):
 *   dst[b, j, :] = src[b, inv_src[perm_dst[j]], :]
 * inv_src is layout A's inv and perm_dst is layout B's perm (device, [L]
 * int32 each, clamped into range as in win_permute).  Other arguments and
 * errors as in win_permute.
 */
int win_transition(const void* src, void* dst, const int32_t* inv_src, const int32_t* perm_dst, int64_t L,
                   int32_t batch, int64_t row_elems, int32_t dtype, void* stream);

/*
 * Variable-length window attention, forward (page sections "Motivation" and
 * "SeedVR2 integration"): for every batch element b, window i (rows
 * cu_seqlens[i] .. cu_seqlens[i+1]-1) and head h,
 *   O = softmax(Q K^T * softmax_scale) V      (no mask inside a window)
 *   lse = rowmax + log(rowsum)                 (natural log, per query row)
 * q, k, v, o   device, bf16 [batch, L, heads, head_dim], window-ordered,
 *              16-byte aligned; o must not overlap q, k or v.
 * lse          device fp32 [batch, heads, L] or NULL (not written).
 * cu_seqlens   device int32 [num_windows + 1], non-decreasing, cu[0] >= 0,
 *              cu[num_windows] <= L; zero-length windows are allowed; every
 *              window must hold at most max_seqlen rows.  Entries that break
 *              these rules are clamped so that no access leaves the tensors;
 *              the rows involved are then unspecified.  Rows outside every
 *              window are not written.
 * head_dim     64 or 128.
 * softmax_scale > 0, or 0 for the default 1/sqrt(head_dim) (the scaled
 *              dot-product convention; computed in double, rounded to float);
 *              negative, NaN or infinite values are WIN_EINVAL.
 * Arithmetic: bf16 inputs, fp32 MFMA accumulation and fp32 online softmax,
 * bf16 output rounded to nearest even.  Deterministic: no atomics, a fixed
 * reduction order per output row, independent of batch size and grid.
 * Errors: WIN_EINVAL, WIN_EUNSUPPORTED (head_dim, alignment), WIN_EOVERFLOW
 * (L >= 2^31, batch * L >= 2^38, batch * num_windows * heads >= 2^31, or
 * heads * head_dim >= 2^24, so that 64 rows span 2^31 bytes or more),
 * WIN_EDEVICE.
 */
int win_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                 int32_t num_windows, int32_t max_seqlen, int64_t L, int32_t batch, int32_t heads,
                 int32_t head_dim, float softmax_scale, void* stream);

/*
 * Window-local coordinates of a layout's rows (window page, section
 * "Reference quirks reproduced on purpose": rotary positions are window-local
 * and restart at 0 in every window).  Row j of the window order (canonical
 * token perm[j] of win_plan) gets local[3j], local[3j+1], local[3j+2] = its
 * t, h, w minus the first t, h, w of its window.  Geometry arguments and
 * errors as in win_plan; local is [3 L] int32, host memory filled before
 * return (on_device 0) or device memory filled by a kernel on `stream` (1).
 */
int win_plan_local(int32_t T, int32_t H, int32_t W, int32_t nt, int32_t nh, int32_t nw, int32_t method,
                   int32_t* local, int32_t on_device, void* stream);

/*
 * (cos, sin) table of window-local 3D rotary position embedding (same
 * section): the rotated span is 3 * (rope_dim / 3) channels, three blocks of
 * d = rope_dim / 3 for the t, h and w axial indices; pair (2i, 2i+1) of a
 * block turns by position * base^(-2i/d) (the rotation of Su et al.,
 * RoFormer).  Rows of the table: t positions text_len .. text_len + wt - 1,
 * then h positions 0 .. wh - 1, then w positions 0 .. ww - 1 (wt, wh, ww are a
 * plan's window extents, win_plan_info); each row holds d / 2 pairs of floats
 * (cos, sin), computed in double and rounded to float.
 *   table: host, (wt + wh + ww) * (rope_dim / 3) floats.
 * Errors: WIN_EINVAL (non-positive extents, negative text_len, base <= 1 or
 * not finite, rope_dim < 6, table NULL), WIN_EUNSUPPORTED (rope_dim / 3 odd).
 */
int win_rope_table(int32_t wt, int32_t wh, int32_t ww, int32_t text_len, int32_t rope_dim, double base,
                   float* table);

/*
 * Gather or transition of query / key rows into a window layout with the
 * layout's window-local rotary embedding applied on the way (same section;
 * one read and one write of every row, as win_permute):
 *   gather     (perm_dst NULL):  row j = rope(src[b, idx[j]], local[j])
 *   transition (perm_dst given): row j = rope(src[b, idx[perm_dst[j]]], local[j])
 * where idx is the gather table of the destination layout (gather) or the
 * source layout's inv (transition, idx = inv_src), and local is the
 * destination layout's win_plan_local table.  src rows are not rotated: each
 * layout rotates the same un-rotated rows with its own positions.
 *   src, dst  device bf16 [batch, L, heads, head_dim], 16-byte aligned, no overlap.
 *   idx, perm_dst, local  device int32 ([L], [L], [3 L]); entries are clamped
 *             into range as in win_permute.
 *   table     device floats in win_rope_table's layout for (wt, wh, ww),
 *             8-byte aligned; local entries are clamped to those extents.
 *   head_dim  64 or 128; rope_dim <= head_dim with rope_dim / 3 even.
 * Channels past 3 * (rope_dim / 3) keep their bits.  Rotated pairs are
 * computed in fp32 and rounded to bf16 (nearest even).
 * Errors: WIN_EINVAL, WIN_EUNSUPPORTED (head_dim, rope_dim, alignment),
 * WIN_EOVERFLOW, WIN_EDEVICE.
 */
int win_permute_rope(const void* src, void* dst, const int32_t* idx, const int32_t* perm_dst, const int32_t* local,
                     const float* table, int32_t wt, int32_t wh, int32_t ww, int64_t L, int32_t batch,
                     int32_t heads, int32_t head_dim, int32_t rope_dim, void* stream);

/*
 * Packing of several requests' plans into one varlen call (page "vLLM-Omni
 * diffusion runtime", section 4.2 on packing).  Request r (r = 0..R-1, in
 * order) occupies rows [offsets[r], offsets[r] + L_r) of the packed token
 * tensor, followed by an alignment tail of (align - L_r % align) % align rows;
 * offsets[r+1] = offsets[r] + L_r + tail.
 *   cu_out:   the request's window boundaries moved by offsets[r], then the
 *             end of its tail, for every request in order after a leading 0:
 *             sum(N_r) + R segments; a zero-length tail repeats a boundary.
 *   perm_out: perm_out[offsets[r] + j] = offsets[r] + perm_r[j]; tail rows map
 *             to themselves.  Use it with win_permute on the packed tensor;
 *             positional coordinates stay request-local.
 *   max_seqlen: the longest segment (windows and tails).
 * Arguments (all host memory)
 *   num_requests R > 0; num_tokens[R] (L_r > 0); num_windows[R] (N_r > 0);
 *   perms       the R perm tables back to back (sum L_r int32), NULL only if
 *               perm_out is NULL;
 *   cu_seqlens  the R cu_seqlens tables back to back (sum (N_r + 1) int32);
 *   align > 0;
 *   offsets     out, R + 1 int64;  perm_out out (total rows int32) or NULL;
 *   cu_out      out, sum(N_r) + R + 1 int32;  max_seqlen out, required.
 * Errors: WIN_EINVAL (a table that is not a plan: cu not starting at 0, not
 * ending at L_r or decreasing, a perm entry outside [0, L_r); null or
 * non-positive arguments), WIN_EOVERFLOW (L_r or the packed rows >= 2^31).
 * Nothing is written unless the call succeeds.
 */
int win_pack(int32_t num_requests, const int64_t* num_tokens, const int32_t* num_windows, const int32_t* perms,
             const int32_t* cu_seqlens, int32_t align, int64_t* offsets, int32_t* perm_out, int32_t* cu_out,
             int32_t* max_seqlen);

/*
 * Deterministic LPT assignment of windows to `ranks` ranks (window page,
 * section "Planner"): windows are taken by decreasing token count, ties by
 * window id; each goes to the rank with the fewest assigned tokens, ties to
 * the lower rank; each rank then lists its windows in ascending id.  This is
 * what each rank of window-aligned sequence parallelism would own; with
 * ranks = 1 every window is on rank 0.
 * Arguments (host): num_windows N >= 0; cu_seqlens [N+1] (window sizes are
 *   its differences); ranks > 0; owner [N] out (rank of each window);
 *   order [N] out (windows grouped by rank, rank 0 first, ascending ids);
 *   rank_offsets [ranks+1] out (rank r's windows are order[rank_offsets[r] ..
 *   rank_offsets[r+1]-1]); rank_tokens [ranks] out (int64 tokens per rank).
 * Errors: WIN_EINVAL (null pointer, cu not starting at 0 or decreasing).
 */
int win_lpt(int32_t num_windows, const int32_t* cu_seqlens, int32_t ranks, int32_t* owner, int32_t* order,
            int32_t* rank_offsets, int64_t* rank_tokens);

/*
 * Plan A redistribution tables between a source and a destination layout,
 * each with its window assignment (window page, section "Plan A
 * redistribution").  Rank r holds, in its local order, the tokens of its
 * windows in listed order (win_lpt's `order`), row-major inside each window
 * (the plan's window order).
 *   counts [ranks*ranks] int64 out, row-major: counts[r*ranks + d] = rows rank
 *     d needs from rank r.  Rank r's input split sizes are row r, its output
 *     split sizes column r.
 *   send_rows [L] out: for each source rank r in turn (its block starts at its
 *     first row in rank order), its local rows to send, grouped by destination
 *     rank and, inside a group, in destination-local order.
 *   recv_pos [L] out: for each destination rank d in turn, the
 *     destination-local position of each row it receives, rows concatenated in
 *     source-rank order; the receiver reorders with one argsort of these.
 *   exchange_required out: 1 if some row changes rank (computed from the whole
 *     count matrix, so every rank takes the same branch), else 0.
 * With ranks = 1 this is the local transition: send_rows = inv_src[perm_dst].
 * Arguments (host): L tokens (both layouts); the source plan's perm [L] and
 *   cu_seqlens [src_windows+1] with its assignment (order, rank_offsets as
 *   win_lpt returns them); the same for the destination.
 * Errors: WIN_EINVAL (inconsistent tables: a perm that is not a permutation,
 *   an assignment that is not a partition, bad cu), WIN_EOVERFLOW (L >= 2^31).
 */
int win_plan_a(int64_t L, int32_t ranks, const int32_t* src_perm, const int32_t* src_cu, int32_t src_windows,
               const int32_t* src_order, const int32_t* src_rank_offsets, const int32_t* dst_perm,
               const int32_t* dst_cu, int32_t dst_windows, const int32_t* dst_order,
               const int32_t* dst_rank_offsets, int64_t* counts, int32_t* send_rows, int32_t* recv_pos,
               int32_t* exchange_required);

/*
 * Text-augmented window attention (window page, sections "SeedVR2
 * integration" and "Text stream"): every window's segment is its video rows
 * followed by the text rows, replicated for each window.
 *   video row of window i: softmax over [window i's keys, text keys] (scale
 *     softmax_scale), written to o (and lse) as in win_attn_fwd;
 *   text rows: once per window, softmax over the same segment; the normalized
 *     per-window outputs go to text_partial (fp32), and text_o receives their
 *     sum over the num_windows segments divided by num_windows (fp32 sum in
 *     window order, rounded once to bf16).
 * Arguments as in win_attn_fwd, plus
 *   text_q, text_k, text_v  device bf16 [batch, text_len, heads, head_dim],
 *                           16-byte aligned (shared by every window);
 *   text_len >= 0           (0: exactly win_attn_fwd; the text pointers are
 *                           then not used);
 *   text_o                  device bf16 [batch, text_len, heads, head_dim] out;
 *   text_partial            device fp32 workspace
 *                           [batch, num_windows, text_len, heads, head_dim],
 *                           16-byte aligned, owned by the caller, overwritten.
 * Every segment counts as a window in the division, zero-length ones too
 * (their text output attends to the text alone).  text_o and text_partial
 * must not overlap any input or output.
 * Errors: as win_attn_fwd; WIN_EINVAL also for text_len > 0 with a null text
 * pointer or num_windows == 0; WIN_EOVERFLOW also for text_len >= 2^25,
 * batch * text_len >= 2^38, or per-window text outputs of 2^40 elements or
 * more.
 */
int win_attn_fwd_text(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                      int32_t num_windows, int32_t max_seqlen, int64_t L, int32_t batch, int32_t heads,
                      int32_t head_dim, float softmax_scale, const void* text_q, const void* text_k,
                      const void* text_v, int32_t text_len, void* text_o, float* text_partial, void* stream);

/*
 * win_attn_fwd_text without the caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator): the per-window text
 * outputs go to a static device array of WIN_TEXT_SCRATCH_BYTES bytes that
 * the library holds on each device it runs on until the process ends.  The
 * caller passes inputs and outputs as for win_attn_fwd_text; nothing is
 * allocated or freed by the call.
 *   batch * num_windows * text_len * heads * head_dim * 4 bytes must fit the
 *   array: WIN_ESCRATCH otherwise (nothing enqueued).  With 24 heads x 128
 *   that is, e.g., 256 text rows on 21 windows or 85 rows on 64 windows.
 * Every call on one device uses that device's one array: calls that overlap
 * on one device (two streams, or two host threads) race and their outputs
 * are unspecified; calls ordered on one stream do not.  Each call writes
 * every slot it reads, so no clearing is needed between calls.
 * Results are bit-identical to win_attn_fwd_text.  Errors: as
 * win_attn_fwd_text, plus WIN_ESCRATCH.
 */
#define WIN_TEXT_SCRATCH_BYTES ((int64_t)64 << 20)
int win_attn_fwd_text_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* cu_seqlens, int32_t num_windows, int32_t max_seqlen, int64_t L,
                              int32_t batch, int32_t heads, int32_t head_dim, float softmax_scale,
                              const void* text_q, const void* text_k, const void* text_v, int32_t text_len,
                              void* text_o, void* stream);

/* Static string naming a status code. */
const char* win_strerror(int status);

/* Static string naming the build: target arch, kernel variants and tiles. */
const char* win_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* WINATTN_H */
