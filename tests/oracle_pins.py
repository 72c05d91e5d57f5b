"""Checks that pin the oracle to facts fixed by the page
"Window-Aligned Sequence Parallelism (SeedVR2)", section "Window layouts"
(size formulas, regular and shifted methods, exact partition, clipping instead
of wrapping, enumeration order, canonical id) and by mathematics (masked
softmax attention, closed forms).  Each check raises AssertionError on
failure; the oracle tests call them on real inputs and the mutation tests call
them on a deliberately broken oracle to show they catch the mistake.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- planner pins

def check_worked_examples(oracle_plan):
    """Hand-derived worked examples (tests/golden/plan_worked_examples.json)."""
    g = load_golden("plan_worked_examples.json")
    for ex in g["examples"]:
        T, H, W = ex["grid"]
        nt, nh, nw = ex["num_windows_param"]
        assert list(oracle_plan.window_size(T, H, W, nt, nh, nw)) == ex["window_size"], ex["name"]
        for mname, method in (("regular", oracle_plan.REGULAR), ("shifted", oracle_plan.SHIFTED)):
            want = ex[mname]
            p = oracle_plan.plan(T, H, W, nt, nh, nw, method)
            if "perm" in want:
                assert p.perm == want["perm"], (ex["name"], mname)
            if want.get("perm_is_identity"):
                assert p.perm == list(range(T * H * W)), (ex["name"], mname)
            if "cu_seqlens" in want:
                assert p.cu_seqlens == want["cu_seqlens"], (ex["name"], mname)
            if "boxes" in want:
                assert [list(b) for b in p.boxes] == want["boxes"], (ex["name"], mname)
            if "num_windows" in want:
                assert p.num_windows == want["num_windows"], (ex["name"], mname)
            if "first_window_tokens" in want:
                assert p.cu_seqlens[1] == want["first_window_tokens"], (ex["name"], mname)
            if "last_window_tokens" in want:
                assert p.cu_seqlens[-1] - p.cu_seqlens[-2] == want["last_window_tokens"], (ex["name"], mname)
            if "max_seqlen" in want:
                assert p.max_seqlen == want["max_seqlen"], (ex["name"], mname)
            if "axis_segments" in want:
                segs = want["axis_segments"]
                assert [list(s) for s in oracle_plan.axis_segments(T, p.wt, method)] == segs["t"]
                assert [list(s) for s in oracle_plan.axis_segments(H, p.wh, method)] == segs["h"]
                assert [list(s) for s in oracle_plan.axis_segments(W, p.ww, method)] == segs["w"]


def check_size_invariance(oracle_plan):
    """Section "Motivation": the window size is normalised to the 720p area, so
    a higher resolution grows the number of windows, never their size."""
    grids = [(21, 45, 80), (21, 68, 120), (21, 90, 160)]
    sizes = [oracle_plan.window_size(T, H, W, 4, 3, 3) for T, H, W in grids]
    assert sizes[0] == sizes[1] == sizes[2] == (6, 15, 27), sizes
    for method in (oracle_plan.REGULAR, oracle_plan.SHIFTED):
        counts = [oracle_plan.plan(T, H, W, 4, 3, 3, method).num_windows for T, H, W in grids]
        assert counts[0] < counts[1] < counts[2], counts


def check_temporal_cap(oracle_plan):
    """Size formula block: the temporal window is ceil(min(T, 30) / nt)."""
    for nt in (1, 2, 3, 4, 7):
        assert oracle_plan.window_size(30, 45, 80, nt, 3, 3)[0] == math.ceil(30 / nt)
        assert oracle_plan.window_size(31, 45, 80, nt, 3, 3)[0] == math.ceil(30 / nt)
        assert oracle_plan.window_size(200, 45, 80, nt, 3, 3)[0] == math.ceil(30 / nt)
        assert oracle_plan.window_size(5, 45, 80, nt, 3, 3)[0] == math.ceil(5 / nt)


def check_exact_scales(oracle_plan):
    """Grids whose area is the reference area over a perfect square have an
    exact scale, so the rescaled extents are known integers; the two tie grids
    check Python's round-half-to-even (22.5 -> 22, 7.5 -> 8)."""
    assert oracle_plan.window_size(1, 45, 80, 1, 1, 1) == (1, 45, 80)        # scale 1
    assert oracle_plan.window_size(1, 9, 16, 1, 1, 1) == (1, 45, 80)         # scale 5
    assert oracle_plan.window_size(1, 90, 160, 1, 1, 1) == (1, 45, 80)       # scale 1/2
    assert oracle_plan.window_size(1, 9, 64, 1, 1, 1) == (1, 22, 160)        # scale 5/2, 22.5 -> 22
    assert oracle_plan.window_size(1, 3, 192, 1, 1, 1) == (1, 8, 480)        # scale 5/2, 7.5 -> 8
    assert oracle_plan.window_size(1, 45, 80, 1, 3, 3) == (1, 15, 27)
    assert oracle_plan.window_size(7, 45, 80, 2, 4, 7) == (4, 12, 12)


def _label_regular(x, w):
    return x // w


def _label_shifted(x, n, w):
    """Segment index of coordinate x under the half-window shift, written as a
    per-coordinate closed form: with offset o = floor(w/2) the cuts are
    o, o+w, o+2w, ...; a zero-width first segment (o == 0) is not counted."""
    if w >= n:
        return 0
    o = w // 2
    idx = (x - o) // w + 1 if x >= o else 0
    return idx - 1 if o == 0 else idx


def check_plan_invariants(oracle_plan, p, T, H, W, nt, nh, nw, method):
    """Exact partition, box membership, enumeration order, row-major tokens,
    canonical ids (windowing np.arange), per-coordinate labelling twin."""
    L = T * H * W
    perm = np.asarray(p.perm, dtype=np.int64)
    assert perm.shape == (L,)
    assert np.array_equal(np.sort(perm), np.arange(L)), "not a partition"
    inv = np.asarray(p.inv, dtype=np.int64)
    assert np.array_equal(inv[perm], np.arange(L))
    cu = np.asarray(p.cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == L and len(cu) == p.num_windows + 1
    vols = [(b[1] - b[0]) * (b[3] - b[2]) * (b[5] - b[4]) for b in p.boxes]
    assert all(v > 0 for v in vols)
    assert np.array_equal(np.diff(cu), vols)
    # windowing np.arange: the window-order ids are the row-major flattening of
    # each box of the canonical id grid, boxes in enumeration order
    grid = np.arange(L).reshape(T, H, W)
    twin = np.concatenate([grid[t0:t1, h0:h1, w0:w1].ravel() for (t0, t1, h0, h1, w0, w1) in p.boxes])
    assert np.array_equal(twin, perm), "perm differs from windowing arange"
    # enumeration order: w outermost, h, t innermost
    keys = [(b[4], b[2], b[0]) for b in p.boxes]
    assert keys == sorted(keys) and len(set(keys)) == len(keys), "enumeration order"
    # per-coordinate labelling twin: window of each token from closed-form labels
    wt, wh, ww = p.wt, p.wh, p.ww
    if method == oracle_plan.REGULAR:
        lt = [_label_regular(x, wt) for x in range(T)]
        lh = [_label_regular(x, wh) for x in range(H)]
        lw = [_label_regular(x, ww) for x in range(W)]
    else:
        lt = [_label_shifted(x, T, wt) for x in range(T)]
        lh = [_label_shifted(x, H, wh) for x in range(H)]
        lw = [_label_shifted(x, W, ww) for x in range(W)]
    nT, nH = max(lt) + 1, max(lh) + 1
    assert p.num_windows == nT * nH * (max(lw) + 1)
    win_of_pos = np.repeat(np.arange(p.num_windows), np.diff(cu))
    for c in range(L):
        t, rem = divmod(c, H * W)
        h, w = divmod(rem, W)
        want = (lw[w] * nH + lh[h]) * nT + lt[t]
        assert win_of_pos[inv[c]] == want, ("label twin", c)
    # clipped, not rolled: no window on a split axis holds both ends of it
    for (t0, t1, h0, h1, w0, w1) in p.boxes:
        for lo, hi, n, nseg in ((t0, t1, T, nT), (h0, h1, H, nH), (w0, w1, W, max(lw) + 1)):
            assert 0 <= lo < hi <= n
            if nseg > 1:
                assert not (lo == 0 and hi == n)


def check_shift_geometry(oracle_plan, n, w):
    """Regular segments are full windows except a short last one; shifted
    segments start with a half window (floor(w/2)), continue with full windows
    and end clipped at n; a covering window is not shifted."""
    reg = oracle_plan.regular_segments(n, w)
    assert reg[0][0] == 0 and reg[-1][1] == n
    assert all(b - a == w for a, b in reg[:-1]) and 0 < reg[-1][1] - reg[-1][0] <= w
    sh = oracle_plan.shifted_segments(n, w)
    assert sh[0][0] == 0 and sh[-1][1] == n
    assert all(sh[i][1] == sh[i + 1][0] for i in range(len(sh) - 1))
    if w >= n:
        assert sh == [(0, n)]
    elif w == 1:
        assert sh == reg
    else:
        assert sh[0] == (0, w // 2)
        assert all(b - a == w for a, b in sh[1:-1])
        assert 0 < sh[-1][1] - sh[-1][0] <= w
        assert sh != reg


# ----------------------------------------------------------------- packing pins

def check_pack_worked_example(pack_fn):
    """The page's teaching layout (tests/golden/pack_worked_example.json):
    ``pack_fn(perms, cus, align)`` returns (offsets, perm, cu_seqlens,
    max_seqlen)."""
    g = load_golden("pack_worked_example.json")
    perms = [list(range(r["rows"])) for r in g["requests"]]
    cus = [r["cu_seqlens"] for r in g["requests"]]
    offsets, perm, cu, mx = pack_fn(perms, cus, g["align"])
    assert list(cu) == g["expected"]["cu_seqlens"]
    assert mx == g["expected"]["max_seqlen"]
    assert list(offsets) == g["expected"]["offsets"]
    assert list(perm) == list(range(128))


def check_pack_invariants(pack_fn, perms, cus, align):
    """What the page fixes for any packing: requests back to back with
    alignment tails; each request's windows and tail as separate segments
    (the tail's boundary present even when it is empty); the physical index
    shifted by the request's offset; max_seqlen the longest segment."""
    offsets, perm, cu, mx = pack_fn(perms, cus, align)
    offsets, perm, cu = list(offsets), list(perm), list(cu)
    R = len(perms)
    assert len(offsets) == R + 1 and offsets[0] == 0
    total = offsets[-1]
    assert len(perm) == total and sorted(perm) == list(range(total))
    assert len(cu) == 1 + sum(len(c) - 1 for c in cus) + R
    assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
    seg = 1
    longest = 0
    for r, (p, c) in enumerate(zip(perms, cus)):
        o, n = offsets[r], len(p)
        pad = offsets[r + 1] - o - n
        assert o % align == 0 and 0 <= pad < align
        # rows: the request's own gather table, moved by its offset
        assert perm[o:o + n] == [o + x for x in p]
        # tail: padding rows stay in place
        assert perm[o + n:o + n + pad] == list(range(o + n, o + n + pad))
        # segments: the request's windows, then its tail
        for a, b in zip(c[:-1], c[1:]):
            assert cu[seg] - cu[seg - 1] == b - a
            assert cu[seg] == o + b
            longest = max(longest, b - a)
            seg += 1
        assert cu[seg] == o + n + pad and cu[seg] - cu[seg - 1] == pad
        longest = max(longest, pad)
        seg += 1
    assert seg == len(cu)
    assert mx == longest


# ------------------------------------------------------- sequence-parallel pins

def check_lpt_worked_examples(lpt_fn):
    """Hand-derived LPT assignments (tests/golden/sp_plan_worked_example.json):
    ``lpt_fn(sizes, ranks)`` returns (owner, lists, loads)."""
    g = load_golden("sp_plan_worked_example.json")
    for e in g["lpt"]:
        owner, lists, loads = lpt_fn(e["sizes"], e["ranks"])
        assert list(owner) == e["owner"] and [list(x) for x in lists] == e["lists"] and list(loads) == e["loads"]


def check_lpt_invariants(lpt_fn, sizes, ranks):
    """A partition of the windows, each rank's list ascending, loads summing
    the sizes, and the bound every greedy list schedule meets: no rank holds
    more than the mean load plus the largest window."""
    owner, lists, loads = lpt_fn(sizes, ranks)
    assert sorted(w for ws in lists for w in ws) == list(range(len(sizes)))
    for r, ws in enumerate(lists):
        assert list(ws) == sorted(ws) and all(owner[w] == r for w in ws)
        assert loads[r] == sum(sizes[w] for w in ws)
    if sizes:
        assert max(loads) <= sum(sizes) / ranks + max(sizes)


def check_plan_a_worked_example(plan_a_fn):
    """The hand-derived two-rank exchange on the 3x4 grid, regular to shifted:
    ``plan_a_fn(z_src, z_dst)`` returns (counts, send_rows, recv_pos,
    exchange_required)."""
    e = load_golden("sp_plan_worked_example.json")["plan_a"]
    counts, send, recv, ex = plan_a_fn(e["z_src"], e["z_dst"])
    assert [list(x) for x in counts] == e["counts"]
    assert [list(x) for x in send] == e["send_rows"] and [list(x) for x in recv] == e["recv_pos"]
    assert bool(ex) == e["exchange_required"]


def check_plan_a_invariants(plan_a_fn, z_src, z_dst):
    """The exchange the tables drive (simulated with lists for the ranks'
    buffers) turns every source holding into the destination holding; split
    sizes are the row and column of the count matrix; each peer segment
    arrives in destination-local order; the exchange flag is global."""
    counts, send, recv, ex = plan_a_fn(z_src, z_dst)
    P = len(z_src)
    assert [sum(counts[r]) for r in range(P)] == [len(z) for z in z_src]
    assert [sum(counts[r][d] for r in range(P)) for d in range(P)] == [len(z) for z in z_dst]
    for d in range(P):
        k = 0
        for r in range(P):
            seg = list(recv[d][k:k + counts[r][d]])
            assert seg == sorted(seg)          # destination-local order within each peer segment
            k += counts[r][d]
        assert sorted(recv[d]) == list(range(len(z_dst[d])))
    # simulated all-to-all: rank r's rows are its canonical ids
    outbox = []
    for r in range(P):
        rows = [z_src[r][i] for i in send[r]]
        segs, k = [], 0
        for d in range(P):
            segs.append(rows[k:k + counts[r][d]])
            k += counts[r][d]
        outbox.append(segs)
    for d in range(P):
        got = [row for r in range(P) for row in outbox[r][d]]
        placed = [None] * len(got)
        for t, pos in enumerate(recv[d]):
            placed[pos] = got[t]
        assert placed == list(z_dst[d])
    assert bool(ex) == any(counts[r][d] for r in range(P) for d in range(P) if r != d)


# ---------------------------------------------------------------------- RoPE pins

def check_rope_worked_example(rotate_fn):
    """Hand-derived rotations of unit vectors (tests/golden/rope_worked_example.json):
    ``rotate_fn(x, pos, rope_dim)`` rotates the last axis of fp64 ``x``."""
    r = load_golden("rope_worked_example.json")["rotation"]
    for cse in r["cases"]:
        x = np.zeros(r["head_dim"])
        x[cse["unit"]] = 1.0
        y = rotate_fn(x, r["position"], r["rope_dim"])
        for k, v in cse["expect"].items():
            assert abs(y[int(k)] - v) < 1e-12, (cse["unit"], k, y[int(k)], v)
        assert abs(np.linalg.norm(y) - 1.0) < 1e-12


def check_rope_positions(positions_fn, oracle_plan):
    """Hand-derived window-local positions on the 3x4 grid, both layouts:
    ``positions_fn(plan, text_len)`` returns one (pt, ph, pw) per row."""
    g = load_golden("rope_worked_example.json")["positions"]
    for m, key in ((oracle_plan.REGULAR, "regular"), (oracle_plan.SHIFTED, "shifted")):
        p = oracle_plan.plan(*g["grid"], *g["window_counts"], m)
        assert [list(x) for x in positions_fn(p, g["text_len"])] == g[key]


def check_rope_properties(rotate_fn, rope_dim, head_dim, seed=0):
    """What makes it a rotary position embedding (Su et al.): a rotation
    (pair norms kept, channels past the span untouched), rotations compose
    (rotating by p then by r equals rotating by p + r), and the dot product of
    a rotated query and key depends only on their position difference."""
    rng = np.random.default_rng(seed)
    span = 3 * (rope_dim // 3)
    for _ in range(4):
        q, k = rng.standard_normal(head_dim), rng.standard_normal(head_dim)
        p1, p2, sh = rng.integers(0, 40, 3), rng.integers(0, 40, 3), rng.integers(0, 40, 3)
        y = rotate_fn(q, p1, rope_dim)
        assert np.allclose(y[span:], q[span:], rtol=0, atol=0)
        pairs = lambda v: np.hypot(v[0:span:2], v[1:span:2])
        assert np.allclose(pairs(y), pairs(q), rtol=1e-13, atol=1e-13)
        assert np.allclose(rotate_fn(y, p2, rope_dim), rotate_fn(q, p1 + p2, rope_dim), rtol=1e-11, atol=1e-11)
        d0 = rotate_fn(q, p1, rope_dim) @ rotate_fn(k, p2, rope_dim)
        d1 = rotate_fn(q, p1 + sh, rope_dim) @ rotate_fn(k, p2 + sh, rope_dim)
        assert abs(d0 - d1) < 1e-10 * (1 + abs(d0))


def check_rope_window_restart(positions_fn, oracle_plan, text_len=3):
    """Every window restarts at 0: each window's first row (its box corner)
    sits at (text_len, 0, 0), and no axial index reaches the window extent."""
    for grid in [(5, 9, 16, 2, 6, 6), (21, 45, 80, 4, 3, 3)]:
        for m in (oracle_plan.REGULAR, oracle_plan.SHIFTED):
            p = oracle_plan.plan(*grid, m)
            pos = positions_fn(p, text_len)
            for i, (t0, t1, h0, h1, w0, w1) in enumerate(p.boxes):
                a, e = p.cu_seqlens[i], p.cu_seqlens[i + 1]
                assert tuple(pos[a]) == (text_len, 0, 0)
                for x in pos[a:e]:
                    assert text_len <= x[0] < text_len + t1 - t0 and 0 <= x[1] < h1 - h0 and 0 <= x[2] < w1 - w0


# ------------------------------------------------------------ text attention pins

def check_text_closed_form(fn, seed=0):
    """Uniform attention, from the page's two rules alone: with zero queries
    every row of a segment attends uniformly, so a video row of window w gets
    the mean of its segment's values, (n_w a_w + T b) / (n_w + T) when the
    window's values are the constant a_w and the text values the constant b;
    the text output is that same per-window mean averaged with equal weight per
    window (not per token).  ``fn(q, k, v, cu, tq, tk, tv)`` returns (video,
    text)."""
    rng = np.random.default_rng(seed)
    cu = [0, 1, 6, 6, 9]                      # windows of 1, 5, 0 and 3 tokens
    B, Hh, D, T = 2, 3, 8, 4
    L = cu[-1]
    q = np.zeros((B, L, Hh, D))
    k = rng.standard_normal((B, L, Hh, D))
    tq = np.zeros((B, T, Hh, D))
    tk = rng.standard_normal((B, T, Hh, D))
    a = rng.standard_normal((B, len(cu) - 1, Hh))
    bval = rng.standard_normal((B, Hh))
    v = np.zeros((B, L, Hh, D))
    for i in range(len(cu) - 1):
        v[:, cu[i]:cu[i + 1]] = a[:, i][:, None, :, None]
    tv = np.broadcast_to(bval[:, None, :, None], (B, T, Hh, D)).copy()
    o, text = fn(q, k, v, cu, tq, tk, tv)[:2]
    seg_mean = [(n * a[:, i] + T * bval) / (n + T) for i, n in enumerate(np.diff(cu))]
    for i in range(len(cu) - 1):
        for t in range(cu[i], cu[i + 1]):
            assert np.allclose(o[:, t], seg_mean[i][:, :, None], rtol=0, atol=1e-12)
    want_text = sum(seg_mean) / (len(cu) - 1)
    assert np.allclose(text, np.broadcast_to(want_text[:, None, :, None], text.shape), rtol=0, atol=1e-12)


def check_text_brute_force(fn, seed=1):
    """Library routine: torch's scaled_dot_product_attention in float64 over
    one sequence in which every window is followed by its own copy of the
    text, with a same-segment mask; the text output is the mean over windows
    of the copies' outputs."""
    import torch
    F = torch.nn.functional
    rng = np.random.default_rng(seed)
    cu = [0, 3, 7, 12]
    B, Hh, D, T = 1, 2, 16, 5
    L, N = cu[-1], len(cu) - 1
    q, k, v = (rng.standard_normal((B, L, Hh, D)) for _ in range(3))
    tq, tk, tv = (rng.standard_normal((B, T, Hh, D)) for _ in range(3))
    seq = {x: [] for x in "qkv"}
    seg = []
    for i in range(N):
        a, e = cu[i], cu[i + 1]
        for name, src, txt in (("q", q, tq), ("k", k, tk), ("v", v, tv)):
            seq[name].append(np.concatenate([src[:, a:e], txt], axis=1))
        seg += [i] * (e - a + T)
    Q, K, V = (torch.as_tensor(np.concatenate(seq[x], axis=1)).permute(0, 2, 1, 3).contiguous() for x in "qkv")
    seg = torch.as_tensor(seg)
    mask = seg[:, None] == seg[None, :]
    out = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=1 / math.sqrt(D)).permute(0, 2, 1, 3).numpy()
    o, text = fn(q, k, v, cu, tq, tk, tv)[:2]
    pos, texts = 0, []
    for i in range(N):
        n = cu[i + 1] - cu[i]
        assert np.allclose(o[:, cu[i]:cu[i + 1]], out[:, pos:pos + n], rtol=0, atol=1e-12)
        texts.append(out[:, pos + n:pos + n + T])
        pos += n + T
    assert np.allclose(text, sum(texts) / N, rtol=0, atol=1e-12)


def check_text_isolation(fn, seed=2):
    """Changing one window's video rows leaves every other window's video
    outputs unchanged, and moves the text output by exactly 1/N of that
    window's text-output change."""
    rng = np.random.default_rng(seed)
    cu = [0, 4, 9, 11]
    B, Hh, D, T = 1, 2, 8, 3
    L, N = cu[-1], len(cu) - 1
    q, k, v = (rng.standard_normal((B, L, Hh, D)) for _ in range(3))
    tq, tk, tv = (rng.standard_normal((B, T, Hh, D)) for _ in range(3))
    o1, t1, per1 = fn(q, k, v, cu, tq, tk, tv)
    q2, k2, v2 = (x.copy() for x in (q, k, v))
    for x in (q2, k2, v2):
        x[:, 4:9] = rng.standard_normal((B, 5, Hh, D))
    o2, t2, per2 = fn(q2, k2, v2, cu, tq, tk, tv)
    assert np.array_equal(o1[:, :4], o2[:, :4]) and np.array_equal(o1[:, 9:], o2[:, 9:])
    assert np.array_equal(per1[:, 0], per2[:, 0]) and np.array_equal(per1[:, 2], per2[:, 2])
    assert np.allclose(t2 - t1, (per2[:, 1] - per1[:, 1]) / N, rtol=0, atol=1e-12)


# --------------------------------------------------------------- attention pins

def torch_sdpa_masked(qc, kc, vc, window_of_token, scale):
    """Library routine: torch's scaled_dot_product_attention in float64 on the
    CPU, over all tokens in canonical order with a boolean same-window mask."""
    import torch
    F = torch.nn.functional
    B, L, Hh, D = qc.shape
    win = torch.as_tensor(np.asarray(window_of_token))
    mask = win[:, None] == win[None, :]
    q = torch.as_tensor(qc).permute(0, 2, 1, 3).contiguous()
    k = torch.as_tensor(kc).permute(0, 2, 1, 3).contiguous()
    v = torch.as_tensor(vc).permute(0, 2, 1, 3).contiguous()
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    s = (q @ k.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()
