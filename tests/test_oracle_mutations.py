"""Plant plausible mistakes in the oracle (CPU only, restored after each test)
and check that at least one pin catches each of them."""
import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import permute as operm
from oracle import plan as oplan
from tests import oracle_pins as pins


def _plan_pins_fail():
    try:
        pins.check_worked_examples(oplan)
        pins.check_size_invariance(oplan)
        pins.check_temporal_cap(oplan)
        pins.check_exact_scales(oplan)
        for n in range(1, 20):
            for w in range(1, 22):
                pins.check_shift_geometry(oplan, n, w)
        for grid in [(1, 3, 4), (3, 5, 7), (4, 6, 6)]:
            for ns in [(1, 26, 35), (2, 17, 9), (3, 9, 9), (1, 5, 33)]:
                for m in (oplan.REGULAR, oplan.SHIFTED):
                    p = oplan.plan(*grid, *ns, m)
                    pins.check_plan_invariants(oplan, p, *grid, *ns, m)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_unmutated_oracle_passes():
    assert not _plan_pins_fail()


def _plan_t_outer(T, H, W, nt, nh, nw, method):
    """Enumeration with t outermost instead of w outermost."""
    wt, wh, ww = oplan.window_size(T, H, W, nt, nh, nw)
    p = oplan.Plan(T, H, W, method, wt, wh, ww)
    p.cu_seqlens.append(0)
    for (t0, t1) in oplan.axis_segments(T, wt, method):
        for (h0, h1) in oplan.axis_segments(H, wh, method):
            for (w0, w1) in oplan.axis_segments(W, ww, method):
                p.boxes.append((t0, t1, h0, h1, w0, w1))
                for t in range(t0, t1):
                    for h in range(h0, h1):
                        for w in range(w0, w1):
                            p.perm.append((t * H + h) * W + w)
                p.cu_seqlens.append(len(p.perm))
    p.inv = [0] * len(p.perm)
    for j, c in enumerate(p.perm):
        p.inv[c] = j
    return p


def _plan_transposed_id(T, H, W, nt, nh, nw, method):
    """Canonical id with h and w swapped."""
    p = _ORIG_PLAN(T, H, W, nt, nh, nw, method)
    p.perm = []
    for (t0, t1, h0, h1, w0, w1) in p.boxes:
        for t in range(t0, t1):
            for h in range(h0, h1):
                for w in range(w0, w1):
                    p.perm.append((t * W + w) * H + h)
    p.inv = [0] * len(p.perm)
    for j, c in enumerate(p.perm):
        if c < len(p.inv):
            p.inv[c] = j
    return p


_ORIG_PLAN = oplan.plan


def _size_floor(T, H, W, nt, nh, nw):
    scale = math.sqrt(oplan.REFERENCE_AREA / (H * W))
    rh, rw = round(H * scale), round(W * scale)
    return min(T, 30) // nt or 1, rh // nh or 1, rw // nw or 1


def _size_trunc_round(T, H, W, nt, nh, nw):
    scale = math.sqrt(oplan.REFERENCE_AREA / (H * W))
    rh, rw = int(H * scale), int(W * scale)
    return -(-min(T, 30) // nt), -(-rh // nh), -(-rw // nw)


def _size_no_cap(T, H, W, nt, nh, nw):
    scale = math.sqrt(oplan.REFERENCE_AREA / (H * W))
    rh, rw = round(H * scale), round(W * scale)
    return -(-T // nt), -(-rh // nh), -(-rw // nw)


def _shifted_ceil_half(n, w):
    """The rejected reading: cut k*w - floor(w/2)."""
    if w >= n:
        return [(0, n)]
    cuts = [0] + [k * w - w // 2 for k in range(1, n + 2) if 0 < k * w - w // 2 < n] + [n]
    return [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]


def _shifted_rolled(n, w):
    """Cyclic shift: the last partial window wraps around to the first."""
    if w >= n:
        return [(0, n)]
    o = w // 2
    return [(a + o, min(a + o + w, n)) for a in range(0, n - o, w)] + ([(0, o)] if o else [])


def _shifted_always(n, w):
    """Shift even when the window covers the axis."""
    o = w // 2
    cuts = [0] + [o + k * w for k in range(n + 1) if 0 < o + k * w < n] + [n]
    return [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]


def _regular_unclipped(n, w):
    return [(k * w, (k + 1) * w) for k in range(-(-n // w))]


PLAN_MUTANTS = {
    "t_outer_enumeration": ("plan", _plan_t_outer),
    "transposed_canonical_id": ("plan", _plan_transposed_id),
    "floor_instead_of_ceil": ("window_size", _size_floor),
    "truncating_round": ("window_size", _size_trunc_round),
    "no_temporal_cap": ("window_size", _size_no_cap),
    "shift_cut_rejected_reading": ("shifted_segments", _shifted_ceil_half),
    "rolled_shift": ("shifted_segments", _shifted_rolled),
    "shift_covering_axis": ("shifted_segments", _shifted_always),
    "regular_unclipped": ("regular_segments", _regular_unclipped),
}


@pytest.mark.parametrize("name", sorted(PLAN_MUTANTS))
def test_plan_mutant_is_caught(name, monkeypatch):
    attr, fn = PLAN_MUTANTS[name]
    monkeypatch.setattr(oplan, attr, fn)
    assert _plan_pins_fail(), f"pins did not catch mutant {name}"


# ------------------------------------------------------------------ attention

def _head_scale_inverted(q, k, v, scale):
    return _ORIG_HEAD(q, k, v, 1.0 / scale)


def _head_softmax_wrong_axis(q, k, v, scale):
    s = (q @ k.T) * scale
    e = np.exp(s - s.max(axis=0, keepdims=True))
    z = e.sum(axis=0, keepdims=True)
    return (e / z) @ v, np.log(z[0]) + s.max(axis=0)


def _head_transposed_p(q, k, v, scale):
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z).T @ v, (m + np.log(z))[:, 0]


def _head_k_for_v(q, k, v, scale):
    return _ORIG_HEAD(q, k, k, scale)


_ORIG_HEAD = oatt.head_attention


def _window_attention_off_by_one(q, k, v, cu, scale=None):
    cu = list(cu)
    cu2 = [cu[0]] + [min(c + 1, cu[-1]) for c in cu[1:-1]] + [cu[-1]]
    return _ORIG_WA(q, k, v, cu2, scale)


_ORIG_WA = oatt.window_attention


def _attention_pins_fail():
    try:
        T, H, W, nt, nh, nw = 3, 5, 7, 2, 17, 9
        p = oplan.plan(T, H, W, nt, nh, nw, oplan.SHIFTED)
        L, Hh, D = T * H * W, 2, 16
        rng = np.random.default_rng(3)
        qc, kc, vc = (rng.standard_normal((1, L, Hh, D)) for _ in range(3))
        ow, lw = oatt.window_attention(operm.gather(qc, p.perm), operm.gather(kc, p.perm),
                                       operm.gather(vc, p.perm), p.cu_seqlens)
        o = operm.scatter(ow, p.perm)
        win = np.empty(L, dtype=np.int64)
        for i in range(p.num_windows):
            win[np.asarray(p.perm[p.cu_seqlens[i]:p.cu_seqlens[i + 1]])] = i
        ot, lt = pins.torch_sdpa_masked(qc, kc, vc, win, 1.0 / math.sqrt(D))
        assert np.max(np.abs(o - ot)) < 1e-12
        assert np.max(np.abs(lw[:, :, p.inv] - lt)) < 1e-12
    except (AssertionError, ValueError, IndexError):
        return True
    return False


ATTN_MUTANTS = {
    "scale_inverted": ("head_attention", _head_scale_inverted),
    "softmax_wrong_axis": ("head_attention", _head_softmax_wrong_axis),
    "transposed_probabilities": ("head_attention", _head_transposed_p),
    "keys_used_as_values": ("head_attention", _head_k_for_v),
    "window_bounds_off_by_one": ("window_attention", _window_attention_off_by_one),
}


def test_unmutated_attention_passes():
    assert not _attention_pins_fail()


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name, monkeypatch):
    attr, fn = ATTN_MUTANTS[name]
    monkeypatch.setattr(oatt, attr, fn)
    assert _attention_pins_fail(), f"pins did not catch mutant {name}"


def test_permute_mutant_is_caught(monkeypatch):
    # scatter written as a gather (perm and its inverse confused)
    monkeypatch.setattr(operm, "scatter", lambda x, perm: x[:, np.argsort(np.argsort(perm))])
    p = oplan.plan(1, 3, 4, 1, 26, 35, oplan.REGULAR)
    x = np.arange(12)[None, :]
    assert not np.array_equal(operm.scatter(operm.gather(x, p.perm), p.perm), x)


# ----------------------------------------------------------------- packing

from oracle import pack as opack  # noqa: E402


def _pack_pins_fail():
    def fn(perms, cus, align):
        k = opack.pack_plans(perms, cus, align)
        return k.offsets, k.perm, k.cu_seqlens, k.max_seqlen
    try:
        pins.check_pack_worked_example(fn)
        plans = [oplan.plan(5, 9, 16, 2, 6, 6, oplan.REGULAR), oplan.plan(2, 5, 7, 1, 2, 3, oplan.SHIFTED)]
        for align in (1, 7, 64):
            pins.check_pack_invariants(fn, [list(p.perm) for p in plans], [list(p.cu_seqlens) for p in plans], align)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _pack_variant(skip_empty_tail=False, unshifted=False, full_tail=False, total_max=False):
    def pack_plans(perms, cus, align):
        offsets, perm, cu, longest = [0], [], [0], 0
        for p, c in zip(perms, cus):
            n, o = len(p), offsets[-1]
            for a, b in zip(c[:-1], c[1:]):
                cu.append(o + b)
                longest = max(longest, b - a)
            perm.extend(x if unshifted else o + x for x in p)
            t = align - n % align if full_tail else (align - n % align) % align
            perm.extend(range(o + n, o + n + t))
            if t or not skip_empty_tail:
                cu.append(o + n + t)
            longest = max(longest, t)
            offsets.append(o + n + t)
        return opack.Packed(offsets, perm, cu, offsets[-1] if total_max else longest)
    return pack_plans


def test_unmutated_pack_passes():
    assert not _pack_pins_fail()


@pytest.mark.parametrize("flag", ["skip_empty_tail", "unshifted", "full_tail", "total_max"])
def test_pack_mutant_is_caught(flag, monkeypatch):
    monkeypatch.setattr(opack, "pack_plans", _pack_variant(**{flag: True}))
    assert _pack_pins_fail(), f"pins did not catch packing mutant {flag}"


# ------------------------------------------------------- sequence-parallel tables

from oracle import sp_plan as osp  # noqa: E402


def _sp_pins_fail():
    try:
        pins.check_lpt_worked_examples(osp.lpt_assign)
        pins.check_plan_a_worked_example(
            lambda a, b: (lambda t: (t.counts, t.send_rows, t.recv_pos, t.exchange_required))(osp.plan_a(a, b)))
        p = oplan.plan(5, 9, 16, 2, 6, 6, oplan.SHIFTED)
        sizes = [p.cu_seqlens[i + 1] - p.cu_seqlens[i] for i in range(p.num_windows)]
        for ranks in (2, 3):
            pins.check_lpt_invariants(osp.lpt_assign, sizes, ranks)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _lpt_variant(rank_tie_high=False, ascending=False, keep_lpt_order=False):
    def lpt_assign(sizes, ranks):
        order = sorted(range(len(sizes)), key=lambda w: ((sizes[w] if ascending else -sizes[w]), w))
        load, owner, lists = [0] * ranks, [-1] * len(sizes), [[] for _ in range(ranks)]
        for w in order:
            r = min(range(ranks), key=lambda x: (load[x], -x if rank_tie_high else x))
            owner[w] = r
            load[r] += sizes[w]
            lists[r].append(w)
        if not keep_lpt_order:
            lists = [sorted(x) for x in lists]
        return owner, lists, load
    return lpt_assign


def _plan_a_source_order(z_src, z_dst):
    # peer segments packed in source-local order instead of destination-local order
    P = len(z_src)
    where = {c: (d, pos) for d, z in enumerate(z_dst) for pos, c in enumerate(z)}
    counts = [[0] * P for _ in range(P)]
    send, recv_parts = [], [[[] for _ in range(P)] for _ in range(P)]
    for r, z in enumerate(z_src):
        groups = [[] for _ in range(P)]
        for i, c in enumerate(z):
            d, pos = where[c]
            counts[r][d] += 1
            groups[d].append(i)
            recv_parts[d][r].append(pos)
        send.append([i for g in groups for i in g])
    recv = [[p for part in recv_parts[d] for p in part] for d in range(P)]
    return osp.PlanA(counts, send, recv, any(counts[r][d] for r in range(P) for d in range(P) if r != d))


def test_unmutated_sp_tables_pass():
    assert not _sp_pins_fail()


@pytest.mark.parametrize("flag", ["rank_tie_high", "ascending", "keep_lpt_order"])
def test_lpt_mutant_is_caught(flag, monkeypatch):
    monkeypatch.setattr(osp, "lpt_assign", _lpt_variant(**{flag: True}))
    assert _sp_pins_fail(), f"pins did not catch LPT mutant {flag}"


def test_plan_a_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(osp, "plan_a", _plan_a_source_order)
    assert _sp_pins_fail(), "pins did not catch Plan A packed in source order"


# ---------------------------------------------------------------------- RoPE

import math as _math  # noqa: E402

from oracle import rope as orope  # noqa: E402


def _rope_pins_fail():
    try:
        pins.check_rope_worked_example(orope.rotate)
        pins.check_rope_positions(orope.window_local_positions, oplan)
        pins.check_rope_properties(orope.rotate, 12, 14)
        pins.check_rope_window_restart(orope.window_local_positions, oplan)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _rotate_variant(axis_order=(0, 1, 2), half_split=False, span_exponent=False):
    def rotate(x, pos, rope_dim, base=orope.DEFAULT_BASE):
        d = rope_dim // 3
        y = np.array(x, dtype=np.float64, copy=True)
        for blk, axis in enumerate(axis_order):
            for i in range(d // 2):
                ang = pos[axis] * base ** (-2.0 * i / (rope_dim if span_exponent else d))
                c, s = _math.cos(ang), _math.sin(ang)
                a, b = (blk * d + i, blk * d + i + d // 2) if half_split else (blk * d + 2 * i, blk * d + 2 * i + 1)
                y[..., a] = x[..., a] * c - x[..., b] * s
                y[..., b] = x[..., a] * s + x[..., b] * c
        return y
    return rotate


def _positions_variant(text_on_h=False, global_pos=False):
    def window_local_positions(plan, text_len):
        H, W = plan.H, plan.W
        out = []
        for i, (t0, t1, h0, h1, w0, w1) in enumerate(plan.boxes):
            for j in range(plan.cu_seqlens[i], plan.cu_seqlens[i + 1]):
                t, rem = divmod(plan.perm[j], H * W)
                h, w = divmod(rem, W)
                if global_pos:
                    t0 = h0 = w0 = 0
                pt, ph = t - t0, h - h0
                out.append((pt, ph + text_len, w - w0) if text_on_h else (pt + text_len, ph, w - w0))
        return out
    return window_local_positions


def test_unmutated_rope_passes():
    assert not _rope_pins_fail()


@pytest.mark.parametrize("kw", [{"axis_order": (2, 1, 0)}, {"half_split": True}, {"span_exponent": True}])
def test_rope_rotation_mutant_is_caught(kw, monkeypatch):
    monkeypatch.setattr(orope, "rotate", _rotate_variant(**kw))
    assert _rope_pins_fail(), f"pins did not catch rotation mutant {kw}"


@pytest.mark.parametrize("kw", [{"text_on_h": True}, {"global_pos": True}])
def test_rope_position_mutant_is_caught(kw, monkeypatch):
    monkeypatch.setattr(orope, "window_local_positions", _positions_variant(**kw))
    assert _rope_pins_fail(), f"pins did not catch position mutant {kw}"


# ------------------------------------------------------------ text attention

from oracle import text_attention as otxt  # noqa: E402


def _text_pins_fail():
    try:
        pins.check_text_closed_form(otxt.text_window_attention)
        pins.check_text_brute_force(otxt.text_window_attention)
        pins.check_text_isolation(otxt.text_window_attention)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _text_variant(video_without_text=False, token_weighted=False, text_only_keys=False, count_plus_one=False):
    def text_window_attention(q, k, v, cu, tq, tk, tv, scale=None):
        B, L, Hh, D = q.shape
        T = tq.shape[1]
        s = 1.0 / math.sqrt(D) if scale is None else scale
        N = len(cu) - 1
        o = np.zeros((B, L, Hh, D))
        per = np.zeros((B, N, T, Hh, D))
        weights = []
        for i in range(N):
            a, e = cu[i], cu[i + 1]
            weights.append(e - a)
            for b in range(B):
                for h in range(Hh):
                    ks = np.concatenate([k[b, a:e, h], tk[b, :, h]])
                    vs = np.concatenate([v[b, a:e, h], tv[b, :, h]])
                    if e > a:
                        kk, vv = (k[b, a:e, h], v[b, a:e, h]) if video_without_text else (ks, vs)
                        o[b, a:e, h] = oatt.head_attention(q[b, a:e, h], kk, vv, s)[0]
                    if T:
                        kk, vv = (tk[b, :, h], tv[b, :, h]) if text_only_keys else (ks, vs)
                        per[b, i, :, h] = oatt.head_attention(tq[b, :, h], kk, vv, s)[0]
        if token_weighted:
            w = np.asarray(weights, dtype=float) + T
            text = np.einsum("bn...,n->b...", per, w) / w.sum()
        else:
            text = per.sum(axis=1) / (N + 1 if count_plus_one else N)
        return o, text, per
    return text_window_attention


def test_unmutated_text_attention_passes():
    assert not _text_pins_fail()


@pytest.mark.parametrize("flag", ["video_without_text", "token_weighted", "text_only_keys", "count_plus_one"])
def test_text_attention_mutant_is_caught(flag, monkeypatch):
    monkeypatch.setattr(otxt, "text_window_attention", _text_variant(**{flag: True}))
    assert _text_pins_fail(), f"pins did not catch text-attention mutant {flag}"
