"""win_attn_fwd against the fp64 oracle (GPU).

Small cases are compared element by element over every output; the full-size
workloads are run in the same launch configuration the benchmark times and
compared on sampled (batch, window, head) blocks that the oracle computes one
by one, choosing the largest, smallest and edge windows."""
import math

import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from oracle import permute as operm
from oracle import plan as oplan
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, assert_close_full, lse_bound, lse_bound_windows, \
    method_of, output_bound, say, to_f64
from window_attention_amd.inputs import bf16_bits, normal, qkv
from window_attention_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lengths", [
    [1, 39, 64, 65, 127, 128, 129, 200],      # single token, sub-tile, tile edges, multi-tile ragged tails
    [300, 0, 0, 257, 5],                      # empty segments in the middle
    [700],                                    # several key tiles and query tiles, ragged tail
])
def test_ragged_segments_full_compare(D, lengths):
    say(f"ragged D={D} lengths={lengths}")
    cu = _cu(lengths)
    L, B, Hh = int(cu[-1]), 2, 3
    q, k, v = (normal((B, L, Hh, D), 500 + t, device=DEV) for t in range(3))
    o, lse = wa.attn_fwd(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), return_lse=True)
    qh, kh = to_f64(q), to_f64(k)
    ref_o, ref_lse = oatt.window_attention(qh, kh, to_f64(v), cu)
    assert_close_full(o, lse, ref_o, ref_lse, lse_bound_windows(qh, kh, cu))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [0.02, 0.3, 1.0])
def test_softmax_scale(D, scale):
    """A caller's softmax scale other than 1/sqrt(D): near-uniform rows
    (0.02) and peaked rows whose reference moves (1.0, scores of standard
    deviation sqrt(D)); O and the LSE, log sum_k exp(scale * s_k), against
    the oracle with the same scale.  V has standard deviation 1/2: a peaked
    row's output is one V row, and above 4 in magnitude the bf16 rounding of
    the output alone (up to 2^-6) would use most of the absolute tolerance."""
    say(f"softmax scale D={D} scale={scale}")
    lengths = [1, 65, 200, 700]
    cu = _cu(lengths)
    L, B, Hh = int(cu[-1]), 1, 2
    q, k = (normal((B, L, Hh, D), 520 + t, device=DEV) for t in range(2))
    v = normal((B, L, Hh, D), 522, sigma=0.5, device=DEV)
    o, lse = wa.attn_fwd(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), softmax_scale=scale,
                         return_lse=True)
    qh, kh = to_f64(q), to_f64(k)
    ref_o, ref_lse = oatt.window_attention(qh, kh, to_f64(v), cu, scale)
    assert_close_full(o, lse, ref_o, ref_lse, lse_bound_windows(qh, kh, cu, scale))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sigma,offset", [(16.0, 0.0), (256.0, 0.0), (1.0, 1000.0)])
def test_large_magnitude_values(D, sigma, offset):
    """V far from unit scale (standard deviation 16 or 256, or 1000 plus unit
    noise), where an absolute tolerance says nothing: every element of O
    against the oracle within output_bound, a bound from the kernel's
    arithmetic that scales with |O| and with sum_k p_k |v_k| (the oracle's
    attention applied to |V|).  The LSE does not depend on V and keeps its
    own bound."""
    say(f"large values D={D} sigma={sigma} offset={offset}")
    lengths = [1, 65, 700, 2430]
    cu = _cu(lengths)
    L, B, Hh = int(cu[-1]), 1, 2
    q, k = (normal((B, L, Hh, D), 540 + t, device=DEV) for t in range(2))
    v = (normal((B, L, Hh, D), 542, device=DEV).float() * sigma + offset).to(torch.bfloat16)
    o, lse = wa.attn_fwd(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), return_lse=True)
    qh, kh, vh = to_f64(q), to_f64(k), to_f64(v)
    ref_o, ref_lse = oatt.window_attention(qh, kh, vh, cu)
    pv_abs, _ = oatt.window_attention(qh, kh, np.abs(vh), cu)
    got = to_f64(o)
    scale = 1.0 / math.sqrt(D)
    worst = 0.0
    for b in range(B):
        for i in range(len(lengths)):
            a, e = int(cu[i]), int(cu[i + 1])
            for h in range(Hh):
                bound = output_bound(qh[b, a:e, h], kh[b, a:e, h], ref_o[b, a:e, h], pv_abs[b, a:e, h], scale)
                err = np.abs(got[b, a:e, h] - ref_o[b, a:e, h])
                assert np.all(err <= bound), f"window {i} head {h}: worst ratio {(err / bound).max():.3f}"
                worst = max(worst, float((err / bound).max()))
    le = np.abs(lse.double().cpu().numpy() - ref_lse)
    assert np.all(le <= lse_bound_windows(qh, kh, cu))
    say(f"  max |O| {np.abs(ref_o).max():.1f}, max abs err {np.abs(got - ref_o).max():.3g}, "
        f"worst error / bound {worst:.3f}")


def _steer_scores(q, k, cu, pattern):
    """Make channel 0 decide the score trend along each window's keys: every
    query gets q_0 = 2 and key j (0-based inside its window) gets
      grow:   k_0 = j       (scores climb about 16 powers of two per key tile,
                             so the reference moves in every tile),
      jump:   k_0 = 3000 at one key in the middle of the window, else 0
              (exp2 against the old reference overflows: only the recompute
              from the K tile gives a finite result),
      shrink: k_0 = -j      (later tiles underflow; the reference never moves).
    Values are set on host copies and cast to bf16, so the oracle reads the
    same bytes."""
    qf, kf = q.float().cpu(), k.float().cpu()
    qf[..., 0] = 2.0
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        j = torch.arange(e - a, dtype=torch.float32)
        if pattern == "grow":
            kf[:, a:e, :, 0] = j[None, :, None]
        elif pattern == "shrink":
            kf[:, a:e, :, 0] = -j[None, :, None]
        else:
            kf[:, a:e, :, 0] = 0.0
            if e > a:
                kf[:, a + (e - a) // 2 + 3 if (e - a) // 2 + 3 < e - a else a, :, 0] = 3000.0
    return qf.to(torch.bfloat16).to(q.device), kf.to(torch.bfloat16).to(k.device)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pattern", ["grow", "jump", "shrink"])
def test_reference_moves(D, pattern):
    """Score trends that move (or never move) the softmax reference, checked
    element by element against the oracle: several key tiles, a window of
    exactly one tile, and one shorter than a tile."""
    say(f"reference moves D={D} pattern={pattern}")
    lengths = [700, 64, 130, 5]
    cu = _cu(lengths)
    L, B, Hh = int(cu[-1]), 1, 2
    q, k, v = (normal((B, L, Hh, D), 520 + t, device=DEV) for t in range(3))
    q, k = _steer_scores(q, k, cu, pattern)
    o, lse = wa.attn_fwd(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), return_lse=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    qh, kh = to_f64(q), to_f64(k)
    ref_o, ref_lse = oatt.window_attention(qh, kh, to_f64(v), cu)
    assert_close_full(o, lse, ref_o, ref_lse, lse_bound_windows(qh, kh, cu))


def test_rows_outside_windows_untouched_and_empty_plan():
    D, Hh, L = 128, 2, 96
    q, k, v = (normal((1, L, Hh, D), 600 + t, device=DEV) for t in range(3))
    cu = torch.tensor([0, 40, 70], dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    lse = wa.attn_fwd(q, k, v, cu, 40, out=out, return_lse=True)[1]
    assert torch.all(out[:, 70:] == 7.0)
    qh, kh = to_f64(q), to_f64(k)
    ref_o, ref_lse = oatt.window_attention(qh, kh, to_f64(v), [0, 40, 70])
    tol = lse_bound_windows(qh, kh, [0, 40, 70])
    assert_close_full(out[:, :70], lse[:, :, :70], ref_o[:, :70], ref_lse[:, :, :70], tol[:, :, :70])
    # no windows at all: nothing is written
    out2 = torch.full_like(q, 3.0)
    wa.attn_fwd(q, k, v, torch.zeros(1, dtype=torch.int32, device=DEV), 0, out=out2)
    torch.cuda.synchronize()
    assert torch.all(out2 == 3.0)


def test_closed_forms_on_device():
    # Q = 0: every row is its window's mean of V; LSE = log(n)
    D, Hh = 128, 2
    lengths = [5, 77, 130]
    cu = _cu(lengths)
    L = int(cu[-1])
    q = torch.zeros((1, L, Hh, D), dtype=torch.bfloat16, device=DEV)
    k, v = (normal((1, L, Hh, D), 700 + t, device=DEV) for t in range(2))
    o, lse = wa.attn_fwd(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), return_lse=True)
    vh = to_f64(v)
    for i, n in enumerate(lengths):
        a, e = cu[i], cu[i + 1]
        mean = vh[:, a:e].mean(axis=1, keepdims=True)
        assert np.max(np.abs(to_f64(o[:, a:e]) - mean)) <= MAX_ABS
        # q = 0: every score is 0 exactly, so only the normaliser's rounding is left
        bound = lse_bound(np.zeros((n, D)), to_f64(k[0, a:e, 0]), 1.0 / math.sqrt(D))
        assert np.all(np.abs(lse[:, :, a:e].double().cpu().numpy() - math.log(n)) <= bound)


@pytest.mark.parametrize("method", [0, 1])
def test_tiny_clip_both_layouts(method):
    """5x9x16 grid, 1 head x 64, fp32 draws cast to bf16 on the device; the
    oracle runs on exactly the bf16 values; outputs compared in canonical
    order against the masked brute force as well."""
    w = WORKLOADS[0]
    qf, kf, vf = qkv(w.wid, 1, w.L, w.heads, w.head_dim, device=DEV, dtype=torch.float32)
    q, k, v = (x.to(torch.bfloat16) for x in (qf, kf, vf))
    p = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    ow, lse = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen, return_lse=True)
    o = wa.scatter(ow, p.perm)
    op = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method)
    win = np.repeat(np.arange(op.num_windows), np.diff(op.cu_seqlens))[np.asarray(op.inv)]
    qh, kh = to_f64(q), to_f64(k)
    ref_o, ref_lse = oatt.masked_full_attention(qh, kh, to_f64(v), win)
    # per-row LSE bound computed in window order, then taken to canonical order
    tol = lse_bound_windows(operm.gather(qh, op.perm), operm.gather(kh, op.perm), op.cu_seqlens)[:, :, op.inv]
    assert_close_full(o, lse[:, :, p.inv.long()], ref_o, ref_lse, tol)


def test_clip_720p_full_compare():
    """4x45x80 clip, 24 heads x 128, regular layout: every output compared."""
    w = WORKLOADS[1]
    say(f"full compare {w.name}")
    q, k, v = qkv(w.wid, w.batch, w.L, w.heads, w.head_dim, w.sigma, device=DEV)
    p = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    ow, lse = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen, return_lse=True)
    o = wa.scatter(ow, p.perm)
    op = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0)
    qw_h, kw_h = operm.gather(to_f64(q), op.perm), operm.gather(to_f64(k), op.perm)
    ref_w, ref_lse = oatt.window_attention(qw_h, kw_h, operm.gather(to_f64(v), op.perm), op.cu_seqlens)
    assert_close_full(o, None, operm.scatter(ref_w, op.perm), None)
    assert np.all(np.abs(lse.double().cpu().numpy() - ref_lse) <= lse_bound_windows(qw_h, kw_h, op.cu_seqlens))


def _run_chain(w, q, k, v):
    """The benchmark's step: gather into the entry layout, then per layer a
    fused transition when the layout changes and window attention; returns
    per-layer (layout, carried q/k/v, o, lse, plan)."""
    plans = {m: wa.plan_cached(w.T, w.H, w.W, w.nt, w.nh, w.nw, method_of(m), device=DEV) for m in "RS"}
    cur = w.entry
    qw, kw, vw = (wa.gather(x, plans[cur].perm) for x in (q, k, v))
    layers = []
    for lay in w.schedule:
        if lay != cur:
            qw, kw, vw = (wa.transition(x, plans[cur].inv, plans[lay].perm) for x in (qw, kw, vw))
            cur = lay
        p = plans[lay]
        o, lse = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen, return_lse=True)
        layers.append((lay, (qw, kw, vw), o, lse, p))
    return layers


@pytest.mark.parametrize("wi", [2, 3, 4])
def test_full_size_workloads(wi):
    """The benchmark's chain on the three full-size grids.  Every layer's
    carried Q, K, V are compared in full with the canonical tensors gathered
    by the oracle's permutation; the attention output of every window and
    batch element is compared with the oracle for three heads (the first, the
    last and one drawn at random; the 21x45x80 grid is compared for every
    head in test_gpu_headline_full)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    w = WORKLOADS[wi]
    q, k, v = qkv(w.wid, w.batch, w.L, w.heads, w.head_dim, w.sigma, device=DEV)
    layers = _run_chain(w, q, k, v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + wi)
    heads = sorted({0, w.heads - 1, int(rng.integers(1, w.heads - 1))})
    for li, (lay, (qw, kw, vw), o, lse, p) in enumerate(layers):
        op = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method_of(lay))
        perm = torch.as_tensor(np.asarray(op.perm, dtype=np.int64), device=DEV)
        for x_can, x_lay in ((q, qw), (k, kw), (v, vw)):
            assert torch.equal(x_lay, x_can[:, perm])
        cu = np.asarray(op.cu_seqlens)
        hq, hk, hv, ho = (bf16_bits(x[:, :, heads]) for x in (qw, kw, vw, o))  # [B, L, 3, D]
        hl = lse[:, heads].double().cpu().numpy()                            # [B, 3, L]
        scale = 1.0 / math.sqrt(w.head_dim)

        def block(job):
            b, i, hi = job
            a, e = int(cu[i]), int(cu[i + 1])
            qh, kh, vh, oh = (oatt.bf16_bits_to_float64(x[b, a:e, hi]) for x in (hq, hk, hv, ho))
            ref, ref_lse = oatt.head_attention(qh, kh, vh, scale)
            err = np.abs(oh - ref)
            lr = np.abs(hl[b, hi, a:e] - ref_lse) / lse_bound(qh, kh, scale)
            return float(err.max()), float(err.sum()), err.size, float(lr.max())

        jobs = [(b, i, hi) for b in range(w.batch) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]
                for hi in range(len(heads))]
        with threadpool_limits(limits=2), ThreadPoolExecutor(max_workers=8) as ex:
            res = list(ex.map(block, jobs))
        mx = max(r[0] for r in res)
        mean = sum(r[1] for r in res) / sum(r[2] for r in res)
        lr = max(r[3] for r in res)
        say(f"{w.name} layer {li} ({lay}): {len(jobs)} (batch, window, head) blocks, heads {heads}: max {mx:.3e} "
            f"mean {mean:.3e} lse/bound {lr:.3f}")
        assert mx <= MAX_ABS and mean <= MEAN_ABS and lr <= 1.0, (w.name, li, mx, mean, lr)


def test_batch_invariance_hd_grid():
    """Element 1 of the B=2 run of the 21x68x120 grid equals a B=1 run on the
    same draws, bit for bit, in both layouts."""
    w = WORKLOADS[3]
    q, k, v = qkv(w.wid, 2, w.L, w.heads, w.head_dim, w.sigma, device=DEV)
    q1, k1, v1 = qkv(w.wid, 1, w.L, w.heads, w.head_dim, w.sigma, device=DEV, batch_offset=1)
    assert torch.equal(q1[0], q[1]) and torch.equal(v1[0], v[1])
    for m in (0, 1):
        p = wa.plan_cached(w.T, w.H, w.W, w.nt, w.nh, w.nw, m, device=DEV)
        o2 = wa.attn_fwd(wa.gather(q, p.perm), wa.gather(k, p.perm), wa.gather(v, p.perm), p.cu_seqlens,
                         p.max_seqlen)
        o1 = wa.attn_fwd(wa.gather(q1, p.perm), wa.gather(k1, p.perm), wa.gather(v1, p.perm), p.cu_seqlens,
                         p.max_seqlen)
        assert torch.equal(o2[1], o1[0])


def test_isolation_and_determinism():
    """Change every token of one window: every other window's output is
    bit-identical; repeated runs are bit-identical."""
    w = WORKLOADS[1]
    q, k, v = qkv(w.wid, 1, w.L, w.heads, w.head_dim, device=DEV)
    p = wa.plan_cached(w.T, w.H, w.W, w.nt, w.nh, w.nw, 1, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    o = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen)
    o_again = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen)
    assert torch.equal(o, o_again)
    cu = p.cu_seqlens.cpu().numpy()
    i = 5
    a, e = int(cu[i]), int(cu[i + 1])
    q2, k2, v2 = qw.clone(), kw.clone(), vw.clone()
    for x in (q2, k2, v2):
        x[:, a:e] = -x[:, a:e] * 0.5
    o2 = wa.attn_fwd(q2, k2, v2, p.cu_seqlens, p.max_seqlen)
    assert torch.equal(o2[:, :a], o[:, :a]) and torch.equal(o2[:, e:], o[:, e:])
    assert not torch.equal(o2[:, a:e], o[:, a:e])


def test_argument_errors():
    q = torch.zeros((1, 8, 1, 96), dtype=torch.bfloat16, device=DEV)
    cu = torch.tensor([0, 8], dtype=torch.int32, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.attn_fwd(q, q, q, cu, 8)            # head_dim 96
    q = torch.zeros((1, 8, 1, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.attn_fwd(q, q, q, cu, 8)            # fp16 inputs
    q = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.attn_fwd(q, q, q, cu, 8, out=q)     # output aliases the inputs


def test_default_scale_sentinel():
    """softmax_scale None passes 0, which the library turns into
    1/sqrt(head_dim): bit-identical to passing that value."""
    lengths = [130, 64, 7]
    cu = torch.as_tensor(_cu(lengths), device=DEV)
    for D in (64, 128):
        q, k, v = (normal((1, sum(lengths), 2, D), 540 + t, device=DEV) for t in range(3))
        o0, l0 = wa.attn_fwd(q, k, v, cu, max(lengths), return_lse=True)
        o1, l1 = wa.attn_fwd(q, k, v, cu, max(lengths), softmax_scale=1.0 / math.sqrt(D), return_lse=True)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
