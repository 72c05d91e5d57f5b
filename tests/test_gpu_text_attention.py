"""Text-augmented window attention (GPU) against the fp64 oracle: segments
[video window, replicated text], and the text output averaged over windows
(window page, sections "SeedVR2 integration" and "Text stream")."""
import math

import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from oracle import text_attention as otxt
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, lse_bound, output_bound, say, to_f64
from window_attention_amd.inputs import normal, qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _text(B, T, Hh, D, seed):
    return tuple(normal((B, T, Hh, D), seed + t, device=DEV) for t in range(3))


def _close(got, want, what):
    err = np.abs(to_f64(got) - want) if isinstance(got, torch.Tensor) else np.abs(got - want)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, float(err.max()), float(err.mean()))
    return float(err.max())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lengths,T", [([1, 39, 64, 65, 127, 0, 200], 77), ([300, 5], 1), ([64, 128], 64),
                                       ([130], 200)])
def test_small_full_compare(D, lengths, T):
    B, Hh = 2, 2
    cu = _cu(lengths)
    L = int(cu[-1])
    q, k, v = (normal((B, L, Hh, D), 500 + t, device=DEV) for t in range(3))
    tq, tk, tv = _text(B, T, Hh, D, 600)
    cu_d = torch.as_tensor(cu, device=DEV)
    ws = torch.full((B, len(lengths), T, Hh, D), float("nan"), dtype=torch.float32, device=DEV)
    o, to, lse = wa.attn_fwd_text(q, k, v, cu_d, max(lengths), tq, tk, tv, workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh, tqh, tkh, tvh = (to_f64(x) for x in (q, k, v, tq, tk, tv))
    ref_o, ref_t, ref_per = otxt.text_window_attention(qh, kh, vh, cu.tolist(), tqh, tkh, tvh)
    _close(o, ref_o, "video")
    _close(to, ref_t, "text")
    _close(ws.double().cpu().numpy(), ref_per, "per-window text")
    # LSE of video rows: over the segment, against the per-row bound
    s = 1 / math.sqrt(D)
    for b in range(B):
        for i in range(len(lengths)):
            a, e = int(cu[i]), int(cu[i + 1])
            if e <= a:
                continue
            for h in range(Hh):
                ks = np.concatenate([kh[b, a:e, h], tkh[b, :, h]])
                vs = np.concatenate([vh[b, a:e, h], tvh[b, :, h]])
                _, ref_lse = oatt.head_attention(qh[b, a:e, h], ks, vs, s)
                got = lse[b, h, a:e].double().cpu().numpy()
                assert np.all(np.abs(got - ref_lse) <= lse_bound(qh[b, a:e, h], ks, s))


@pytest.mark.parametrize("D", [64, 128])
def test_large_magnitude_values_with_text(D):
    """Window and text values of standard deviation 256: video rows and the
    fp32 per-window text outputs against output_bound over each segment's
    keys, and the text output against the mean of those bounds plus the fp32
    sum over the windows (N + 1 roundings of 2^-24 relative to the mean of
    |per-window output|) and its bf16 rounding (2^-8 relative)."""
    say(f"large values with text D={D}")
    B, Hh, T, sigma = 1, 2, 77, 256.0
    lengths = [1, 65, 700]
    cu = _cu(lengths)
    L, N = int(cu[-1]), len(lengths)
    q, k = (normal((B, L, Hh, D), 560 + t, device=DEV) for t in range(2))
    v = (normal((B, L, Hh, D), 562, device=DEV).float() * sigma).to(torch.bfloat16)
    tq, tk = (normal((B, T, Hh, D), 570 + t, device=DEV) for t in range(2))
    tv = (normal((B, T, Hh, D), 572, device=DEV).float() * sigma).to(torch.bfloat16)
    ws = torch.full((B, N, T, Hh, D), float("nan"), dtype=torch.float32, device=DEV)
    o, to = wa.attn_fwd_text(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), tq, tk, tv, workspace=ws)
    torch.cuda.synchronize()
    qh, kh, vh, tqh, tkh, tvh = (to_f64(x) for x in (q, k, v, tq, tk, tv))
    ref_o, ref_t, ref_per = otxt.text_window_attention(qh, kh, vh, cu.tolist(), tqh, tkh, tvh)
    abs_o, _, abs_per = otxt.text_window_attention(qh, kh, np.abs(vh), cu.tolist(), tqh, tkh, np.abs(tvh))
    got_o, got_t, got_per = to_f64(o), to_f64(to), ws.double().cpu().numpy()
    s = 1 / math.sqrt(D)
    worst = 0.0
    for b in range(B):
        for h in range(Hh):
            per_bounds = []
            for i in range(N):
                a, e = int(cu[i]), int(cu[i + 1])
                ks = np.concatenate([kh[b, a:e, h], tkh[b, :, h]])
                if e > a:
                    bd = output_bound(qh[b, a:e, h], ks, ref_o[b, a:e, h], abs_o[b, a:e, h], s)
                    err = np.abs(got_o[b, a:e, h] - ref_o[b, a:e, h])
                    assert np.all(err <= bd), ("video", i, h, float((err / bd).max()))
                    worst = max(worst, float((err / bd).max()))
                bt = output_bound(tqh[b, :, h], ks, ref_per[b, i, :, h], abs_per[b, i, :, h], s)
                err = np.abs(got_per[b, i, :, h] - ref_per[b, i, :, h])
                assert np.all(err <= bt), ("per-window text", i, h, float((err / bt).max()))
                per_bounds.append(bt)
            mean_abs = np.mean([np.abs(ref_per[b, i, :, h]) for i in range(N)], axis=0)
            bound_t = np.mean(per_bounds, axis=0) * (1 + 2.0 ** -8) + (N + 1) * 2.0 ** -24 * mean_abs \
                + 2.0 ** -8 * np.abs(ref_t[b, :, h])
            err = np.abs(got_t[b, :, h] - ref_t[b, :, h])
            assert np.all(err <= bound_t), ("text", h, float((err / bound_t).max()))
            worst = max(worst, float((err / bound_t).max()))
    say(f"  max |text out| {np.abs(ref_t).max():.1f}, worst error / bound {worst:.3f}")


@pytest.mark.parametrize("scale", [0.05, 0.5])
def test_softmax_scale_with_text(scale):
    """A caller's softmax scale reaches the text keys and the text queries as
    well as the window's."""
    B, Hh, D, T = 1, 2, 128, 70
    lengths = [130, 0, 64, 300]
    cu = _cu(lengths)
    L = int(cu[-1])
    q, k, v = (normal((B, L, Hh, D), 530 + t, device=DEV) for t in range(3))
    tq, tk, tv = _text(B, T, Hh, D, 640)
    o, to = wa.attn_fwd_text(q, k, v, torch.as_tensor(cu, device=DEV), max(lengths), tq, tk, tv,
                             softmax_scale=scale)
    torch.cuda.synchronize()
    qh, kh, vh, tqh, tkh, tvh = (to_f64(x) for x in (q, k, v, tq, tk, tv))
    ref_o, ref_t, _ = otxt.text_window_attention(qh, kh, vh, cu.tolist(), tqh, tkh, tvh, scale)
    _close(o, ref_o, "video")
    _close(to, ref_t, "text")


@pytest.mark.parametrize("where", ["window", "text"])
def test_reference_moves_with_text(where):
    """Scores that climb along the keys, in the window rows or in the text
    rows, so that the softmax reference moves inside window tiles or inside
    text tiles (checked against the oracle element by element)."""
    B, Hh, D, T = 1, 2, 128, 150
    lengths = [300, 64, 7]
    cu = _cu(lengths)
    L = int(cu[-1])
    q, k, v = (normal((B, L, Hh, D), 540 + t, device=DEV) for t in range(3))
    tq, tk, tv = _text(B, T, Hh, D, 560)
    qf, kf, tqf, tkf = (x.float().cpu() for x in (q, k, tq, tk))
    qf[..., 0] = 2.0
    tqf[..., 0] = 2.0
    if where == "window":
        for i in range(len(lengths)):
            a, e = int(cu[i]), int(cu[i + 1])
            kf[:, a:e, :, 0] = torch.arange(e - a, dtype=torch.float32)[None, :, None]
        tkf[..., 0] = 0.0
    else:
        kf[..., 0] = 0.0
        tkf[..., 0] = torch.arange(T, dtype=torch.float32)[None, :, None]
    q, k, tq, tk = (x.to(torch.bfloat16).to(DEV) for x in (qf, kf, tqf, tkf))
    cu_d = torch.as_tensor(cu, device=DEV)
    o, to = wa.attn_fwd_text(q, k, v, cu_d, max(lengths), tq, tk, tv)
    torch.cuda.synchronize()
    qh, kh, vh, tqh, tkh, tvh = (to_f64(x) for x in (q, k, v, tq, tk, tv))
    ref_o, ref_t, _ = otxt.text_window_attention(qh, kh, vh, cu.tolist(), tqh, tkh, tvh)
    _close(o, ref_o, "video")
    _close(to, ref_t, "text")


def test_no_text_is_plain_window_attention_bit_for_bit():
    B, Hh, D = 1, 3, 128
    cu = _cu([1, 130, 64, 257])
    L = int(cu[-1])
    q, k, v = (normal((B, L, Hh, D), 700 + t, device=DEV) for t in range(3))
    cu_d = torch.as_tensor(cu, device=DEV)
    empty = torch.empty((B, 0, Hh, D), dtype=torch.bfloat16, device=DEV)
    o1 = wa.attn_fwd(q, k, v, cu_d, 257)
    o2, t2 = wa.attn_fwd_text(q, k, v, cu_d, 257, empty, empty, empty)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and t2.numel() == 0


def test_full_size_shifted_layout_sampled():
    """21x45x80 shifted layout, 24 heads x 128, 256 text rows: sampled windows
    against the oracle, the text output against the mean of the per-window
    outputs, and the per-window text outputs of sampled windows against the
    oracle."""
    T_, H_, W_ = 21, 45, 80
    p = wa.plan(T_, H_, W_, 4, 3, 3, wa.SHIFTED, device=DEV)
    q, k, v = qkv(31, 1, p.num_tokens, 24, 128, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    Tt = 256
    tq, tk, tv = _text(1, Tt, 24, 128, 800)
    ws = torch.empty((1, p.num_windows, Tt, 24, 128), dtype=torch.float32, device=DEV)
    o, to = wa.attn_fwd_text(qw, kw, vw, p.cu_seqlens, p.max_seqlen, tq, tk, tv, workspace=ws)
    torch.cuda.synchronize()
    mean = ws.double().mean(dim=1).cpu().numpy()
    assert np.abs(to_f64(to) - mean).max() <= 2.0 ** -8 * np.abs(mean).max() + 1e-6   # one bf16 rounding
    cu = p.cu_seqlens.cpu().numpy()
    sizes = np.diff(cu)
    rng = np.random.default_rng(11)
    s = 1 / math.sqrt(128)
    tkh, tvh, tqh = (to_f64(x)[0] for x in (tk, tv, tq))
    worst = 0.0
    for i in sorted({int(np.argmax(sizes)), int(np.argmin(sizes)), *rng.choice(len(sizes), 3, replace=False)}):
        a, e = int(cu[i]), int(cu[i + 1])
        for h in (0, 23):
            ks = np.concatenate([to_f64(kw[0, a:e, h]), tkh[:, h]])
            vs = np.concatenate([to_f64(vw[0, a:e, h]), tvh[:, h]])
            qs = np.concatenate([to_f64(qw[0, a:e, h]), tqh[:, h]])
            ref, _ = oatt.head_attention(qs, ks, vs, s)
            worst = max(worst, _close(o[0, a:e, h], ref[:e - a], "video"))
            worst = max(worst, _close(ws[0, i, :, h].double().cpu().numpy(), ref[e - a:], "text of window"))
    say(f"text attention 21x45x80 S, 256 text rows: worst sampled max-abs {worst:.2e}")


def test_windows_are_isolated():
    B, Hh, D, T = 1, 2, 128, 50
    cu = _cu([90, 200, 33])
    L = int(cu[-1])
    q, k, v = (normal((B, L, Hh, D), 900 + t, device=DEV) for t in range(3))
    tq, tk, tv = _text(B, T, Hh, D, 950)
    cu_d = torch.as_tensor(cu, device=DEV)
    ws1 = torch.empty((B, 3, T, Hh, D), dtype=torch.float32, device=DEV)
    ws2 = torch.empty_like(ws1)
    o1, _ = wa.attn_fwd_text(q, k, v, cu_d, 200, tq, tk, tv, workspace=ws1)
    q2, k2, v2 = (x.clone() for x in (q, k, v))
    for t, x in enumerate((q2, k2, v2)):
        x[:, 90:290] = normal((B, 200, Hh, D), 990 + t, device=DEV)
    o2, _ = wa.attn_fwd_text(q2, k2, v2, cu_d, 200, tq, tk, tv, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :90], o2[:, :90]) and torch.equal(o1[:, 290:], o2[:, 290:])
    assert torch.equal(ws1[:, 0], ws2[:, 0]) and torch.equal(ws1[:, 2], ws2[:, 2])
    assert not torch.equal(ws1[:, 1], ws2[:, 1])


def test_errors():
    B, Hh, D = 1, 2, 128
    q = normal((B, 64, Hh, D), 1, device=DEV)
    cu = torch.as_tensor(_cu([64]), device=DEV)
    t = normal((B, 8, Hh, D), 2, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.attn_fwd_text(q, q.clone(), q.clone(), torch.zeros(1, dtype=torch.int32, device=DEV), 0, t, t, t)
    with pytest.raises(wa.WinAttnError):   # workspace too small
        wa.attn_fwd_text(q, q.clone(), q.clone(), cu, 64, t, t, t,
                         workspace=torch.empty(8, dtype=torch.float32, device=DEV))
    with pytest.raises(wa.WinAttnError):   # text shape does not match
        wa.attn_fwd_text(q, q.clone(), q.clone(), cu, 64, t, t, normal((B, 9, Hh, D), 3, device=DEV))
