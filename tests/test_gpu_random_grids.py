"""The whole path on seeded random grids (GPU).

For each case a host RNG draws a grid, window counts, a layout, the batch,
heads, head_dim and the input scale.  The device plans the layout, gathers
Q, K, V into it, runs window attention and scatters O back to canonical
order; the result is compared element by element, in canonical order, with
the oracle's brute force (full attention over the grid with a same-window
mask), and the LSE with its per-row bound.  The draws cover grids inside one
window and grids of up to 30 windows, windows of 10 to 1632 tokens, ragged last
tiles, both layouts, batch 2, both head sizes and peaked score rows."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from oracle import permute as operm
from oracle import plan as oplan
from oracle import text_attention as otxt
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, assert_close_full, lse_bound_windows, say, to_f64
from window_attention_amd.inputs import qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"
MAX_TOKENS = 3000


def _draw(seed):
    rng = np.random.default_rng(seed)
    while True:
        T, H, W = int(rng.integers(1, 5)), int(rng.integers(4, 61)), int(rng.integers(4, 81))
        if T * H * W <= MAX_TOKENS:
            break
    nt, nh, nw = int(rng.integers(1, 4)), int(rng.integers(1, 7)), int(rng.integers(1, 7))
    method = int(rng.integers(0, 2))
    batch = int(rng.integers(1, 3))
    heads = 1 if batch == 2 else int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    sigma = float(rng.choice([1.0, 2.0]))
    return T, H, W, nt, nh, nw, method, batch, heads, D, sigma


@pytest.mark.parametrize("seed", range(12))
def test_random_grid_whole_path(seed):
    T, H, W, nt, nh, nw, method, batch, heads, D, sigma = _draw(seed)
    say(f"random grid seed={seed}: {T}x{H}x{W} counts {nt},{nh},{nw} method {method} B={batch} "
        f"heads={heads} D={D} sigma={sigma}")
    L = T * H * W
    # sigma scales the scores only: V stays unit-scale, since the absolute
    # tolerance is that of unit-scale outputs (at |o| >= 4 the bf16 rounding
    # of the output alone is up to 2^-6)
    q, k, _ = qkv(100 + seed, batch, L, heads, D, sigma, device=DEV)
    v = qkv(100 + seed, batch, L, heads, D, 1.0, device=DEV)[2]
    p = wa.plan(T, H, W, nt, nh, nw, method, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    ow, lse = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen, return_lse=True)
    o = wa.scatter(ow, p.perm)
    torch.cuda.synchronize()

    op = oplan.plan(T, H, W, nt, nh, nw, method)
    assert np.array_equal(p.cu_seqlens.cpu().numpy(), np.asarray(op.cu_seqlens))
    win = np.repeat(np.arange(op.num_windows), np.diff(op.cu_seqlens))[np.asarray(op.inv)]
    qh, kh, vh = to_f64(q), to_f64(k), to_f64(v)
    ref_o, ref_lse = oatt.masked_full_attention(qh, kh, vh, win)
    tol = lse_bound_windows(operm.gather(qh, op.perm), operm.gather(kh, op.perm), op.cu_seqlens)[:, :, op.inv]
    assert_close_full(o, lse[:, :, p.inv.long()], ref_o, ref_lse, tol)


@pytest.mark.parametrize("seed", range(6))
def test_random_grid_with_text(seed):
    """The text-augmented call on the same kind of draws, with 1 to 300 text
    rows: video rows in window order, the text output and the per-window
    text outputs against the oracle's [window, text] segments."""
    T, H, W, nt, nh, nw, method, batch, heads, D, sigma = _draw(1000 + seed)
    text_len = int(np.random.default_rng(2000 + seed).integers(1, 301))
    say(f"random grid with text seed={seed}: {T}x{H}x{W} counts {nt},{nh},{nw} method {method} B={batch} "
        f"heads={heads} D={D} sigma={sigma} text={text_len}")
    L = T * H * W
    q, k, _ = qkv(200 + seed, batch, L, heads, D, sigma, device=DEV)
    v = qkv(200 + seed, batch, L, heads, D, 1.0, device=DEV)[2]
    tq, tk, _ = qkv(300 + seed, batch, text_len, heads, D, sigma, device=DEV)
    tv = qkv(300 + seed, batch, text_len, heads, D, 1.0, device=DEV)[2]
    p = wa.plan(T, H, W, nt, nh, nw, method, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    ws = torch.full((batch, p.num_windows, text_len, heads, D), float("nan"), dtype=torch.float32, device=DEV)
    ow, to = wa.attn_fwd_text(qw, kw, vw, p.cu_seqlens, p.max_seqlen, tq, tk, tv, workspace=ws)
    torch.cuda.synchronize()

    op = oplan.plan(T, H, W, nt, nh, nw, method)
    qh, kh, vh = (operm.gather(to_f64(x), op.perm) for x in (q, k, v))
    ref_o, ref_t, ref_per = otxt.text_window_attention(qh, kh, vh, list(op.cu_seqlens), to_f64(tq), to_f64(tk),
                                                       to_f64(tv))
    for got, want, what in ((to_f64(ow), ref_o, "video"), (to_f64(to), ref_t, "text"),
                            (ws.double().cpu().numpy(), ref_per, "per-window text")):
        err = np.abs(got - want)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, float(err.max()), float(err.mean()))
