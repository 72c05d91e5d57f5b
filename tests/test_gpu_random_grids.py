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
from tests.gpu_helpers import assert_close_full, lse_bound_windows, say, to_f64
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
