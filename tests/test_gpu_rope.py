"""Window-local 3D RoPE fused into the gather / transition (GPU), against the
fp64 oracle: every rotated value within half a bf16 unit in the last place of
the exact rotation plus the fp32 evaluation slack of its pair, channels past
the span bit-identical, and a transition equal to the direct rotated gather."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import plan as oplan
from oracle import rope as orope
from tests.gpu_helpers import say, to_f64
from window_attention_amd.inputs import normal

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ulp_bf16(x):
    """Spacing of bf16 values at |x| (normal range; the smallest normal
    spacing below it)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def _assert_rotated(got, src_rows_f64, positions, rope_dim):
    """Each rotated value is the bf16 rounding of x0*c - x1*s (or x0*s +
    x1*c) evaluated in fp32 with fp32-rounded (c, s): that evaluation is off
    the exact value by a few units of 2^-24 * (|x0| + |x1|) -- relative to
    the pair, not to the result, which can be small when the two products
    cancel -- so the rounded value may land on the far side of a rounding
    boundary by that much.  Bound: half a bf16 spacing of the exact value plus
    2^-21 * (|x0| + |x1|)."""
    want = orope.rope_rows(src_rows_f64, positions, rope_dim)
    g = to_f64(got)
    span = 3 * (rope_dim // 3)
    err = np.abs(g[..., :span] - want[..., :span])
    x = np.abs(src_rows_f64[..., :span])
    pair = np.repeat(x[..., 0::2] + x[..., 1::2], 2, axis=-1)
    bound = 0.5 * _ulp_bf16(want[..., :span]) + 2.0 ** -21 * pair + 2.0 ** -130
    assert np.all(err <= bound), f"worst error / bound {np.max(err / bound):.3f}"
    assert np.array_equal(g[..., span:], src_rows_f64[..., span:])
    return float(np.max(err / bound))


def _oplan(T, H, W, nt, nh, nw, m):
    return oplan.plan(T, H, W, nt, nh, nw, m)


@pytest.mark.parametrize("grid", [(5, 9, 16, 2, 6, 6), (3, 10, 12, 2, 2, 2), (21, 45, 80, 4, 3, 3)])
@pytest.mark.parametrize("method", [wa.REGULAR, wa.SHIFTED])
def test_device_local_positions_match_oracle(grid, method):
    p = wa.plan(*grid, method, device=DEV)
    loc = wa.local_positions(p, device=DEV).cpu().numpy()
    want = np.asarray(orope.window_local_positions(_oplan(*grid, method), 0))
    assert np.array_equal(loc, want)


@pytest.mark.parametrize("D,rope_dim,heads", [(128, 128, 4), (128, 126, 3), (64, 60, 5)])
@pytest.mark.parametrize("text_len", [0, 37])
def test_gather_rope_small_full_compare(D, rope_dim, heads, text_len):
    grid = (5, 9, 16, 2, 6, 6)
    for method in (wa.REGULAR, wa.SHIFTED):
        p = wa.plan(*grid, method, device=DEV)
        loc = wa.local_positions(p, device=DEV)
        tab = wa.rope_table(p, text_len, rope_dim, device=DEV)
        x = normal((2, p.num_tokens, heads, D), 70 + D + heads, device=DEV)
        y = wa.gather_rope(x, p, loc, tab, rope_dim)
        op = _oplan(*grid, method)
        rows = to_f64(x)[:, np.asarray(op.perm)]
        worst = _assert_rotated(y, rows, orope.window_local_positions(op, text_len), rope_dim)
        say(f"rope gather D={D} rope_dim={rope_dim} text_len={text_len} method={method}: worst err/bound {worst:.3f}")


def test_transition_rope_equals_direct_gather_and_full_size_sampled():
    """21x45x80, 24 heads x 128: R -> S transition of un-rotated rows with the
    shifted layout's rotation equals the rotated gather into S, bit for bit;
    sampled rows against the oracle."""
    T, H, W, nt, nh, nw = 21, 45, 80, 4, 3, 3
    pr = wa.plan(T, H, W, nt, nh, nw, wa.REGULAR, device=DEV)
    ps = wa.plan(T, H, W, nt, nh, nw, wa.SHIFTED, device=DEV)
    rope_dim, text_len = 126, 58
    loc_s = wa.local_positions(ps, device=DEV)
    tab = wa.rope_table(ps, text_len, rope_dim, device=DEV)
    q = normal((1, pr.num_tokens, 24, 128), 4711, device=DEV)
    q_r = wa.gather(q, pr.perm)                                   # un-rotated, regular window order
    via_transition = wa.transition_rope(q_r, pr, ps, loc_s, tab, rope_dim)
    direct = wa.gather_rope(q, ps, loc_s, tab, rope_dim)
    torch.cuda.synchronize()
    assert torch.equal(via_transition, direct)
    os_ = _oplan(T, H, W, nt, nh, nw, wa.SHIFTED)
    pos = orope.window_local_positions(os_, text_len)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, pr.num_tokens, 300), [0, pr.num_tokens - 1]]))
    src = to_f64(q[:, torch.as_tensor(np.asarray(os_.perm)[rows], device=DEV)])
    worst = _assert_rotated(direct[:, torch.as_tensor(rows, device=DEV)], src, [pos[j] for j in rows], rope_dim)
    say(f"rope 21x45x80 R->S transition: bit-identical to the direct gather; sampled worst err/bound {worst:.3f}")


def test_rope_permute_empty_and_errors():
    p = wa.plan(5, 9, 16, 2, 6, 6, wa.REGULAR, device=DEV)
    loc = wa.local_positions(p, device=DEV)
    tab = wa.rope_table(p, 0, 128, device=DEV)
    x = normal((1, p.num_tokens, 2, 128), 3, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.gather_rope(x, p, loc, tab, 64)          # 64 / 3 = 21 channels per axis: odd
    with pytest.raises(wa.WinAttnError):
        wa.gather_rope(x, p, loc, tab, 132)         # rope_dim > head_dim
    with pytest.raises(wa.WinAttnError):
        wa.gather_rope(x.float(), p, loc, tab, 128)  # bf16 only
