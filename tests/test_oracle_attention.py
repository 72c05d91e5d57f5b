"""Oracle window attention against its pins (CPU only)."""
import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import permute as operm
from oracle import plan as oplan
from tests import oracle_pins as pins


def _window_of_canonical(p):
    """Window index of every canonical token."""
    win = np.empty(len(p.perm), dtype=np.int64)
    for i in range(p.num_windows):
        win[np.asarray(p.perm[p.cu_seqlens[i]:p.cu_seqlens[i + 1]])] = i
    return win


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


CASES = [
    # (T, H, W, nt, nh, nw, heads, D)
    (5, 9, 16, 2, 3, 3, 1, 64),      # the tiny clip workload
    (1, 3, 4, 1, 26, 35, 2, 8),      # ragged 2x2 windows
    (3, 5, 7, 2, 17, 9, 2, 16),
    (4, 6, 6, 3, 9, 9, 3, 32),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("method", [oplan.REGULAR, oplan.SHIFTED])
def test_matches_masked_full_attention(case, method):
    T, H, W, nt, nh, nw, Hh, D = case
    p = oplan.plan(T, H, W, nt, nh, nw, method)
    L = T * H * W
    qc, kc, vc = (_rand((2, L, Hh, D), s) for s in (1, 2, 3))
    scale = 1.0 / math.sqrt(D)
    # oracle: gather into window order, attend per window, scatter back
    ow, lw = oatt.window_attention(operm.gather(qc, p.perm), operm.gather(kc, p.perm), operm.gather(vc, p.perm),
                                   p.cu_seqlens)
    o = operm.scatter(ow, p.perm)
    lse = lw[:, :, p.inv]
    win = _window_of_canonical(p)
    # twin 1: brute-force masked attention over canonical order
    ob, lb = oatt.masked_full_attention(qc, kc, vc, win, scale)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12
    # twin 2: torch scaled_dot_product_attention with a boolean mask (fp64, CPU)
    ot, lt = pins.torch_sdpa_masked(qc, kc, vc, win, scale)
    assert np.max(np.abs(o - ot)) < 1e-12
    assert np.max(np.abs(lse - lt)) < 1e-12


def test_zero_query_gives_window_mean():
    p = oplan.plan(3, 5, 7, 2, 17, 9, oplan.SHIFTED)
    L = 3 * 5 * 7
    q = np.zeros((1, L, 2, 16))
    k = _rand((1, L, 2, 16), 5)
    v = _rand((1, L, 2, 16), 6)
    o, lse = oatt.window_attention(q, k, v, p.cu_seqlens)
    for i in range(p.num_windows):
        a, e = p.cu_seqlens[i], p.cu_seqlens[i + 1]
        assert np.allclose(o[0, a:e], v[0, a:e].mean(axis=0, keepdims=True), atol=1e-13, rtol=0)
        assert np.allclose(lse[0, :, a:e], math.log(e - a), atol=1e-13, rtol=0)


def test_constant_value_is_reproduced():
    cu = [0, 3, 10, 10, 17]
    q, k = _rand((1, 17, 1, 8), 7), _rand((1, 17, 1, 8), 8)
    v = np.empty((1, 17, 1, 8))
    for i in range(4):
        v[0, cu[i]:cu[i + 1]] = float(i) - 1.5
    o, _ = oatt.window_attention(q, k, v, cu)
    assert np.allclose(o, v, atol=1e-14, rtol=0)


def test_single_token_windows_copy_value():
    L = 6
    q, k, v = (_rand((1, L, 3, 4), s) for s in (9, 10, 11))
    o, lse = oatt.window_attention(q, k, v, list(range(L + 1)))
    assert np.allclose(o, v, atol=0, rtol=0)
    s = np.einsum("blhd,blhd->bhl", q, k) / 2.0
    assert np.allclose(lse, s, atol=1e-14, rtol=0)


def test_permutation_inside_window_permutes_output():
    cu = [0, 9, 20]
    q, k, v = (_rand((1, 20, 2, 8), s) for s in (12, 13, 14))
    o, _ = oatt.window_attention(q, k, v, cu)
    rng = np.random.default_rng(15)
    perm = np.concatenate([rng.permutation(9), 9 + rng.permutation(11)])
    o2, _ = oatt.window_attention(q[:, perm], k[:, perm], v[:, perm], cu)
    assert np.allclose(o2, o[:, perm], atol=1e-13, rtol=0)


def test_windows_are_isolated():
    # change every token of one window; no other window's output may change
    cu = [0, 5, 12, 12, 20]
    q, k, v = (_rand((1, 20, 2, 8), s) for s in (16, 17, 18))
    o, _ = oatt.window_attention(q, k, v, cu)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, 5:12] += 3.0
    o2, _ = oatt.window_attention(q2, k2, v2, cu)
    assert np.array_equal(o2[:, :5], o[:, :5]) and np.array_equal(o2[:, 12:], o[:, 12:])
    assert not np.allclose(o2[:, 5:12], o[:, 5:12])


def test_bf16_decode_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x3C00], dtype=np.uint16)
    vals = oatt.bf16_bits_to_float64(bits)
    assert vals[0] == 0.0 and vals[1] == 1.0 and vals[2] == -1.0
    assert vals[3] == 3.140625
    assert vals[4] == np.inf and vals[5] == -np.inf
    assert vals[6] == 2.0 ** -133
    assert vals[7] == 2.0 ** -7


def test_flops_count_closed_form():
    # 720p reference grid, regular layout: windows of 2430, 2340, 1215, 1170
    # tokens (full, w-edge, t-edge, both), counted 9, 3, 18, 6 ... per layout
    p = oplan.plan(21, 45, 80, 4, 3, 3, oplan.REGULAR)
    sizes = sorted(p.cu_seqlens[i + 1] - p.cu_seqlens[i] for i in range(p.num_windows))
    assert sizes.count(2430) == 3 * 2 * 3 and sizes.count(2340) == 3 * 3
    assert sizes.count(1215) == 2 * 3 and sizes.count(1170) == 3
    want = 4 * 128 * 24 * (18 * 2430 ** 2 + 9 * 2340 ** 2 + 6 * 1215 ** 2 + 3 * 1170 ** 2)
    assert oatt.attention_flops(p.cu_seqlens, 1, 24, 128) == want
