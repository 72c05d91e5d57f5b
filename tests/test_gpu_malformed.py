"""Malformed device tables stay inside the tensors (GPU).

include/winattn.h promises that out-of-range permute indices are clamped
into [0, L), and that cu_seqlens entries breaking the rules (decreasing, past
L, windows longer than max_seqlen) are clamped so that no access leaves the
tensors.  Each tensor here is a slice of a larger buffer: the input guard rows
hold NaN (a read of them would poison an output) and the output guard rows a
sentinel (a write to them would change it).  Rows whose result the header
leaves unspecified are only checked for being finite; well-formed rows are
checked against their definition."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, say, to_f64
from window_attention_amd.inputs import normal

pytestmark = pytest.mark.gpu
DEV = "cuda"
G = 64  # guard rows on each side


def _guarded(x, fill):
    """x [1, L, ...] copied into the middle of a [1, L + 2G, ...] buffer whose
    guard rows hold `fill`; returns (view of the middle, whole buffer)."""
    big = torch.full((1, x.shape[1] + 2 * G, *x.shape[2:]), fill, dtype=x.dtype, device=x.device)
    big[:, G:G + x.shape[1]] = x
    return big[:, G:G + x.shape[1]], big


def _guards_hold(big, L, value):
    g = torch.cat([big[:, :G], big[:, G + L:]], dim=1).float()
    return bool(torch.all(g == value)) if not np.isnan(value) else bool(torch.all(torch.isnan(g)))


def test_permutes_clamp_out_of_range_indices():
    say("malformed permute indices")
    L, heads, D = 100, 3, 8
    src, src_big = _guarded(normal((1, L, heads, D), 900, device=DEV), float("nan"))
    rng = np.random.default_rng(3)
    idx = rng.integers(-40, L + 40, size=L).astype(np.int32)
    idx_d = torch.as_tensor(idx, device=DEV)
    clamped = np.clip(idx, 0, L - 1)
    s = src.float().cpu().numpy()

    out, out_big = _guarded(torch.zeros((1, L, heads, D), dtype=torch.bfloat16, device=DEV), 7.0)
    wa.gather(src, idx_d, out=out)
    torch.cuda.synchronize()
    assert _guards_hold(out_big, L, 7.0)
    assert np.array_equal(out.float().cpu().numpy(), s[:, clamped])

    perm = rng.integers(-10, L + 10, size=L).astype(np.int32)
    out.zero_()
    wa.transition(src, idx_d, torch.as_tensor(perm, device=DEV), out=out)
    torch.cuda.synchronize()
    assert _guards_hold(out_big, L, 7.0)
    assert np.array_equal(out.float().cpu().numpy(), s[:, clamped[np.clip(perm, 0, L - 1)]])

    # scatter: rows no index reaches keep their value, a row one index
    # reaches is that source row, and where clamped targets collide (the
    # header leaves those rows unspecified: the racing copies interleave) every
    # 16-byte chunk is still that chunk of one of the colliding sources
    out.fill_(5.0)
    wa.scatter(src, idx_d, out=out)
    torch.cuda.synchronize()
    assert _guards_hold(out_big, L, 7.0)
    got = out.float().cpu().numpy().reshape(L, -1, 8)   # [row, 16-byte chunk, 8 bf16]
    srcs = s.reshape(L, -1, 8)
    for row in range(L):
        sources = np.nonzero(clamped == row)[0]
        if len(sources) == 0:
            assert np.all(got[row] == 5.0), row
        elif len(sources) == 1:
            assert np.array_equal(got[row], srcs[sources[0]]), row
        else:
            for c in range(got.shape[1]):
                assert any(np.array_equal(got[row, c], srcs[j, c]) for j in sources), (row, c)


@pytest.mark.parametrize("D", [64, 128])
def test_attention_malformed_cu_seqlens_stays_inside(D):
    say(f"malformed cu_seqlens D={D}")
    L, heads = 300, 2
    q, q_big = _guarded(normal((1, L, heads, D), 910, device=DEV), float("nan"))
    k, k_big = _guarded(normal((1, L, heads, D), 911, device=DEV), float("nan"))
    v, v_big = _guarded(normal((1, L, heads, D), 912, device=DEV), float("nan"))
    out, out_big = _guarded(torch.zeros((1, L, heads, D), dtype=torch.bfloat16, device=DEV), 7.0)
    # windows: [0,100) well formed; a decreasing entry (empty); [80,260) overlapping
    # the first and longer than max_seqlen; [260, 300) cut at L; a window past L
    cu = torch.tensor([0, 100, 80, 260, 400, 250], dtype=torch.int32, device=DEV)
    # the LSE [1, heads, L] in the middle of a guarded flat buffer
    lse_big = torch.full((heads * L + 2 * G,), 3.0, dtype=torch.float32, device=DEV)
    lse = lse_big[G:G + heads * L].view(1, heads, L)
    lib = wa.load_library()
    st = wa._stream(q)
    assert lib.win_attn_fwd(wa._ptr(q), wa._ptr(k), wa._ptr(v), wa._ptr(out), wa._ptr(lse), wa._ptr(cu), 5, 128, L,
                            1, heads, D, float(D) ** -0.5, st) == 0
    torch.cuda.synchronize()
    assert bool(torch.all(lse_big[:G] == 3.0)) and bool(torch.all(lse_big[G + heads * L:] == 3.0))
    assert _guards_hold(out_big, L, 7.0)
    for big in (q_big, k_big, v_big):
        assert _guards_hold(big, L, float("nan"))  # inputs are not written
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o)), "a guard row (NaN) was read"
    assert np.all(np.isfinite(lse.cpu().numpy()))
    qh, kh, vh = (to_f64(x) for x in (q, k, v))
    for a, e, rows in ((0, 100, range(0, 80)), (260, 300, range(260, 300))):
        ref, _ = oatt.window_attention(qh[:, a:e], kh[:, a:e], vh[:, a:e], [0, e - a])
        got = o[:, list(rows)]
        err = np.abs(got - ref[:, [r - a for r in rows]])
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (a, e, err.max())
