"""win_attn_fwd_text_noalloc (GPU): the text-augmented attention with its
per-window text outputs in the library's static device scratch, for callers
that cannot allocate.  Its outputs must equal win_attn_fwd_text's (same
kernels, the same arithmetic) bit for bit, on two calls in a row with the
second one smaller, so that the scratch keeps the first call's contents when
the second one runs; sizes past the scratch are refused before anything is
enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import window_attention_amd as wa
from tests.gpu_helpers import say
from window_attention_amd.inputs import normal

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_BYTES = 64 << 20


def _case(lengths, T, Hh, D, B, seed):
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=DEV)
    L = int(sum(lengths))
    q, k, v = (normal((B, L, Hh, D), seed + t, device=DEV) for t in range(3))
    tq, tk, tv = (normal((B, T, Hh, D), seed + 10 + t, device=DEV) for t in range(3))
    return q, k, v, cu, max(lengths), tq, tk, tv


def _both(case):
    q, k, v, cu, mx, tq, tk, tv = case
    B, L, Hh, _ = q.shape
    o1, t1, l1 = wa.attn_fwd_text(q, k, v, cu, mx, tq, tk, tv, return_lse=True)
    o2, t2 = torch.full_like(q, 9.0), torch.full_like(tq, 9.0)
    l2 = torch.full((B, Hh, L), 9.0, dtype=torch.float32, device=DEV)
    wa.attn_fwd_text_noalloc(q, k, v, cu, mx, tq, tk, tv, out=o2, text_out=t2, lse=l2)
    torch.cuda.synchronize()
    return (o1, t1, l1), (o2, t2, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_noalloc_equals_workspace_call_twice_second_smaller(D):
    first = _case([700, 0, 129, 64, 1], 200, 3, D, 2, 900)   # 2 * 5 * 200 * 3 * D * 4 bytes of scratch
    second = _case([65, 3], 17, 2, D, 1, 950)                # smaller: the scratch holds the first call's data
    for name, case in (("first", first), ("second", second)):
        say(f"noalloc D={D} {name} call")
        (o1, t1, l1), (o2, t2, l2) = _both(case)
        assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(l1, l2), name


def test_noalloc_near_the_scratch_limit_and_refused_past_it():
    """The largest text a 24 x 128 call on 8 windows can take (682 rows:
    8 * 682 * 24 * 128 * 4 bytes fit the 64 MiB, 683 do not), then one row
    more is refused with WIN_ESCRATCH and the outputs stay untouched."""
    Hh, D, N = 24, 128, 8
    T = SCRATCH_BYTES // (4 * N * Hh * D)
    lengths = [300, 5, 64, 128, 200, 1, 90, 450]
    case = _case(lengths, T, Hh, D, 1, 960)
    (o1, t1, l1), (o2, t2, l2) = _both(case)
    assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(l1, l2)
    q, k, v, cu, mx, _, _, _ = case
    tq, tk, tv = (normal((1, T + 1, Hh, D), 970 + t, device=DEV) for t in range(3))
    o, to = torch.full_like(q, 5.0), torch.full_like(tq, 5.0)
    with pytest.raises(wa.WinAttnError) as e:
        wa.attn_fwd_text_noalloc(q, k, v, cu, mx, tq, tk, tv, out=o, text_out=to)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.all(o == 5.0) and torch.all(to == 5.0)


def test_noalloc_without_text_is_the_plain_call():
    q, k, v, cu, mx, tq, tk, tv = _case([130, 64], 4, 2, 128, 1, 980)
    lib = wa.load_library()
    o = torch.empty_like(q)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.win_attn_fwd_text_noalloc(p(q), p(k), p(v), p(o), None, p(cu), 2, mx, q.shape[1], 1, 2, 128,
                                       ctypes.c_float(0.0), None, None, None, 0, None, s)
    assert rc == 0
    assert torch.equal(o, wa.attn_fwd(q, k, v, cu, mx))
