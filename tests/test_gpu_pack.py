"""Several requests packed into one varlen call (GPU): the packed gather,
attention and scatter give each request exactly the rows it gets alone, match
the oracle, and keep requests isolated (page "vLLM-Omni diffusion runtime",
section 4.2: packed segments are independent documents)."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import pack as opack
from oracle import plan as oplan
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, check_window_head, say
from window_attention_amd.inputs import normal, qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"
HEADS, D = 24, 128
# (T, H, W, nt, nh, nw, method): a 720p clip, the tiny grid, a small shifted grid
REQUESTS = [(4, 45, 80, 4, 3, 3, wa.REGULAR), (5, 9, 16, 2, 3, 3, wa.SHIFTED), (3, 10, 12, 2, 2, 2, wa.SHIFTED)]


def _canonical(r, L):
    return qkv(900 + r, 1, L, HEADS, D, device=DEV)


def _run(qc, kc, vc, perm, cu, max_seqlen):
    qw, kw, vw = (wa.gather(x, perm) for x in (qc, kc, vc))
    o = wa.attn_fwd(qw, kw, vw, cu, max_seqlen)
    return wa.scatter(o, perm), (qw, kw, vw, o)


def _packed_inputs(plans, packed, pad_value):
    """Canonical packed tensors: each request's rows at its offset, its tail
    rows filled with pad_value."""
    out = []
    for t in range(3):
        x = torch.full((1, packed.num_tokens, HEADS, D), pad_value, dtype=torch.bfloat16, device=DEV)
        for r, p in enumerate(plans):
            o = packed.offsets[r]
            x[:, o:o + p.num_tokens] = _canonical(r, p.num_tokens)[t]
        out.append(x)
    return out


@pytest.mark.parametrize("align", [64, 1])
def test_packed_equals_each_request_alone(align):
    plans = [wa.plan(*r, device=DEV) for r in REQUESTS]
    packed = wa.pack(plans, align, device=DEV)
    # the tables are the oracle's, bit for bit
    op = [oplan.plan(*r) for r in REQUESTS]
    want = opack.pack_plans([list(p.perm) for p in op], [list(p.cu_seqlens) for p in op], align)
    assert packed.perm.cpu().tolist() == want.perm and packed.cu_seqlens.cpu().tolist() == want.cu_seqlens
    qp, kp, vp = _packed_inputs(plans, packed, 0.25)
    o_packed, (qw, kw, vw, ow) = _run(qp, kp, vp, packed.perm, packed.cu_seqlens, packed.max_seqlen)
    torch.cuda.synchronize()
    for r, p in enumerate(plans):
        q, k, v = _canonical(r, p.num_tokens)
        o_alone, _ = _run(q, k, v, p.perm, p.cu_seqlens, p.max_seqlen)
        o = packed.offsets[r]
        assert torch.equal(o_packed[:, o:o + p.num_tokens], o_alone), f"request {r}"
    # tail rows are padding attended among themselves: constant rows give the constant back
    for r, p in enumerate(plans):
        a, e = packed.offsets[r] + p.num_tokens, packed.offsets[r + 1]
        if e > a:
            assert torch.all(o_packed[:, a:e] == 0.25)
    # oracle on sampled windows of the packed call (window order), every request
    cu = packed.cu_seqlens.cpu().numpy()
    rng = np.random.default_rng(7 + align)
    nonempty = np.nonzero(np.diff(cu))[0]
    worst = 0.0
    for i in sorted(set(rng.choice(nonempty, size=min(6, len(nonempty)), replace=False).tolist()) | {int(nonempty[-1])}):
        for h in (0, HEADS - 1):
            mx, mean, _, n = check_window_head(qw, kw, vw, ow, None, cu, 0, i, h)
            assert mx <= MAX_ABS and mean <= MEAN_ABS, (i, h, n, mx, mean)
            worst = max(worst, mx)
    say(f"packed call, align {align}: {packed.num_windows} segments, max_seqlen {packed.max_seqlen}, "
        f"worst sampled max-abs {worst:.2e}")


def test_requests_are_isolated():
    plans = [wa.plan(*r, device=DEV) for r in REQUESTS]
    packed = wa.pack(plans, 64, device=DEV)
    qp, kp, vp = _packed_inputs(plans, packed, 0.0)
    o1, _ = _run(qp, kp, vp, packed.perm, packed.cu_seqlens, packed.max_seqlen)
    # replace request 1's rows and tail: requests 0 and 2 are bit-identical
    a, e = packed.offsets[1], packed.offsets[2]
    q2, k2, v2 = (x.clone() for x in (qp, kp, vp))
    for t, x in enumerate((q2, k2, v2)):
        x[:, a:e] = normal((1, e - a, HEADS, D), 4242 + t, device=DEV)
    o2, _ = _run(q2, k2, v2, packed.perm, packed.cu_seqlens, packed.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(o2[:, :a], o1[:, :a]) and torch.equal(o2[:, e:], o1[:, e:])
    assert not torch.equal(o2[:, a:e], o1[:, a:e])
