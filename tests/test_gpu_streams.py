"""Stream ordering of the boundary (GPU).

Every entry point enqueues on the stream it is given, and the binding passes
torch's current stream.  Here the whole path (device plan, gather, attention,
transition, scatter) is issued under a side stream whose queue starts with a
spin kernel: while the spin holds the side stream, the outputs must still hold
their sentinel (nothing ran on another stream), and once the side stream
drains they must equal the same path run on the default stream."""
import pytest
import torch

import window_attention_amd as wa
from tests.gpu_helpers import say
from window_attention_amd.inputs import qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"
SPIN_CYCLES = 50_000_000  # tens of milliseconds whichever clock the spin counts


def _path(q, k, v, out):
    p = wa.plan(4, 45, 80, 4, 3, 3, wa.REGULAR, device=DEV)
    ps = wa.plan(4, 45, 80, 4, 3, 3, wa.SHIFTED, device=DEV)
    qw, kw, vw = (wa.gather(x, p.perm) for x in (q, k, v))
    ow = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen)
    os_ = wa.transition(ow, p.inv, ps.perm)
    wa.scatter(os_, ps.perm, out=out)


def test_path_runs_on_the_callers_stream():
    say("side-stream ordering")
    L, heads, D = 4 * 45 * 80, 4, 128
    q, k, v = qkv(7, 1, L, heads, D, device=DEV)
    ref = torch.empty_like(q)
    _path(q, k, v, ref)
    torch.cuda.synchronize()

    out = torch.full_like(q, 3.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)  # default priority
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)
        _path(q, k, v, out)
    # the default stream sees the sentinel while the side stream still spins
    early = out[0, :64].clone()
    torch.cuda.current_stream().synchronize()
    assert not side.query(), "the spin ended before the check: raise SPIN_CYCLES"
    assert torch.all(early == 3.0)
    side.synchronize()
    assert torch.equal(out, ref)
