"""The hot path inside a captured HIP graph (GPU).

No entry point allocates, synchronizes or sets memory from the host, so a
whole step (gather of Q, K, V, attention, transition to the shifted layout,
scatter) can be captured once and replayed.  Each replay is checked against
the same step run eagerly into separate buffers, with eager work and input
changes between the replays."""
import pytest
import torch

import window_attention_amd as wa
from tests.gpu_helpers import say
from window_attention_amd.inputs import qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _buffers(q):
    e = torch.empty_like
    return {"qw": e(q), "kw": e(q), "vw": e(q), "ow": e(q), "os": e(q), "out": e(q)}


def _step(q, k, v, p, ps, b):
    for x, name in ((q, "qw"), (k, "kw"), (v, "vw")):
        wa.gather(x, p.perm, out=b[name])
    wa.attn_fwd(b["qw"], b["kw"], b["vw"], p.cu_seqlens, p.max_seqlen, out=b["ow"])
    wa.transition(b["ow"], p.inv, ps.perm, out=b["os"])
    wa.scatter(b["os"], ps.perm, out=b["out"])


def test_step_replays_from_a_graph():
    say("graph capture of one step")
    L, heads, D = 4 * 45 * 80, 4, 128
    q, k, v = qkv(8, 1, L, heads, D, device=DEV)
    p = wa.plan(4, 45, 80, 4, 3, 3, wa.REGULAR, device=DEV)
    ps = wa.plan(4, 45, 80, 4, 3, 3, wa.SHIFTED, device=DEV)
    graph_bufs, eager_bufs = _buffers(q), _buffers(q)

    side = torch.cuda.Stream(device=DEV)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(q, k, v, p, ps, graph_bufs)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(q, k, v, p, ps, graph_bufs)

    for replay in range(3):
        graph_bufs["out"].fill_(7.0)
        if replay:
            # new inputs in the captured tensors (eager work between replays)
            q.mul_(-0.5)
            v.add_(0.25)
        _step(q, k, v, p, ps, eager_bufs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graph_bufs["out"], eager_bufs["out"]), f"replay {replay}"
        assert torch.equal(graph_bufs["ow"], eager_bufs["ow"]), f"replay {replay}"


def test_text_and_rope_calls_replay_from_a_graph():
    """The RoPE gather into the shifted layout and the text-augmented call
    (its per-window workspace passed in) captured together and replayed."""
    say("graph capture of the rope gather and the text call")
    L, heads, D, T = 4 * 45 * 80, 2, 128, 40
    q, k, v = qkv(9, 1, L, heads, D, device=DEV)
    tq, tk, tv = qkv(10, 1, T, heads, D, device=DEV)
    ps = wa.plan(4, 45, 80, 4, 3, 3, wa.SHIFTED, device=DEV)
    loc = wa.local_positions(ps, device=DEV)
    tab = wa.rope_table(ps, T, 126, device=DEV)

    def bufs():
        e = torch.empty_like
        return {"qr": e(q), "kr": e(q), "vw": e(q), "o": e(q), "to": e(tq),
                "ws": torch.empty((1, ps.num_windows, T, heads, D), dtype=torch.float32, device=DEV)}

    def step(b):
        wa.gather_rope(q, ps, loc, tab, 126, out=b["qr"])
        wa.gather_rope(k, ps, loc, tab, 126, out=b["kr"])
        wa.gather(v, ps.perm, out=b["vw"])
        wa.attn_fwd_text(b["qr"], b["kr"], b["vw"], ps.cu_seqlens, ps.max_seqlen, tq, tk, tv, out=b["o"],
                         text_out=b["to"], workspace=b["ws"])

    gb, eb = bufs(), bufs()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for replay in range(3):
        gb["o"].fill_(7.0)
        gb["to"].fill_(7.0)
        if replay:
            k.mul_(-1.0)
            tv.add_(0.5)
        step(eb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("qr", "kr", "o", "to", "ws"):
            assert torch.equal(gb[name], eb[name]), (name, replay)
