"""The 21x45x80 video workload compared in full (GPU).

Layers 0 (regular) and 1 (shifted) of the benchmark's R, S, R, S chain, run
exactly as the benchmark runs them (entry gather, fused transition, the same
win_attn_fwd launch): every (window, head) output block and every LSE row is
compared with the fp64 oracle, and the carried Q, K, V of each layer with the
oracle's permutation of the canonical tensors, bit for bit.  Page "Window-
Aligned Sequence Parallelism (SeedVR2)", section "Motivation" (attention only
inside each window)."""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from oracle import plan as oplan
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, lse_bound, method_of, say
from window_attention_amd.inputs import bf16_bits, qkv
from window_attention_amd.workloads import BY_NAME

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKERS = 8          # host threads over (window, head) blocks
BLAS_PER_WORKER = 2  # 16 host threads in all


def _chain_layers(w, q, k, v, upto):
    """The benchmark's chain up to layer `upto`: per layer (layout, carried
    q/k/v, o, lse)."""
    plans = {m: wa.plan_cached(w.T, w.H, w.W, w.nt, w.nh, w.nw, method_of(m), device=DEV) for m in "RS"}
    cur = w.entry
    qw, kw, vw = (wa.gather(x, plans[cur].perm) for x in (q, k, v))
    out = []
    for lay in w.schedule[:upto + 1]:
        if lay != cur:
            qw, kw, vw = (wa.transition(x, plans[cur].inv, plans[lay].perm) for x in (qw, kw, vw))
            cur = lay
        p = plans[lay]
        o, lse = wa.attn_fwd(qw, kw, vw, p.cu_seqlens, p.max_seqlen, return_lse=True)
        out.append((lay, (qw, kw, vw), o, lse))
    return out


@pytest.mark.parametrize("layer", [0, 1])
def test_video_layer_every_window_and_head(layer):
    from threadpoolctl import threadpool_limits
    w = BY_NAME["video_21x45x80"]
    q, k, v = qkv(w.wid, w.batch, w.L, w.heads, w.head_dim, w.sigma, device=DEV)
    lay, (qw, kw, vw), o, lse = _chain_layers(w, q, k, v, layer)[layer]
    op = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method_of(lay))
    # carried tensors: the canonical tensors in the oracle's window order, every row
    perm = torch.as_tensor(np.asarray(op.perm, dtype=np.int64), device=DEV)
    for x_can, x_lay in ((q, qw), (k, kw), (v, vw)):
        assert torch.equal(x_lay, x_can[:, perm])
    torch.cuda.synchronize()
    say(f"layer {layer} ({lay}): {op.num_windows} windows x {w.heads} heads, oracle on the host")
    hq, hk, hv, ho = (bf16_bits(x)[0] for x in (qw, kw, vw, o))  # [L, heads, D] uint16
    hl = lse[0].double().cpu().numpy()                             # [heads, L]
    cu = [int(c) for c in op.cu_seqlens]
    scale = 1.0 / math.sqrt(w.head_dim)

    def block(job):
        i, h = job
        a, e = cu[i], cu[i + 1]
        qh, kh, vh, oh = (oatt.bf16_bits_to_float64(x[a:e, h]) for x in (hq, hk, hv, ho))
        ref_o, ref_lse = oatt.head_attention(qh, kh, vh, scale)
        err = np.abs(oh - ref_o)
        lratio = np.abs(hl[h, a:e] - ref_lse) / lse_bound(qh, kh, scale)
        return float(err.max()), float(err.sum()), err.size, float(lratio.max()), float(np.abs(hl[h, a:e] -
                                                                                             ref_lse).max())

    jobs = [(i, h) for i in range(op.num_windows) for h in range(w.heads) if cu[i + 1] > cu[i]]
    with threadpool_limits(limits=BLAS_PER_WORKER), ThreadPoolExecutor(max_workers=WORKERS) as ex:
        res = list(ex.map(block, jobs))
    mx = max(r[0] for r in res)
    mean = sum(r[1] for r in res) / sum(r[2] for r in res)
    lr = max(r[3] for r in res)
    le = max(r[4] for r in res)
    say(f"layer {layer} ({lay}): {len(jobs)} blocks, {sum(r[2] for r in res)} outputs: max abs {mx:.3e}, "
        f"mean abs {mean:.3e}, LSE max abs {le:.3e} (worst ratio to its bound {lr:.3f})")
    worst = max(range(len(res)), key=lambda t: res[t][0])
    assert mx <= MAX_ABS, ("max abs", jobs[worst], mx)
    assert mean <= MEAN_ABS, ("mean abs", mean)
    assert lr <= 1.0, ("lse", jobs[max(range(len(res)), key=lambda t: res[t][3])], lr)
