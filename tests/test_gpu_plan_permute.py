"""Device planner and permutes against the oracle, bit for bit (GPU)."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import permute as operm
from oracle import plan as oplan
from tests.gpu_helpers import say
from window_attention_amd.inputs import bf16_bits, normal
from window_attention_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
@pytest.mark.parametrize("method", [0, 1])
def test_device_plan_matches_oracle(w, method):
    say(f"device plan {w.name} method={method}")
    o = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method)
    p = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method, device=DEV)
    torch.cuda.synchronize()
    assert (p.wt, p.wh, p.ww, p.num_windows, p.max_seqlen) == (o.wt, o.wh, o.ww, o.num_windows, o.max_seqlen)
    assert np.array_equal(p.perm.cpu().numpy(), np.asarray(o.perm, dtype=np.int32))
    assert np.array_equal(p.inv.cpu().numpy(), np.asarray(o.inv, dtype=np.int32))
    assert np.array_equal(p.cu_seqlens.cpu().numpy(), np.asarray(o.cu_seqlens, dtype=np.int32))
    assert np.array_equal(p.boxes.cpu().numpy(), np.asarray(o.boxes, dtype=np.int32).reshape(-1, 6))


@pytest.mark.parametrize("grid", [(1, 3, 4, 1, 26, 35), (3, 5, 7, 2, 17, 9), (7, 4, 13, 3, 33, 9),
                                  (31, 3, 2, 4, 65, 129)])
@pytest.mark.parametrize("method", [0, 1])
def test_device_plan_small_ragged_grids(grid, method):
    o = oplan.plan(*grid, method)
    p = wa.plan(*grid, method, device=DEV)
    assert np.array_equal(p.perm.cpu().numpy(), np.asarray(o.perm, dtype=np.int32))
    assert np.array_equal(p.cu_seqlens.cpu().numpy(), np.asarray(o.cu_seqlens, dtype=np.int32))


def _host(x):
    if x.dtype == torch.bfloat16:
        return bf16_bits(x)
    return x.cpu().numpy()


@pytest.mark.parametrize("wi", [0, 1, 2])
def test_permutes_full_compare(wi):
    w = WORKLOADS[wi]
    say(f"permutes full compare {w.name}")
    dtype = torch.float32 if w.input_dtype == "fp32" else torch.bfloat16
    x = normal((w.batch, w.L, w.heads, w.head_dim), 77 + wi, device=DEV, dtype=dtype)
    xh = _host(x)
    r = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0)
    s = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 1)
    pr = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0, device=DEV)
    ps = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 1, device=DEV)
    xr = wa.gather(x, pr.perm)
    xs = wa.gather(x, ps.perm)
    ref_r, ref_s = operm.gather(xh, r.perm), operm.gather(xh, s.perm)
    assert np.array_equal(_host(xr), ref_r)
    assert np.array_equal(_host(xs), ref_s)
    assert np.array_equal(_host(wa.scatter(xr, pr.perm)), xh)
    assert np.array_equal(_host(wa.transition(xr, pr.inv, ps.perm)), operm.transition(ref_r, r.perm, s.perm))
    assert np.array_equal(_host(wa.transition(xs, ps.inv, pr.perm)), ref_r)


@pytest.mark.parametrize("wi", [3, 4])
def test_permutes_full_size(wi):
    """Full-size grids, every row: the gathers, the transitions and the
    scatter against the canonical tensor indexed with the oracle's tables
    (the oracle's gather is that indexing)."""
    w = WORKLOADS[wi]
    say(f"permutes full size {w.name}")
    x = normal((w.batch, w.L, w.heads, w.head_dim), 99 + wi, device=DEV)
    r = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0)
    s = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 1)
    pr = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 0, device=DEV)
    ps = wa.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, 1, device=DEV)
    perm_r = torch.as_tensor(np.asarray(r.perm, dtype=np.int64), device=DEV)
    perm_s = torch.as_tensor(np.asarray(s.perm, dtype=np.int64), device=DEV)
    xr = wa.gather(x, pr.perm)
    assert torch.equal(xr, x[:, perm_r])
    xs = wa.gather(x, ps.perm)
    assert torch.equal(xs, x[:, perm_s])
    assert torch.equal(wa.transition(xr, pr.inv, ps.perm), xs)
    assert torch.equal(wa.transition(xs, ps.inv, pr.perm), xr)
    assert torch.equal(wa.scatter(xs, ps.perm), x)
    assert torch.equal(wa.scatter(xr, pr.perm), x)


@pytest.mark.parametrize("row_bytes", [16, 48, 128, 6144, 16 * 1000, 16 * 1537])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_row_sizes(row_bytes, dtype):
    esz = 2 if dtype == torch.bfloat16 else 4
    if row_bytes % esz:
        pytest.skip("row not a whole number of elements")
    L, B = 523, 2
    x = torch.randint(-2 ** 15, 2 ** 15, (B, L, row_bytes // 2), dtype=torch.int16, device=DEV).view(dtype)
    xh = x.view(torch.int16).cpu().numpy()
    perm = torch.randperm(L, device=DEV, dtype=torch.int64).to(torch.int32)
    perm_h = perm.cpu().numpy()
    g = wa.gather(x, perm)
    assert np.array_equal(g.view(torch.int16).cpu().numpy(), operm.gather(xh, perm_h))
    assert np.array_equal(wa.scatter(g, perm).view(torch.int16).cpu().numpy(), xh)
    perm2 = torch.randperm(L, device=DEV, dtype=torch.int64).to(torch.int32)
    inv = torch.as_tensor(np.argsort(perm_h).astype(np.int32), device=DEV)
    t = wa.transition(g, inv, perm2)
    assert np.array_equal(t.view(torch.int16).cpu().numpy(), operm.transition(operm.gather(xh, perm_h), perm_h,
                                                                              perm2.cpu().numpy()))


def test_permute_empty_and_errors():
    x = torch.zeros((1, 0, 64), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(0, dtype=torch.int32, device=DEV)
    assert wa.gather(x, idx).shape == x.shape
    y = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wa.WinAttnError):
        wa.gather(y, torch.zeros(7, dtype=torch.int32, device=DEV))
    with pytest.raises(wa.WinAttnError):
        wa.gather(y, torch.arange(8, dtype=torch.int32, device=DEV), out=y)
