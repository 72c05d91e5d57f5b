"""MI355X (gfx950) 3D window attention: Python binding of ``libwinattn.so``.

Argument marshalling only: every step runs in the library's HIP kernels (or,
for ``plan(..., device=None)``, its host planner).  PyTorch supplies device
memory and the current stream.  The C entry points are documented in
``include/winattn.h``; their names are kept here:

    plan()        -> win_plan
    gather()      -> win_permute(mode=WIN_GATHER)
    scatter()     -> win_permute(mode=WIN_SCATTER)
    transition()  -> win_transition
    attn_fwd()    -> win_attn_fwd
    attn_fwd_text() -> win_attn_fwd_text
    attn_fwd_text_noalloc() -> win_attn_fwd_text_noalloc
    pack()        -> win_pack
    lpt()         -> win_lpt
    local_positions() -> win_plan_local
    rope_table()      -> win_rope_table
    gather_rope(), transition_rope() -> win_permute_rope
    plan_a()      -> win_plan_a

If the library has not been built the first call raises ``WinAttnError``;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from collections import OrderedDict
from dataclasses import dataclass

__all__ = ["WinAttnError", "Plan", "Packed", "Assignment", "Redistribution", "plan", "plan_cached", "pack", "lpt",
           "plan_a", "local_positions", "rope_table", "gather_rope", "transition_rope", "gather", "scatter",
           "transition", "attn_fwd", "attn_fwd_text", "attn_fwd_text_noalloc", "build_info", "REGULAR", "SHIFTED", "LIB_PATH"]

REGULAR = 0
SHIFTED = 1
_DTYPES = {}  # torch dtype -> WIN_DTYPE_*, filled lazily
_GATHER, _SCATTER = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwinattn.so")
_lib = None


class WinAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = what
        if _lib is not None and code < 0:
            msg = f"{what}: {_lib.win_strerror(code).decode()} (status {code})"
        super().__init__(msg)


class _PlanInfo(ctypes.Structure):
    _fields_ = [("wt", ctypes.c_int32), ("wh", ctypes.c_int32), ("ww", ctypes.c_int32),
                ("segs_t", ctypes.c_int32), ("segs_h", ctypes.c_int32), ("segs_w", ctypes.c_int32),
                ("num_windows", ctypes.c_int32), ("max_seqlen", ctypes.c_int32), ("num_tokens", ctypes.c_int64)]


def load_library():
    """Load ``libwinattn.so`` (built in-tree by ``window_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise WinAttnError(-4, f"{LIB_PATH} is missing: build it with 'python -m window_attention_amd.build'")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.win_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(_PlanInfo), vp, vp, vp, vp, i32, vp]
    lib.win_plan.restype = ctypes.c_int
    lib.win_permute.argtypes = [vp, vp, vp, i64, i32, i64, i32, i32, vp]
    lib.win_permute.restype = ctypes.c_int
    lib.win_transition.argtypes = [vp, vp, vp, vp, i64, i32, i64, i32, vp]
    lib.win_transition.restype = ctypes.c_int
    lib.win_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp]
    lib.win_attn_fwd.restype = ctypes.c_int
    lib.win_pack.argtypes = [i32, vp, vp, vp, vp, i32, vp, vp, vp, ctypes.POINTER(i32)]
    lib.win_pack.restype = ctypes.c_int
    lib.win_lpt.argtypes = [i32, vp, i32, vp, vp, vp, vp]
    lib.win_lpt.restype = ctypes.c_int
    lib.win_plan_a.argtypes = [i64, i32, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.win_plan_a.restype = ctypes.c_int
    lib.win_plan_local.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, i32, vp]
    lib.win_plan_local.restype = ctypes.c_int
    lib.win_rope_table.argtypes = [i32, i32, i32, i32, i32, ctypes.c_double, vp]
    lib.win_rope_table.restype = ctypes.c_int
    lib.win_permute_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, i32, i32, vp]
    lib.win_permute_rope.restype = ctypes.c_int
    lib.win_attn_fwd_text.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp, vp, vp, i32,
                                      vp, vp, vp]
    lib.win_attn_fwd_text.restype = ctypes.c_int
    lib.win_attn_fwd_text_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, f32, vp, vp, vp,
                                              i32, vp, vp]
    lib.win_attn_fwd_text_noalloc.restype = ctypes.c_int
    lib.win_strerror.argtypes = [ctypes.c_int]
    lib.win_strerror.restype = ctypes.c_char_p
    lib.win_build_info.argtypes = []
    lib.win_build_info.restype = ctypes.c_char_p
    _lib = lib
    return lib


def build_info() -> str:
    return load_library().win_build_info().decode()


def _check(status: int, what: str):
    if status != 0:
        raise WinAttnError(status, what)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t):
    import torch
    if not _DTYPES:
        _DTYPES.update({torch.bfloat16: 0, torch.float16: 1, torch.float32: 2})
    if t.dtype not in _DTYPES:
        raise WinAttnError(-2, f"dtype {t.dtype} is not supported")
    return _DTYPES[t.dtype]


def _require_cuda(name, t, dtype=None, device=None):
    if not t.is_cuda:
        raise WinAttnError(-1, f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise WinAttnError(-1, f"{name} is on {t.device}, the call runs on {device}")
    if not t.is_contiguous():
        raise WinAttnError(-1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise WinAttnError(-2, f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class Plan:
    """Tables of one window layout (see ``win_plan`` in include/winattn.h)."""
    T: int
    H: int
    W: int
    method: int
    wt: int
    wh: int
    ww: int
    segs: tuple
    num_windows: int
    max_seqlen: int
    num_tokens: int
    perm: object        # torch.int32 [L]
    inv: object         # torch.int32 [L]
    cu_seqlens: object  # torch.int32 [N+1]
    boxes: object       # torch.int32 [N, 6]
    counts: tuple = None  # (nt, nh, nw) it was built with


def plan(T, H, W, nt, nh, nw, method=REGULAR, device=None) -> Plan:
    """Window layout tables.  ``device=None`` fills host (CPU) tensors with the
    host planner; a CUDA device fills device tensors with the device kernel on
    the current stream."""
    import torch
    lib = load_library()
    info = _PlanInfo()
    _check(lib.win_plan(T, H, W, nt, nh, nw, method, ctypes.byref(info), None, None, None, None, 0, None),
           "win_plan(size query)")
    L, N = info.num_tokens, info.num_windows
    dev = torch.device("cpu") if device is None else torch.device(device)
    on_dev = dev.type == "cuda"
    perm = torch.empty(L, dtype=torch.int32, device=dev)
    inv = torch.empty(L, dtype=torch.int32, device=dev)
    cu = torch.empty(N + 1, dtype=torch.int32, device=dev)
    boxes = torch.empty((N, 6), dtype=torch.int32, device=dev)
    stream = _stream(perm) if on_dev else None
    _check(lib.win_plan(T, H, W, nt, nh, nw, method, ctypes.byref(info), _ptr(perm), _ptr(inv), _ptr(cu),
                        _ptr(boxes), 1 if on_dev else 0, stream), "win_plan")
    return Plan(T, H, W, method, info.wt, info.wh, info.ww, (info.segs_t, info.segs_h, info.segs_w),
                N, info.max_seqlen, L, perm, inv, cu, boxes, (nt, nh, nw))


_PLAN_CACHE: "OrderedDict[tuple, Plan]" = OrderedDict()
PLAN_CACHE_SIZE = 32


def plan_cached(T, H, W, nt, nh, nw, method=REGULAR, device=None) -> Plan:
    """``plan`` behind an LRU cache keyed on the grid, the window counts, the
    method and the device (a plan is a pure function of these)."""
    import torch
    dev = str(torch.device("cpu" if device is None else device))  # None means host tables, as "cpu"
    key = (T, H, W, nt, nh, nw, method, dev)
    p = _PLAN_CACHE.get(key)
    if p is not None:
        _PLAN_CACHE.move_to_end(key)
        return p
    p = plan(T, H, W, nt, nh, nw, method, device)
    _PLAN_CACHE[key] = p
    while len(_PLAN_CACHE) > PLAN_CACHE_SIZE:
        _PLAN_CACHE.popitem(last=False)
    return p


@dataclass
class Packed:
    """Several requests' plans as one varlen call (see ``win_pack`` in
    include/winattn.h): request r owns rows ``offsets[r] .. offsets[r+1]-1``
    of the packed token tensor (its rows, then its alignment tail)."""
    offsets: list
    num_tokens: int     # packed rows, tails included
    num_windows: int    # segments of the packed call (windows and tails)
    max_seqlen: int
    perm: object        # torch.int32 [num_tokens]
    cu_seqlens: object  # torch.int32 [num_windows + 1]


def pack(plans, align=64, device=None) -> Packed:
    """Pack ``plans`` (in request order) into one varlen call; tables are
    returned on ``device`` (None: host)."""
    import torch
    lib = load_library()
    R = len(plans)
    if R == 0:
        raise WinAttnError(-1, "pack needs at least one plan")
    toks = (ctypes.c_int64 * R)(*[p.num_tokens for p in plans])
    nwin = (ctypes.c_int32 * R)(*[p.num_windows for p in plans])
    perms = torch.cat([p.perm.cpu() for p in plans]).contiguous()
    cus = torch.cat([p.cu_seqlens.cpu() for p in plans]).contiguous()
    offsets = (ctypes.c_int64 * (R + 1))()
    total_max = sum(p.num_tokens + align for p in plans)
    perm_out = torch.empty(total_max, dtype=torch.int32)
    cu_out = torch.empty(sum(p.num_windows for p in plans) + R + 1, dtype=torch.int32)
    mx = ctypes.c_int32()
    _check(lib.win_pack(R, toks, nwin, _ptr(perms), _ptr(cus), int(align), offsets, _ptr(perm_out), _ptr(cu_out),
                        ctypes.byref(mx)), "win_pack")
    total = offsets[R]
    dev = torch.device("cpu") if device is None else torch.device(device)
    return Packed(list(offsets), total, cu_out.numel() - 1, mx.value, perm_out[:total].to(dev), cu_out.to(dev))


@dataclass
class Assignment:
    """Windows of one layout on `ranks` ranks (see ``win_lpt``)."""
    ranks: int
    owner: object         # torch.int32 [N]: rank of each window
    order: object         # torch.int32 [N]: windows grouped by rank, ascending inside a rank
    rank_offsets: object  # torch.int32 [ranks + 1]
    rank_tokens: object   # torch.int64 [ranks]

    def windows_of(self, r):
        return self.order[int(self.rank_offsets[r]):int(self.rank_offsets[r + 1])].tolist()


def _host_i32(t):
    import torch
    return t.detach().to("cpu", torch.int32).contiguous()


def lpt(plan_or_cu, ranks) -> Assignment:
    """LPT assignment of a plan's windows (or of the windows of a host or
    device ``cu_seqlens``) to ``ranks`` ranks; host tensors out."""
    import torch
    lib = load_library()
    cu = _host_i32(plan_or_cu.cu_seqlens if isinstance(plan_or_cu, Plan) else torch.as_tensor(plan_or_cu))
    N = cu.numel() - 1
    owner = torch.empty(N, dtype=torch.int32)
    order = torch.empty(N, dtype=torch.int32)
    offs = torch.empty(ranks + 1, dtype=torch.int32)
    toks = torch.empty(ranks, dtype=torch.int64)
    _check(lib.win_lpt(N, _ptr(cu), int(ranks), _ptr(owner), _ptr(order), _ptr(offs), _ptr(toks)), "win_lpt")
    return Assignment(int(ranks), owner, order, offs, toks)


@dataclass
class Redistribution:
    """Plan A tables between two (plan, assignment) pairs (see
    ``win_plan_a``); host tensors."""
    counts: object        # torch.int64 [ranks, ranks]
    send_rows: object     # torch.int32 [L]
    recv_pos: object      # torch.int32 [L]
    exchange_required: bool


def plan_a(src: Plan, src_assignment: Assignment, dst: Plan, dst_assignment: Assignment) -> Redistribution:
    import torch
    lib = load_library()
    P = src_assignment.ranks
    if dst_assignment.ranks != P or src.num_tokens != dst.num_tokens:
        raise WinAttnError(-1, "plan_a needs two layouts of one grid on the same number of ranks")
    L = src.num_tokens
    sp, sc, so, sr = (_host_i32(x) for x in (src.perm, src.cu_seqlens, src_assignment.order,
                                             src_assignment.rank_offsets))
    dp, dc, do, dr = (_host_i32(x) for x in (dst.perm, dst.cu_seqlens, dst_assignment.order,
                                             dst_assignment.rank_offsets))
    counts = torch.empty((P, P), dtype=torch.int64)
    send = torch.empty(L, dtype=torch.int32)
    recv = torch.empty(L, dtype=torch.int32)
    ex = ctypes.c_int32()
    _check(lib.win_plan_a(L, P, _ptr(sp), _ptr(sc), src.num_windows, _ptr(so), _ptr(sr), _ptr(dp), _ptr(dc),
                          dst.num_windows, _ptr(do), _ptr(dr), _ptr(counts), _ptr(send), _ptr(recv),
                          ctypes.byref(ex)), "win_plan_a")
    return Redistribution(counts, send, recv, bool(ex.value))


def local_positions(p: Plan, device=None):
    """Window-local (t, h, w) of every row of ``p``'s window order: int32
    [L, 3], filled on the host (device None) or by a device kernel."""
    import torch
    lib = load_library()
    dev = torch.device("cpu") if device is None else torch.device(device)
    out = torch.empty((p.num_tokens, 3), dtype=torch.int32, device=dev)
    on_dev = dev.type == "cuda"
    _check(lib.win_plan_local(p.T, p.H, p.W, *_window_counts(p), p.method, _ptr(out), 1 if on_dev else 0,
                              _stream(out) if on_dev else None), "win_plan_local")
    return out


def _window_counts(p: Plan):
    if getattr(p, "counts", None) is None:
        raise WinAttnError(-1, "this plan does not record its window counts; build it with plan()")
    return p.counts


def rope_table(p: Plan, text_len, rope_dim, base=10000.0, device=None):
    """(cos, sin) table for ``p``'s window extents (see win_rope_table)."""
    import torch
    lib = load_library()
    n = (p.wt + p.wh + p.ww) * (rope_dim // 3)
    t = torch.empty(n, dtype=torch.float32)
    _check(lib.win_rope_table(p.wt, p.wh, p.ww, int(text_len), int(rope_dim), float(base), _ptr(t)), "win_rope_table")
    return t if device is None else t.to(device)


def _permute_rope(src, idx, perm_dst, local, table, p: Plan, rope_dim, out):
    import torch
    lib = load_library()
    if src.dim() != 4:
        raise WinAttnError(-1, "src must be [B, L, heads, head_dim]")
    B, L, Hh, D = src.shape
    # the kernel reads these tables through raw pointers: sizes from another
    # grid, layout or rope_dim would send it past their ends (checked before
    # anything else, so a mismatch is reported whatever the devices)
    if idx.numel() != L or (perm_dst is not None and perm_dst.numel() != L):
        raise WinAttnError(-1, f"index tables must have L={L} entries")
    if local.numel() != 3 * L:
        raise WinAttnError(-1, f"local must have 3*L={3 * L} entries, got {local.numel()}")
    if rope_dim < 6 or rope_dim > D or (rope_dim // 3) % 2:
        raise WinAttnError(-2, f"rope_dim {rope_dim} is not supported for head_dim {D}")
    want = (p.wt + p.wh + p.ww) * (rope_dim // 3)
    if table.numel() != want:
        raise WinAttnError(-1, f"table must hold (wt+wh+ww)*(rope_dim//3)={want} floats, got {table.numel()}")
    _require_cuda("src", src, torch.bfloat16)
    dev = src.device
    for name, t in (("idx", idx), ("local", local)):
        _require_cuda(name, t, torch.int32, dev)
    if perm_dst is not None:
        _require_cuda("perm_dst", perm_dst, torch.int32, dev)
    _require_cuda("table", table, torch.float32, dev)
    if out is None:
        out = torch.empty_like(src)
    _require_cuda("out", out, torch.bfloat16, dev)
    if out.shape != src.shape:
        raise WinAttnError(-1, "out must have the shape of src")
    _check(lib.win_permute_rope(_ptr(src), _ptr(out), _ptr(idx), _ptr(perm_dst), _ptr(local), _ptr(table), p.wt,
                                p.wh, p.ww, L, B, Hh, D, int(rope_dim), _stream(src)), "win_permute_rope")
    return out


def gather_rope(src, p: Plan, local, table, rope_dim, out=None):
    """Canonical -> ``p``'s window order with ``p``'s window-local RoPE:
    ``out[b, j] = rope(src[b, p.perm[j]], local[j])``."""
    return _permute_rope(src, p.perm, None, local, table, p, rope_dim, out)


def transition_rope(src, src_plan: Plan, dst_plan: Plan, local_dst, table, rope_dim, out=None):
    """Un-rotated rows in ``src_plan``'s window order -> ``dst_plan``'s window
    order with ``dst_plan``'s window-local RoPE."""
    return _permute_rope(src, src_plan.inv, dst_plan.perm, local_dst, table, dst_plan, rope_dim, out)


def _rows(x):
    if x.dim() < 2:
        raise WinAttnError(-1, "token tensors are [B, L, ...]")
    B, L = x.shape[0], x.shape[1]
    return B, L, math.prod(x.shape[2:])


def _permute(src, idx, mode, out):
    import torch
    lib = load_library()
    _require_cuda("src", src)
    _require_cuda("idx", idx, torch.int32, src.device)
    B, L, row = _rows(src)
    if idx.numel() != L:
        raise WinAttnError(-1, f"index has {idx.numel()} entries, expected L={L}")
    if out is None:
        out = torch.empty_like(src)
    _require_cuda("out", out, src.dtype, src.device)
    if out.shape != src.shape:
        raise WinAttnError(-1, "out must have the shape of src")
    _check(lib.win_permute(_ptr(src), _ptr(out), _ptr(idx), L, B, row, _dtype_code(src), mode, _stream(src)),
           "win_permute")
    return out


def gather(src, perm, out=None):
    """Canonical -> window order: ``out[b, j] = src[b, perm[j]]``."""
    return _permute(src, perm, _GATHER, out)


def scatter(src, perm, out=None):
    """Window -> canonical order: ``out[b, perm[j]] = src[b, j]``."""
    return _permute(src, perm, _SCATTER, out)


def transition(src, inv_src, perm_dst, out=None):
    """Layout A -> layout B in one pass: ``out[b, j] = src[b, inv_src[perm_dst[j]]]``."""
    import torch
    lib = load_library()
    _require_cuda("src", src)
    _require_cuda("inv_src", inv_src, torch.int32, src.device)
    _require_cuda("perm_dst", perm_dst, torch.int32, src.device)
    B, L, row = _rows(src)
    if inv_src.numel() != L or perm_dst.numel() != L:
        raise WinAttnError(-1, "index tables must have L entries")
    if out is None:
        out = torch.empty_like(src)
    _require_cuda("out", out, src.dtype, src.device)
    if out.shape != src.shape:
        raise WinAttnError(-1, "out must have the shape of src")
    _check(lib.win_transition(_ptr(src), _ptr(out), _ptr(inv_src), _ptr(perm_dst), L, B, row, _dtype_code(src),
                              _stream(src)), "win_transition")
    return out


def attn_fwd(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, out=None, return_lse=False):
    """Window attention over window-ordered bf16 ``[B, L, heads, head_dim]``
    tensors; windows are the ``cu_seqlens`` segments.  ``softmax_scale`` None
    passes 0, the library's sentinel for ``1/sqrt(head_dim)``.  Returns ``out``
    or ``(out, lse)`` with ``lse`` fp32 ``[B, heads, L]``."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(name, t, torch.bfloat16, q.device)
        if t.dim() != 4 or t.shape != q.shape:
            raise WinAttnError(-1, f"{name} must be [B, L, heads, head_dim] like q")
    _require_cuda("cu_seqlens", cu_seqlens, torch.int32, q.device)
    B, L, Hh, D = q.shape
    if softmax_scale is None:
        softmax_scale = 0.0  # the library's default, 1/sqrt(head_dim)
    if out is None:
        out = torch.empty_like(q)
    _require_cuda("out", out, torch.bfloat16, q.device)
    if out.shape != q.shape:
        raise WinAttnError(-1, "out must have the shape of q")
    lse = torch.empty((B, Hh, L), dtype=torch.float32, device=q.device) if return_lse else None
    N = cu_seqlens.numel() - 1
    _check(lib.win_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), N, int(max_seqlen),
                            L, B, Hh, D, float(softmax_scale), _stream(q)), "win_attn_fwd")
    return (out, lse) if return_lse else out


def attn_fwd_text(q, k, v, cu_seqlens, max_seqlen, text_q, text_k, text_v, softmax_scale=None, out=None,
                  text_out=None, workspace=None, return_lse=False):
    """Window attention over [video window, replicated text] segments; returns
    ``(out, text_out)`` (plus ``lse`` when asked).  ``workspace`` is the fp32
    [B, num_windows, text_len, heads, head_dim] buffer of per-window text
    outputs (allocated here when not given)."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(name, t, torch.bfloat16, q.device)
        if t.dim() != 4 or t.shape != q.shape:
            raise WinAttnError(-1, f"{name} must be [B, L, heads, head_dim] like q")
    B, L, Hh, D = q.shape
    for name, t in (("text_q", text_q), ("text_k", text_k), ("text_v", text_v)):
        _require_cuda(name, t, torch.bfloat16, q.device)
        if t.dim() != 4 or t.shape != text_q.shape or t.shape[0] != B or t.shape[2:] != q.shape[2:]:
            raise WinAttnError(-1, f"{name} must be [B, text_len, heads, head_dim] like text_q")
    _require_cuda("cu_seqlens", cu_seqlens, torch.int32, q.device)
    T = text_q.shape[1]
    N = cu_seqlens.numel() - 1
    if softmax_scale is None:
        softmax_scale = 0.0  # the library's default, 1/sqrt(head_dim)
    if out is None:
        out = torch.empty_like(q)
    if text_out is None:
        text_out = torch.empty_like(text_q)
    if workspace is None:
        workspace = torch.empty((B, max(N, 0), T, Hh, D), dtype=torch.float32, device=q.device)
    _require_cuda("out", out, torch.bfloat16, q.device)
    _require_cuda("text_out", text_out, torch.bfloat16, q.device)
    _require_cuda("workspace", workspace, torch.float32, q.device)
    if out.shape != q.shape or text_out.shape != text_q.shape or workspace.numel() < B * N * T * Hh * D:
        raise WinAttnError(-1, "out, text_out or workspace has the wrong size")
    lse = torch.empty((B, Hh, L), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.win_attn_fwd_text(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), N,
                                 int(max_seqlen), L, B, Hh, D, float(softmax_scale), _ptr(text_q), _ptr(text_k),
                                 _ptr(text_v), T, _ptr(text_out), _ptr(workspace), _stream(q)), "win_attn_fwd_text")
    return (out, text_out, lse) if return_lse else (out, text_out)


def attn_fwd_text_noalloc(q, k, v, cu_seqlens, max_seqlen, text_q, text_k, text_v, softmax_scale=None, out=None,
                          text_out=None, lse=None):
    """``attn_fwd_text`` whose per-window text outputs live in the library's
    static device scratch instead of a caller workspace (see
    ``win_attn_fwd_text_noalloc``).  ``out``, ``text_out`` and the optional
    fp32 ``lse`` [B, heads, L] are the caller's; pass them all for a call that
    allocates nothing.  Returns ``(out, text_out)``."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_cuda(name, t, torch.bfloat16, q.device)
        if t.dim() != 4 or t.shape != q.shape:
            raise WinAttnError(-1, f"{name} must be [B, L, heads, head_dim] like q")
    B, L, Hh, D = q.shape
    for name, t in (("text_q", text_q), ("text_k", text_k), ("text_v", text_v)):
        _require_cuda(name, t, torch.bfloat16, q.device)
        if t.dim() != 4 or t.shape != text_q.shape or t.shape[0] != B or t.shape[2:] != q.shape[2:]:
            raise WinAttnError(-1, f"{name} must be [B, text_len, heads, head_dim] like text_q")
    _require_cuda("cu_seqlens", cu_seqlens, torch.int32, q.device)
    if out is None:
        out = torch.empty_like(q)
    if text_out is None:
        text_out = torch.empty_like(text_q)
    _require_cuda("out", out, torch.bfloat16, q.device)
    _require_cuda("text_out", text_out, torch.bfloat16, q.device)
    if out.shape != q.shape or text_out.shape != text_q.shape:
        raise WinAttnError(-1, "out or text_out has the wrong shape")
    if lse is not None:
        _require_cuda("lse", lse, torch.float32, q.device)
        if lse.shape != (B, Hh, L):
            raise WinAttnError(-1, "lse must be [B, heads, L]")
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(lib.win_attn_fwd_text_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                         cu_seqlens.numel() - 1, int(max_seqlen), L, B, Hh, D, scale, _ptr(text_q),
                                         _ptr(text_k), _ptr(text_v), text_q.shape[1], _ptr(text_out), _stream(q)),
           "win_attn_fwd_text_noalloc")
    return out, text_out
