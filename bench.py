#!/usr/bin/env python3
"""Benchmark of the window-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
entry gather of Q, K, V into the first layout, then for every attention layer
of the workload's schedule a fused layout transition of Q, K, V (when the
layout changes) and window attention, then the exit scatter of the last
layer's output back to canonical order.  Inputs are resident in HBM before
the timed region starts; nothing is allocated inside it.

Prints ONE JSON line.  `value` is whole-step useful attention TFLOP/s
(useful flops / step time); the attention kernels alone and the permute
kernels alone are reported beside it, each against its roofline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
ATTN_KERNEL = "attn_fwd_kernel<128,4,1,"  # kernel-name prefix of the traffic records


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_21x45x80")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the practical-ceiling measurements (vendor GEMM and plain copy)")
    ap.add_argument("--attn-segments", default=None, metavar="NxLEN",
                    help="also time win_attn_fwd alone on N equal synthetic windows of LEN rows (the workload's heads "
                         "and head_dim), e.g. 4x8192: the kernel's rate where per-window costs vanish")
    ap.add_argument("--clock", action="store_true",
                    help="also sample the shader clock (rocm-smi, read-only) while each attention layer runs in a loop")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (one capture, then --steps replays)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only time a plain device-to-device copy of one workload tensor (the reference kernel of "
                         "known size for HBM byte counters)")
    return ap.parse_args()


class Step:
    """Pre-allocated buffers and the launch sequence of one step."""

    def __init__(self, w, wa, torch, dev):
        from window_attention_amd.inputs import qkv
        self.w, self.wa, self.torch = w, wa, torch
        method = {"R": wa.REGULAR, "S": wa.SHIFTED}
        self.plans = {m: wa.plan_cached(w.T, w.H, w.W, w.nt, w.nh, w.nw, method[m], device=dev) for m in "RS"}
        self.q, self.k, self.v = qkv(w.wid, w.batch, w.L, w.heads, w.head_dim, w.sigma, device=dev)
        e = torch.empty_like
        self.bufs = [[e(self.q), e(self.q), e(self.q)], [e(self.q), e(self.q), e(self.q)]]
        self.o = e(self.q)
        self.out = e(self.q)
        self.stream = torch.cuda.current_stream()
        self.attn_events = []
        self.perm_events = []
        self.row_bytes = w.heads * w.head_dim * 2
        # algorithmic work
        from window_attention_amd.workloads import Workload  # noqa: F401
        self.attn_flops = []
        cur = w.entry
        self.n_perm = 3  # entry gather
        for lay in w.schedule:
            if lay != cur:
                self.n_perm += 3
                cur = lay
            cu = self.plans[lay].cu_seqlens.cpu().tolist()
            self.attn_flops.append(sum(4 * (cu[i + 1] - cu[i]) ** 2 * w.head_dim for i in range(len(cu) - 1))
                                   * w.heads * w.batch)
        self.n_perm += 1  # exit scatter
        # one read and one write of every row, plus the index reads (4 B per
        # row for gather/scatter, 8 B for a transition)
        self.perm_bytes_data = 2 * w.batch * w.L * self.row_bytes

    def permute_launches(self):
        """The step's permute launches in order (entry gather, the fused
        transitions, exit scatter) as closures over the step's buffers."""
        wa, w = self.wa, self.w
        out = []
        cur = w.entry
        src = self.bufs[0]
        p = self.plans[cur]
        for x, dst in zip((self.q, self.k, self.v), src):
            out.append(lambda x=x, dst=dst, p=p: wa.gather(x, p.perm, out=dst))
        side = 0
        for lay in w.schedule:
            if lay != cur:
                pa, pb = self.plans[cur], self.plans[lay]
                dst = self.bufs[1 - side]
                for s_, d_ in zip(src, dst):
                    out.append(lambda s_=s_, d_=d_, pa=pa, pb=pb: wa.transition(s_, pa.inv, pb.perm, out=d_))
                side = 1 - side
                src = dst
                cur = lay
        pl = self.plans[cur]
        out.append(lambda pl=pl: wa.scatter(self.o, pl.perm, out=self.out))
        return out

    def run(self, timed=False):
        wa, w, torch = self.wa, self.w, self.torch
        ev = (lambda: torch.cuda.Event(enable_timing=True)) if timed else None
        cur = w.entry
        src = self.bufs[0]

        def perm_launch(fn):
            if timed:
                a, b = ev(), ev()
                a.record(self.stream)
                fn()
                b.record(self.stream)
                self.perm_events.append((a, b))
            else:
                fn()

        p = self.plans[cur]
        for x, dst in zip((self.q, self.k, self.v), src):
            perm_launch(lambda x=x, dst=dst: wa.gather(x, p.perm, out=dst))
        side = 0
        for lay in w.schedule:
            if lay != cur:
                pa, pb = self.plans[cur], self.plans[lay]
                dst = self.bufs[1 - side]
                for s_, d_ in zip(src, dst):
                    perm_launch(lambda s_=s_, d_=d_: wa.transition(s_, pa.inv, pb.perm, out=d_))
                side = 1 - side
                src = dst
                cur = lay
            pl = self.plans[lay]
            if timed:
                a, b = ev(), ev()
                a.record(self.stream)
            wa.attn_fwd(src[0], src[1], src[2], pl.cu_seqlens, pl.max_seqlen, out=self.o)
            if timed:
                b.record(self.stream)
                self.attn_events.append((a, b))
        pl = self.plans[cur]
        perm_launch(lambda: wa.scatter(self.o, pl.perm, out=self.out))


def graph_step_rate(st, torch, steps):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph) and
    replayed: no host launch work per kernel.  The replayed step's output is
    compared bit for bit with the eager step's."""
    st.run()
    torch.cuda.synchronize()
    eager_out = st.out.clone()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()  # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    st.out.fill_(7.0)
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(st.out, eager_out))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"ms_per_step": round(ms, 4), "value": round(sum(st.attn_flops) / (ms * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s", "bit_identical_to_eager": same}


def rope_gather_rate(st, torch, reps=20, text_len=58):
    """The window-local RoPE gather of Q into the shifted layout (rotary span
    126 of 128 channels), timed on its own beside the step: GB/s of its one
    read and one write of every row."""
    wa, w = st.wa, st.w
    if w.head_dim != 128:
        return None
    p = st.plans["S"]
    loc = wa.local_positions(p, device="cuda")
    tab = wa.rope_table(p, text_len, 126, device="cuda")
    dst = st.bufs[0][0]
    for _ in range(3):
        wa.gather_rope(st.q, p, loc, tab, 126, out=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(st.stream)
    for _ in range(reps):
        wa.gather_rope(st.q, p, loc, tab, 126, out=dst)
    b.record(st.stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = st.perm_bytes_data / (ms * 1e-3) / 1e9
    return {"kernel": "rope_rows_kernel (gather, shifted layout, rotary span 126/128, text_len 58)",
            "avg_launch_ms": round(ms, 4), "bytes_per_launch": st.perm_bytes_data, "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}


def text_attention_rate(st, torch, text_len=256, reps=10):
    """Window attention over [video window, replicated text] segments in the
    shifted layout, timed on its own beside the step (the text stream is not
    part of the step's schedule): useful TFLOP/s of the segment attention of
    every window, the per-window text rows included, over the whole call (the
    attention kernel and the text mean)."""
    from window_attention_amd.inputs import normal
    wa, w = st.wa, st.w
    p = st.plans["S"]
    tq, tk, tv = (normal((w.batch, text_len, w.heads, w.head_dim), 800 + t, w.sigma, device="cuda") for t in range(3))
    N = p.num_windows
    ws = torch.empty((w.batch, N, text_len, w.heads, w.head_dim), dtype=torch.float32, device="cuda")
    o, to = torch.empty_like(st.q), torch.empty_like(tq)
    src = st.bufs[0]
    for x, dst in zip((st.q, st.k, st.v), src):
        wa.gather(x, p.perm, out=dst)
    for _ in range(3):
        wa.attn_fwd_text(src[0], src[1], src[2], p.cu_seqlens, p.max_seqlen, tq, tk, tv, out=o, text_out=to,
                         workspace=ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(st.stream)
    for _ in range(reps):
        wa.attn_fwd_text(src[0], src[1], src[2], p.cu_seqlens, p.max_seqlen, tq, tk, tv, out=o, text_out=to,
                         workspace=ws)
    b.record(st.stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    cu = p.cu_seqlens.cpu().tolist()
    flops = sum(4 * (cu[i + 1] - cu[i] + text_len) ** 2 * w.head_dim for i in range(N)) * w.heads * w.batch
    tfs = flops / (ms * 1e-3) / 1e12
    return {"kernel": f"attn_fwd_kernel (text rows) + text_mean_kernel, shifted layout, {text_len} text rows",
            "avg_call_ms": round(ms, 4), "flops_per_call": flops, "achieved": round(tfs, 2),
            "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / BF16_MFMA_PEAK_TFS, 4)}


FLUSH_BYTES = 1 << 30  # at least the 256 MB Infinity Cache plus the 8 x 4 MB of L2, four times over


def permute_rate_flushed(st, torch, reps):
    """The step's permutes with the caches flushed before each launch: a
    1 GiB scratch buffer is overwritten and a second 1 GiB buffer is read
    (which writes the first one's dirty lines back and leaves the caches
    full of unrelated clean lines), then the permute runs between two
    events on the launch stream.  GB/s of its algorithmic bytes."""
    n = FLUSH_BYTES // 4
    fill = torch.empty(n, dtype=torch.float32, device="cuda")
    other = torch.zeros(n, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    launches = st.permute_launches()
    ev = []
    for r in range(reps + 1):
        for fn in launches:
            fill.fill_(float(r))
            torch.sum(other, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st.stream)
            fn()
            b.record(st.stream)
            if r > 0:  # the first round is a warm-up
                ev.append((a, b))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    del fill, other
    avg = sum(ms) / len(ms)
    gbs = st.perm_bytes_data / (avg * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(avg, 4),
            "bytes_per_launch": st.perm_bytes_data, "launches": len(ms),
            "kernel": "permute_rows_kernel (gather, transition, scatter)",
            "flush": f"{FLUSH_BYTES >> 20} MiB overwritten and another {FLUSH_BYTES >> 20} MiB read before each "
                     "launch"}


def measured_traffic(kernel_prefix, workload):
    """HBM bytes per launch (read + write) recorded in profiles/hbm_traffic.txt
    for a kernel, or None when there is no record for this workload or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if line.startswith("#") or not line.strip():
            continue
        rec = dict(kv.split("=", 1) for kv in line.split())
        if not rec["kernel"].startswith(kernel_prefix) or rec.get("workload") != workload:
            continue
        src = os.path.join(ROOT, rec["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["sha256"]:
            return None
        return {"fetch_bytes": int(rec["fetch_bytes"]), "write_bytes": int(rec["write_bytes"]),
                "total_bytes": int(rec["fetch_bytes"]) + int(rec["write_bytes"])}
    return None


def practical_ceilings(torch, w, reps=20):
    """What this machine sustains, measured here beside the path (context only, not
    part of it): a vendor dense bf16 GEMM on N(0,1) data, whose power-limited
    clock is the practical ceiling of an MFMA-bound kernel on real data, and a
    plain device copy of one workload-sized tensor, the practical ceiling of a
    permute."""
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty_like(a)
    for _ in range(3):
        torch.matmul(a, a, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, a, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tfs = 2 * n ** 3 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
    del a, c
    x = torch.empty((w.batch, w.L, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda").fill_(1.0)
    x_bytes = x.numel() * 2
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 2 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del x, y
    res = {"gemm_bf16_tflops": round(gemm_tfs, 1), "gemm": f"torch.matmul bf16 {n}x{n}x{n}, N(0,1) data",
           "copy_gbps": round(copy_gbs, 1), "copy": f"device copy of {x_bytes} bytes"}
    res.update(mfma_loop_rate(torch))
    return res


def mfma_loop_rate(torch, reps=10, iters=32768):
    """The chip's sustained bf16 MFMA rate on changing N(0,1) register data
    (libwinprobe.so: eight independent 32x32x16 chains per wave, two
    workgroups of four waves per CU, no memory traffic in the loop): the
    ceiling of any kernel's MFMA work under the power limit."""
    import ctypes
    path = os.path.join(ROOT, "window_attention_amd", "libwinprobe.so")
    if not os.path.exists(path):
        return {"mfma_loop_tflops": None, "mfma_loop": "libwinprobe.so not built"}
    lib = ctypes.CDLL(path)
    lib.win_probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p]
    lib.win_probe_mfma_loop.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    src = torch.randn(1 << 19, device="cuda").to(torch.bfloat16)
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: lib.win_probe_mfma_loop(src.data_ptr(), src.numel(), out.data_ptr(), blocks, iters, st)  # noqa
    for _ in range(2):
        if call() != 0:
            return {"mfma_loop_tflops": None, "mfma_loop": "launch failed"}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = blocks * 4 * 8 * ((iters + 3) // 4 * 4) * 32768
    return {"mfma_loop_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_loop": f"{blocks} workgroups x 4 waves x 8 chains of mfma_f32_32x32x16_bf16 on N(0,1) "
                         f"register operands, {iters} per chain"}


def sample_sclk(stop, out):
    """Shader clock readings (MHz) of `rocm-smi --showclocks` until stop is set."""
    import subprocess
    while not stop.is_set():
        try:
            r = subprocess.run(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                               text=True, timeout=5).stdout
            for ln in r.splitlines():
                if "sclk" in ln and "(" in ln and "Mhz" in ln:
                    out.append(int(ln.split("(")[1].split("Mhz")[0]))
                    break
        except Exception:
            return
        time.sleep(0.1)


def attention_clock(st, torch, seconds=2.0):
    """Each distinct layout's attention call in a loop for about `seconds`,
    with the shader clock sampled meanwhile: per layout the median clock, the
    rate and the useful flops per clock cycle per CU."""
    import threading
    wa, w = st.wa, st.w
    out = {}
    cur = w.entry
    src = st.bufs[0]
    for x, dst in zip((st.q, st.k, st.v), src):
        wa.gather(x, st.plans[cur].perm, out=dst)
    for li, lay in enumerate(w.schedule):
        if lay in out:
            continue
        pl = st.plans[lay]
        if lay != cur:
            for s_, d_ in zip(src, st.bufs[1]):
                wa.transition(s_, st.plans[cur].inv, pl.perm, out=d_)
            src, cur = st.bufs[1], lay
        call = lambda: wa.attn_fwd(src[0], src[1], src[2], pl.cu_seqlens, pl.max_seqlen, out=st.o)  # noqa: E731
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        clk, stop = [], threading.Event()
        th = threading.Thread(target=sample_sclk, args=(stop, clk))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(1, int(seconds / 1.5e-3))
        th.start()
        a.record(st.stream)
        for _ in range(n):
            call()
        b.record(st.stream)
        torch.cuda.synchronize()
        stop.set()
        th.join()
        ms = a.elapsed_time(b) / n
        tfs = st.attn_flops[li] / (ms * 1e-3) / 1e12
        mhz = sorted(clk)[len(clk) // 2] if clk else None
        out[lay] = {"ms": round(ms, 4), "tflops": round(tfs, 1), "sclk_mhz": mhz, "samples": len(clk),
                    "flop_per_cycle_per_cu": round(tfs * 1e12 / (mhz * 1e6) / 256, 1) if mhz else None}
    return out


def attention_on_segments(st, torch, spec, reps=10):
    """win_attn_fwd alone on `spec` = "NxLEN" equal windows of synthetic
    N(0,1) rows with the workload's heads and head_dim: TFLOP/s of the best of
    five timed loops of `reps` calls."""
    from window_attention_amd.inputs import normal
    wa, w = st.wa, st.w
    n, length = (int(x) for x in spec.lower().split("x"))
    L = n * length
    q, k, v = (normal((1, L, w.heads, w.head_dim), 7000 + t, device="cuda") for t in range(3))
    cu = torch.arange(0, L + 1, length, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    for _ in range(3):
        wa.attn_fwd(q, k, v, cu, length, out=o)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(5):
        a.record(st.stream)
        for _ in range(reps):
            wa.attn_fwd(q, k, v, cu, length, out=o)
        b.record(st.stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        best = ms if best is None else min(best, ms)
    flops = 4 * n * length * length * w.head_dim * w.heads
    return {"windows": n, "rows": length, "heads": w.heads, "head_dim": w.head_dim, "ms": round(best, 4),
            "tflops": round(flops / (best * 1e-3) / 1e12, 1),
            "frac": round(flops / (best * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS, 4)}


def host_cpu_model():
    """The host's CPU model name as lscpu reports it (None if unavailable)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True,
                             timeout=10).stdout
    except Exception:
        return None
    for line in out.splitlines():
        if line.lower().startswith("model name"):
            return line.split(":", 1)[1].strip()
    return None


def cpu_baseline(st, seconds):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload, on the workload's own bf16 bytes (copied from the
    device, decoded exactly with the oracle's bf16 decoder): the planner on
    the whole grid (single-threaded Python), the gather of the whole Q into
    the first layout (a NumPy take of bf16 bit patterns), and fp64
    per-window attention over the first layout's windows, head by head,
    until the time budget is used.  `value` is the attention rate."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import permute as operm
    from oracle import plan as oplan
    from window_attention_amd.inputs import bf16_bits
    w = st.w
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=None)
    except Exception:
        threads = None
    ncpu = os.cpu_count() or 1
    threads = threads or ncpu
    method = 0 if w.schedule[0] == "R" else 1
    t0 = time.perf_counter()
    p = oplan.plan(w.T, w.H, w.W, w.nt, w.nh, w.nw, method)
    t_plan = time.perf_counter() - t0
    # the workload's canonical bf16 bytes, [B, L, heads, D] as uint16 bit patterns
    hq, hk, hv = (bf16_bits(x) for x in (st.q, st.k, st.v))
    t0 = time.perf_counter()
    qw = operm.gather(hq, p.perm)
    t_gather = time.perf_counter() - t0
    kw, vw = operm.gather(hk, p.perm), operm.gather(hv, p.perm)
    gather_gbs = 2 * qw.nbytes / t_gather / 1e9
    D = w.head_dim
    scale = 1.0 / math.sqrt(D)
    flops, done, t_attn = 0, 0, 0.0
    for i in range(p.num_windows):
        a, e = p.cu_seqlens[i], p.cu_seqlens[i + 1]
        for h in range(w.heads):
            x = [oatt.bf16_bits_to_float64(t[0, a:e, h]) for t in (qw, kw, vw)]
            t0 = time.perf_counter()
            oatt.head_attention(x[0], x[1], x[2], scale)
            t_attn += time.perf_counter() - t0
            flops += 4 * (e - a) ** 2 * D
            done += 1
            if t_attn > seconds:
                break
        if t_attn > seconds:
            break
    lay = "regular" if method == 0 else "shifted"
    return {
        "value": flops / t_attn / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"fp64 attention (oracle head_attention) of the first {done} (window, head) pairs of the "
                  f"{w.name} {lay} layout on the workload's own bf16 inputs ({flops / 1e9:.1f} GFLOP in "
                  f"{t_attn:.1f} s); planner {t_plan:.3f} s for the whole grid; gather of the whole Q "
                  f"({qw.nbytes / 1e6:.0f} MB) at {gather_gbs:.2f} GB/s",
        "attention_tflops": round(flops / t_attn / 1e12, 4),
        "planner_s": round(t_plan, 4),
        "gather_gbps": round(gather_gbs, 3),
        "host": {"cpu_count": ncpu, "blas_threads": threads, "model": host_cpu_model()},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import window_attention_amd as wa
    from window_attention_amd.workloads import BY_NAME
    w = BY_NAME[args.workload]
    dev = "cuda"
    wa.load_library()
    if args.copy_calibration:
        x = torch.empty((w.batch, w.L, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            y.copy_(x)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        nbytes = x.numel() * 2
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms_per_copy": round(ms, 4),
                          "gbps": round(2 * nbytes / ms / 1e6, 1)}), flush=True)
        return
    log(f"[bench] {w.name}: grid {w.T}x{w.H}x{w.W} B={w.batch} heads={w.heads} D={w.head_dim} "
        f"entry={w.entry} schedule={','.join(w.schedule)}")
    st = Step(w, wa, torch, dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    # whole-step timing, no per-kernel events inside
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        st.run()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step")
    # per-kernel timing pass (events around every launch, same stream)
    for _ in range(args.steps):
        st.run(timed=True)
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in st.attn_events]
    perm_ms = [a.elapsed_time(b) for a, b in st.perm_events]
    nl = len(w.schedule)
    attn_flops_step = sum(st.attn_flops)
    attn_ms_step = sum(attn_ms) / args.steps
    attn_tfs = attn_flops_step / (attn_ms_step * 1e-3) / 1e12
    perm_bytes_launch = st.perm_bytes_data
    perm_gbs = perm_bytes_launch / (sum(perm_ms) / len(perm_ms) * 1e-3) / 1e9
    layers = []
    for li, lay in enumerate(w.schedule):
        ms = sorted(attn_ms[li::nl])[len(attn_ms[li::nl]) // 2]
        layers.append({"layout": lay, "median_ms": round(ms, 4),
                       "tflops": round(st.attn_flops[li] / ms / 1e9, 2)})
        log(f"[bench] attn layer {li} ({lay}): median {ms:.3f} ms, {st.attn_flops[li] / ms / 1e9:.1f} TFLOP/s")
    log(f"[bench] permutes in the step: {len(perm_ms) // args.steps}/step, mean "
        f"{sum(perm_ms) / len(perm_ms) * 1e3:.1f} us, {perm_gbs:.0f} GB/s")
    flushed = permute_rate_flushed(st, torch, args.steps)
    log(f"[bench] permutes after a cache flush: mean {flushed['avg_launch_ms'] * 1e3:.1f} us, "
        f"{flushed['achieved']:.0f} GB/s")
    value = attn_flops_step / (ms_step * 1e-3) / 1e12
    rope = rope_gather_rate(st, torch)
    if rope:
        log(f"[bench] rope gather (beside the step): {rope['avg_launch_ms'] * 1e3:.1f} us, {rope['achieved']:.0f} GB/s")
    text = text_attention_rate(st, torch) if w.head_dim == 128 else None
    if rope:
        t = measured_traffic("rope_rows_kernel", w.name)
        rope["traffic"], rope["traffic_detail"] = (t["total_bytes"] if t else None), t
    if text:
        t = measured_traffic(ATTN_KERNEL + "true>", w.name)
        m = measured_traffic("text_mean_kernel", w.name)
        text["traffic"] = t["total_bytes"] + m["total_bytes"] if t and m else None
        text["traffic_detail"] = {"attn_fwd_kernel": t, "text_mean_kernel": m} if t and m else None
        log(f"[bench] text attention (beside the step): {text['avg_call_ms']:.3f} ms, {text['achieved']:.0f} TFLOP/s")
    attn_traffic = measured_traffic(ATTN_KERNEL + "false>", w.name)
    perm_traffic = measured_traffic("permute_rows_kernel<transition>", w.name)
    # Roofline of the attention kernel.  Its algorithmic HBM bytes per launch
    # are one read of Q, K, V and one write of O; below the ridge point
    # (peak flops / peak bandwidth, 312.5 flop/B) the kernel is HBM-bound and
    # its ceiling is the bytes at 8 TB/s.
    attn_bytes = 4 * w.batch * w.L * w.heads * w.head_dim * 2
    flops_launch = attn_flops_step / nl
    intensity = flops_launch / attn_bytes
    ceiling_tfs = min(BF16_MFMA_PEAK_TFS, intensity * HBM_PEAK_GBS / 1e3)
    launch_ms = attn_ms_step / nl
    if intensity < BF16_MFMA_PEAK_TFS * 1e3 / HBM_PEAK_GBS:
        gbs = attn_bytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(attn_tfs, 2), "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(attn_tfs / BF16_MFMA_PEAK_TFS, 4)}
    roof.update({"traffic": attn_traffic["total_bytes"] if attn_traffic else None,
                 "traffic_detail": attn_traffic, "kernel": "attn_fwd_kernel", "avg_launch_ms": round(launch_ms, 4),
                 "flops_per_launch": flops_launch, "bytes_per_launch": attn_bytes,
                 "flop_per_byte": round(intensity, 1), "ceiling_tflops": round(ceiling_tfs, 1),
                 "frac_of_ceiling": round(attn_tfs / ceiling_tfs, 4), "layers": layers})
    res = {
        "metric": "window-attn useful TFLOP/s + permute GB/s, 21x45x80 grid bf16, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "grid": [w.T, w.H, w.W], "window_counts": [w.nt, w.nh, w.nw],
                   "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "entry": w.entry,
                   "schedule": ",".join(w.schedule), "parallelism": "none (1 GPU)"},
        "attn_tflops": round(attn_tfs, 2),
        "permute_gbps": round(flushed["achieved"], 1),
        "roofline": roof,
        "roofline_permute": dict(flushed, traffic=perm_traffic["total_bytes"] if perm_traffic else None,
                                 traffic_detail=perm_traffic),
        "roofline_permute_in_step": {"bound": "hbm", "achieved": round(perm_gbs, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(perm_gbs / HBM_PEAK_GBS, 4),
                                     "kernel": "permute_rows_kernel (gather, transition, scatter)",
                                     "avg_launch_ms": round(sum(perm_ms) / len(perm_ms), 4),
                                     "bytes_per_launch": perm_bytes_launch,
                                     "note": "timed inside the step, caches as the step leaves them"},
        "roofline_rope_permute": rope,
        "roofline_text_attention": text,
    }
    if args.graph:
        res["graph"] = graph_step_rate(st, torch, args.steps)
        log(f"[bench] step replayed from a HIP graph: {res['graph']}")
    if args.attn_segments:
        res["attn_segments"] = attention_on_segments(st, torch, args.attn_segments)
        log(f"[bench] attention alone on {args.attn_segments} equal windows: {res['attn_segments']}")
    if args.clock:
        res["roofline"]["clock"] = attention_clock(st, torch)
        log(f"[bench] attention under a sampled clock: {res['roofline']['clock']}")
    if not args.no_ceilings:
        ceil = practical_ceilings(torch, w)
        ceil["attn_frac_of_gemm"] = round(attn_tfs / ceil["gemm_bf16_tflops"], 4)
        ceil["permute_frac_of_copy"] = round(perm_gbs / ceil["copy_gbps"], 4)
        if ceil.get("mfma_loop_tflops"):
            ceil["attn_frac_of_mfma_loop"] = round(attn_tfs / ceil["mfma_loop_tflops"], 4)
        log(f"[bench] practical ceilings: vendor bf16 GEMM {ceil['gemm_bf16_tflops']} TFLOP/s "
            f"(attention at {ceil['attn_frac_of_gemm']:.2f} of it), device copy {ceil['copy_gbps']} GB/s "
            f"(permutes at {ceil['permute_frac_of_copy']:.2f} of it), MFMA loop on N(0,1) registers "
            f"{ceil.get('mfma_loop_tflops')} TFLOP/s (attention at {ceil.get('attn_frac_of_mfma_loop')} of it)")
        res["practical_ceilings"] = ceil
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle sample, about {args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
