"""Shared helpers of the GPU parity tests: layout chains, oracle calls on
host copies of device data, and the error measures."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from window_attention_amd.inputs import bf16_bits

# tolerance of bf16-in / fp32-accumulate attention against the fp64 oracle
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# The kernel's normaliser is the fp32 sum of the probabilities after their
# round-to-nearest bf16 cast (the weights the P V product uses), each within a
# relative 2^-9 of the exact value, so the sum is too and its log moves by at
# most ln(1 + 2^-9) < 2^-9; 5e-4 more covers exp2/log and fp32 accumulation.
LSE_ABS = 2.0 ** -9 + 5e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(x: torch.Tensor) -> np.ndarray:
    if x.dtype == torch.bfloat16:
        return oatt.bf16_bits_to_float64(bf16_bits(x))
    return x.detach().cpu().double().numpy()


def method_of(letter: str) -> int:
    return wa.REGULAR if letter == "R" else wa.SHIFTED


def check_window_head(q, k, v, o, lse, cu_host, b, i, h, scale=None):
    """Oracle attention of (batch b, window i, head h) on host copies of the
    device inputs; returns (max_abs, mean_abs, lse_max_abs, rows)."""
    a, e = int(cu_host[i]), int(cu_host[i + 1])
    if e <= a:
        return 0.0, 0.0, 0.0, 0
    D = q.shape[3]
    s = 1.0 / math.sqrt(D) if scale is None else scale
    qh, kh, vh = (to_f64(x[b, a:e, h]) for x in (q, k, v))
    ref, ref_lse = oatt.head_attention(qh, kh, vh, s)
    got = to_f64(o[b, a:e, h])
    err = np.abs(got - ref)
    lerr = 0.0
    if lse is not None:
        lerr = float(np.max(np.abs(lse[b, h, a:e].double().cpu().numpy() - ref_lse)))
    return float(err.max()), float(err.mean()), lerr, e - a


def assert_close_full(o, lse, ref_o, ref_lse, mask_rows=None):
    got = to_f64(o)
    err = np.abs(got - ref_o)
    if mask_rows is not None:
        err = err[:, mask_rows]
    assert err.max() <= MAX_ABS, f"max abs err {err.max()}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean()}"
    if lse is not None:
        le = np.abs(lse.double().cpu().numpy() - ref_lse)
        if mask_rows is not None:
            le = le[:, :, mask_rows]
        assert le.max() <= LSE_ABS, f"lse err {le.max()}"
    return float(err.max()), float(err.mean())
