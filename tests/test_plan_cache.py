"""The binding's plan cache (window page, section "Planner": plans are cached
by geometry): hits return the same tables, the least recently used plan is
evicted at capacity, and the key separates method and device.  CPU only."""
import numpy as np

import window_attention_amd as wa
from oracle import plan as oplan


def test_plan_cache_hits_lru_and_eviction(monkeypatch):
    monkeypatch.setattr(wa, "PLAN_CACHE_SIZE", 3)
    wa._PLAN_CACHE.clear()
    a = wa.plan_cached(3, 5, 7, 2, 17, 9, wa.REGULAR)
    assert wa.plan_cached(3, 5, 7, 2, 17, 9, wa.REGULAR) is a            # hit: same object
    s = wa.plan_cached(3, 5, 7, 2, 17, 9, wa.SHIFTED)                     # method is part of the key
    assert s is not a and not np.array_equal(s.cu_seqlens.numpy(), a.cu_seqlens.numpy())
    b = wa.plan_cached(1, 3, 4, 1, 26, 35, wa.REGULAR)
    assert len(wa._PLAN_CACHE) == 3
    assert wa.plan_cached(3, 5, 7, 2, 17, 9, wa.REGULAR) is a            # refresh a: s is now the oldest
    c = wa.plan_cached(5, 9, 16, 2, 3, 3, wa.REGULAR)                     # evicts s
    assert len(wa._PLAN_CACHE) == 3
    keys = list(wa._PLAN_CACHE)
    assert all(k[6] == wa.REGULAR for k in keys)
    assert wa.plan_cached(3, 5, 7, 2, 17, 9, wa.SHIFTED) is not s         # rebuilt after eviction
    # a cached plan is still the plan: it matches the oracle
    for p, g in ((a, (3, 5, 7, 2, 17, 9)), (b, (1, 3, 4, 1, 26, 35)), (c, (5, 9, 16, 2, 3, 3))):
        op = oplan.plan(*g, 0)
        assert np.array_equal(p.perm.numpy(), np.asarray(op.perm, dtype=np.int32))
        assert np.array_equal(p.cu_seqlens.numpy(), np.asarray(op.cu_seqlens, dtype=np.int32))
    wa._PLAN_CACHE.clear()


def test_plan_cache_host_key():
    wa._PLAN_CACHE.clear()
    h = wa.plan_cached(2, 5, 7, 1, 3, 3, wa.REGULAR)
    # None and "cpu" both mean host tables: one entry
    assert wa.plan_cached(2, 5, 7, 1, 3, 3, wa.REGULAR, device="cpu") is h
    assert len(wa._PLAN_CACHE) == 1
    assert list(wa._PLAN_CACHE)[0][7] == "cpu"
    wa._PLAN_CACHE.clear()
