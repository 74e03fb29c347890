"""The expert cache's replacement policy (moe_cache_*, bookkeeping only: the
dry-run mode issues no copies), against a plain model of least-recently-used
replacement written here: experts with a load stay resident; each missing
expert, in ascending order, takes the lowest free slot, else the slot whose
last use is oldest among those the step does not need (lowest slot first
among equals).  Runs on the CPU."""
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBPATH = os.path.join(ROOT, "fine_grained_moe_amd", "libfgmoe.so")


@pytest.fixture(scope="module")
def moe():
    if not os.path.exists(LIBPATH):
        pytest.fail("libfgmoe.so is not built; run python -m fine_grained_moe_amd.build")
    from fine_grained_moe_amd import moe as m
    return m


class LruModel:
    def __init__(self, E, n_slots):
        self.slot_of = [-1] * E
        self.expert_in = [-1] * n_slots
        self.last = [-1] * n_slots
        self.step = 0
        self.hits = self.misses = 0

    def prepare(self, needed):
        self.step += 1
        for e in needed:
            if self.slot_of[e] >= 0:
                self.last[self.slot_of[e]] = self.step
                self.hits += 1
        m = 0
        for e in sorted(needed):
            if self.slot_of[e] >= 0:
                continue
            free = [s for s in range(len(self.expert_in)) if self.expert_in[s] < 0]
            if free:
                v = free[0]
            else:
                cands = [s for s in range(len(self.expert_in)) if self.last[s] < self.step]
                v = min(cands, key=lambda s: (self.last[s], s))
                self.slot_of[self.expert_in[v]] = -1
            self.slot_of[e] = v
            self.expert_in[v] = e
            self.last[v] = self.step
            self.misses += 1
            m += 1
        return m


def _counts(E, needed):
    c = np.zeros(E, np.int32)
    c[list(needed)] = 1
    return c


@pytest.mark.parametrize("n_slots,max_need,skew", [(4, 2, 0.0), (8, 8, 0.0), (16, 8, 1.0), (64, 40, 0.0)])
def test_policy_matches_the_model(moe, n_slots, max_need, skew):
    E = 64
    rng = np.random.default_rng(n_slots * 100 + max_need)
    dims = moe.make_dims(8, 1024, E, 512, 2048, 1, "bf16", w_routed="int4")
    cache = moe.ExpertCache(dims, n_slots, dry_run=True)
    model = LruModel(E, n_slots)
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    for _ in range(300):
        k = int(rng.integers(1, max_need + 1))
        needed = set(rng.choice(E, size=k, replace=False, p=p).tolist())
        got = cache.prepare(_counts(E, needed))
        want = model.prepare(needed)
        assert got == want
        so, hits, misses = cache.state()
        assert so.tolist() == model.slot_of
        assert (hits, misses) == (model.hits, model.misses)
        for e in needed:                       # every expert with a load is resident
            assert so[e] >= 0
    assert len(set(s for s in so.tolist() if s >= 0)) == sum(s >= 0 for s in so.tolist())   # slots distinct
    cache.close()


def test_more_experts_than_slots_is_refused(moe):
    E = 64
    dims = moe.make_dims(8, 1024, E, 512, 2048, 1, "bf16", w_routed="int4")
    cache = moe.ExpertCache(dims, 3, dry_run=True)
    assert cache.prepare(_counts(E, {1, 2})) == 2
    before = cache.state()
    with pytest.raises(moe.MoeError) as ei:
        cache.prepare(_counts(E, {4, 5, 6, 7}))
    assert ei.value.code == moe.MOE_E_UNSUPPORTED
    after = cache.state()
    assert before[0].tolist() == after[0].tolist() and before[1:] == after[1:]   # nothing changed
    cache.close()


def test_create_checks(moe):
    import ctypes
    d = moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    h = ctypes.c_void_p()
    W = moe.MoeWeights()
    assert moe.LIB.moe_cache_create(ctypes.byref(d), 0, ctypes.byref(W), ctypes.byref(W), None, 1,
                                    ctypes.byref(h)) == moe.MOE_E_ARG
    assert moe.LIB.moe_cache_create(ctypes.byref(d), 65, ctypes.byref(W), ctypes.byref(W), None, 1,
                                    ctypes.byref(h)) == moe.MOE_E_ARG
    # a real (not dry) cache needs its buffers
    assert moe.LIB.moe_cache_create(ctypes.byref(d), 8, ctypes.byref(W), ctypes.byref(W), None, 0,
                                    ctypes.byref(h)) == moe.MOE_E_ARG
    bf = moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16")
    assert moe.LIB.moe_cache_create(ctypes.byref(bf), 8, None, None, None, 1,
                                    ctypes.byref(h)) == moe.MOE_E_UNSUPPORTED
    assert moe.LIB.moe_cache_prepare(None, None, None, None) == moe.MOE_E_ARG


def test_forward_cached_host_checks(moe):
    import ctypes
    d = moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    need = moe.moe_workspace_bytes(d)
    W = moe.MoeWeights(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000)
    R = moe.MoeRouting(*[0x40000000 + i * 0x1000000 for i in range(6)])
    f = moe.LIB.moe_forward_cached
    args = lambda slot, n, dims=d: (ctypes.byref(dims), 0x1000, ctypes.byref(W), slot, n, 0x8000, 0x9000,
                                    ctypes.byref(R), 0x90000000, need, None)
    assert f(*args(None, 8)) == moe.MOE_E_ARG
    assert f(*args(0xA000, 0)) == moe.MOE_E_ARG
    assert f(*args(0xA000, 65)) == moe.MOE_E_ARG
    big = moe.make_dims(65, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")   # the prefill: not streamed
    assert f(*args(0xA000, 8, big)) == moe.MOE_E_UNSUPPORTED
    bf = moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16")
    assert f(*args(0xA000, 8, bf)) == moe.MOE_E_UNSUPPORTED


def test_cache_create_rejects_unknown_flags(moe):
    """moe_cache_create takes MOE_CACHE_DRY_RUN and MOE_CACHE_COPY_FILLS; any
    other bit is an argument error, before anything is created."""
    import ctypes
    dims = moe.make_dims(8, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
    h = ctypes.c_void_p()
    w = moe.MoeWeights()
    for flags in (4, 8, 1 << 30, -1):
        assert moe.LIB.moe_cache_create(ctypes.byref(dims), 4, ctypes.byref(w), ctypes.byref(w), None, flags,
                                        ctypes.byref(h)) == moe.MOE_E_ARG
    code = moe.LIB.moe_cache_create(ctypes.byref(dims), 4, ctypes.byref(w), ctypes.byref(w), None,
                                    moe.MOE_CACHE_DRY_RUN | moe.MOE_CACHE_COPY_FILLS, ctypes.byref(h))
    assert code == moe.MOE_OK and h.value
    moe.LIB.moe_cache_destroy(h)
