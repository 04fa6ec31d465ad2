"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, validates descriptors before touching the device, and
its host-side cache policy matches the oracle's replay."""
import os
import re

import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, make_layer
from oracle.lfu import LfuReplay, LruPoolReplay

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = M.load()
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(M.exported_symbols()) == names


def test_invalid_descriptors_rejected_without_gpu():
    w = WORKLOADS[0]
    arrays = make_layer(w)
    bad = [dict(d_model=100), dict(top_k=0), dict(top_k=17), dict(d_ff=100), dict(n_experts=0),
           dict(act_dtype=7), dict(max_tokens=0), dict(d_ff_shared=10), dict(residency=3)]
    for b in bad:
        kw = dict(d_model=w.d, n_experts=w.E, top_k=w.K, d_ff=w.f, d_ff_shared=w.fs,
                  act_dtype=M.MOE_ACT_F32, max_tokens=4)
        kw.update(b)
        desc, keep = M.make_desc(arrays, **kw)
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_create(desc)
        assert ei.value.status == M.MOE_ERR_INVALID, b
    a2 = dict(arrays, gate_q=None)
    desc, keep = M.make_desc(a2, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_F32, 4)
    with pytest.raises(M.MoeError):
        M.moe_layer_create(desc)


def test_lfu_golden_trace_through_abi():
    here = os.path.dirname(os.path.abspath(__file__))
    lfu = M.moe_lfu_create(4)
    try:
        for line in open(os.path.join(here, "golden", "lfu_trace.txt")):
            line = line.split("#")[0].strip()
            if not line:
                continue
            step, chosen, slots, misses = [list(map(int, p.split())) for p in line.split("|")]
            s, m = M.moe_lfu_step(lfu, chosen)
            assert list(s) == slots and list(m) == misses, step
        st = M.moe_lfu_stats(lfu)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == (10, 2, 8, 4)
    finally:
        M.moe_lfu_destroy(lfu)


def test_lfu_prefetch_golden_trace_through_abi():
    here = os.path.dirname(os.path.abspath(__file__))
    lfu = M.moe_lfu_create(4)
    try:
        for line in open(os.path.join(here, "golden", "lfu_prefetch_trace.txt")):
            line = line.split("#")[0].strip()
            if not line:
                continue
            op, experts, slots, misses = [p.strip() for p in line.split("|")]
            experts, slots = list(map(int, experts.split())), list(map(int, slots.split()))
            if op == "step":
                s, m = M.moe_lfu_step(lfu, experts)
                assert list(s) == slots and list(m) == list(map(int, misses.split())), line
            else:
                assert list(M.moe_lfu_prefetch(lfu, experts)) == slots, line
        st = M.moe_lfu_stats(lfu)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"], st["prefetches"],
                st["prefetch_used"]) == (6, 2, 4, 4, 4, 2)
    finally:
        M.moe_lfu_destroy(lfu)


@pytest.mark.parametrize("seed", range(3))
def test_lfu_prefetch_matches_replay_on_random_traces(seed):
    rng = np.random.default_rng(200 + seed)
    n_slots, E, K = 16, 128, 8
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    zipf /= zipf.sum()
    lfu = M.moe_lfu_create(n_slots)
    ref = LfuReplay(n_slots)
    try:
        for step in range(300):
            if rng.random() < 0.5:
                guess = rng.choice(E, int(rng.integers(1, 9)), replace=False, p=zipf).astype(np.int32)
                got = M.moe_lfu_prefetch(lfu, guess)
                placed = ref.prefetch(guess.tolist())
                assert list(got) == [placed.get(int(e), -1) for e in guess], step
            chosen = np.sort(rng.choice(E, K, replace=False, p=zipf)).astype(np.int32)
            s, m = M.moe_lfu_step(lfu, chosen)
            rs, rm = ref.step(chosen.tolist())
            assert list(s) == rs and [bool(v) for v in m] == rm, step
        st = M.moe_lfu_stats(lfu)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"], st["prefetches"],
                st["prefetch_used"]) == (ref.accesses, ref.hits, ref.misses, ref.evictions, ref.prefetches,
                                         ref.prefetch_used)
    finally:
        M.moe_lfu_destroy(lfu)


def test_lru_golden_trace_through_abi():
    here = os.path.dirname(os.path.abspath(__file__))
    lru = M.moe_lru_create(4)
    try:
        for line in open(os.path.join(here, "golden", "lru_pool_trace.txt")):
            line = line.split("#")[0].strip()
            if not line:
                continue
            step, layer, chosen, slots, misses = [list(map(int, p.split())) for p in line.split("|")]
            s, m = M.moe_lru_step(lru, layer[0], chosen)
            assert list(s) == slots and list(m) == misses, step
        st = M.moe_lru_stats(lru)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == (13, 4, 9, 5)
        with pytest.raises(M.MoeError):
            M.moe_lru_step(lru, 0, [1, 1])
        with pytest.raises(M.MoeError):
            M.moe_lru_step(lru, 0, [1, 2, 3, 4, 5])
        with pytest.raises(M.MoeError):
            M.moe_lru_step(lru, -1, [1])
    finally:
        M.moe_lru_destroy(lru)


@pytest.mark.parametrize("seed", range(3))
def test_lru_matches_replay_on_random_stack_traces(seed):
    rng = np.random.default_rng(100 + seed)
    n_slots, E, K, layers = 40, 64, 8, 5
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    zipf /= zipf.sum()
    lru = M.moe_lru_create(n_slots)
    ref = LruPoolReplay(n_slots)
    prev = [None] * layers
    try:
        for step in range(120):
            for l in range(layers):
                if prev[l] is not None and rng.random() < 0.6:
                    chosen = prev[l]
                else:
                    chosen = np.sort(rng.choice(E, K, replace=False, p=zipf)).astype(np.int32)
                s, m = M.moe_lru_step(lru, l, chosen)
                rs, rm = ref.step(l, chosen.tolist())
                assert list(s) == rs and [bool(v) for v in m] == rm, (step, l)
                prev[l] = chosen
        st = M.moe_lru_stats(lru)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == \
            (ref.accesses, ref.hits, ref.misses, ref.evictions)
    finally:
        M.moe_lru_destroy(lru)


@pytest.mark.parametrize("seed", range(5))
def test_lfu_matches_replay_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    n_slots, E, K = 16, 256, 8
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    zipf /= zipf.sum()
    lfu = M.moe_lfu_create(n_slots)
    ref = LfuReplay(n_slots)
    prev = None
    try:
        for step in range(400):
            if prev is not None and rng.random() < 0.6:
                chosen = prev
            else:
                chosen = np.sort(rng.choice(E, K, replace=False, p=zipf)).astype(np.int32)
            s, m = M.moe_lfu_step(lfu, chosen)
            rs, rm = ref.step(chosen.tolist())
            assert list(s) == rs and [bool(v) for v in m] == rm, step
            prev = chosen
        st = M.moe_lfu_stats(lfu)
        assert (st["accesses"], st["hits"], st["misses"], st["evictions"]) == \
            (ref.accesses, ref.hits, ref.misses, ref.evictions)
    finally:
        M.moe_lfu_destroy(lfu)


def test_lfu_rejects_bad_steps():
    lfu = M.moe_lfu_create(2)
    try:
        with pytest.raises(M.MoeError):
            M.moe_lfu_step(lfu, [1, 1])
        with pytest.raises(M.MoeError):
            M.moe_lfu_step(lfu, [1, 2, 3])
    finally:
        M.moe_lfu_destroy(lfu)
