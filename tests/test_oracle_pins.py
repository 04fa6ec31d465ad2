"""Pins of the fp64 oracle against things other than itself: closed forms,
special cases that reduce to library routines, brute force on tiny inputs,
invariants of the method and a hand-worked cache trace.  CPU only."""
import os

import numpy as np
import pytest

from gen.workloads import WORKLOADS, Workload, make_layer, make_tokens, f32_to_bf16_bits
from oracle import brute
from oracle import oracle as O
from oracle.lfu import LfuReplay, LruPoolReplay

HERE = os.path.dirname(os.path.abspath(__file__))


def tiny(d=128, E=8, K=2, f=64, fs=64, zipf=None, seed=0, wid=90):
    w = Workload(wid, "tiny", d=d, E=E, K=K, f=f, fs=fs, act="f32", zipf=zipf, T=3)
    return w, make_layer(w, seed=seed)


def f16bits(v):
    return np.array(v, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------- formats
def test_f16_decoding_matches_numpy():
    bits = np.arange(0, 0x10000, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]  # finite only
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(b) for b in bits])
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_fp32_route_and_ties_to_even():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)  # exactly fp32
    ref = f32_to_bf16_bits(v)
    got = np.array([O.f64_to_bf16(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert O.f64_to_bf16(1.0) == 0x3F80
    assert O.f64_to_bf16(1.0 + 2.0**-8) == 0x3F80          # tie -> even
    assert O.f64_to_bf16(1.0 + 3 * 2.0**-8) == 0x3F82      # tie -> even (up)
    assert O.f64_to_bf16(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81  # above the tie (fp64 only)
    assert O.f64_to_bf16(-2.0) == 0xC000


# ---------------------------------------------------------------- dequant
@pytest.mark.parametrize("qval", [0, 8, 15])
def test_dequant_constant_nibbles(qval):
    rows, cols = 3, 128
    word = sum(qval << (4 * k) for k in range(8))
    q = np.full((rows, cols // 8), word, np.uint32)
    s = f16bits(np.linspace(0.002, 0.02, rows * 2).reshape(rows, 2))
    b = f16bits(-8 * np.linspace(0.002, 0.02, rows * 2).reshape(rows, 2) + 1e-4)
    W = O.dequant(q, s, b)
    S = s.view(np.float16).astype(np.float64)
    B = b.view(np.float16).astype(np.float64)
    expect = np.repeat(qval * S + B, 64, axis=1)   # all-q=v group equals v*scale + bias
    assert np.array_equal(W, expect)


def test_dequant_one_hot_pins_nibble_order_and_group():
    rows, cols = 2, 256
    s = f16bits(np.arange(1, 1 + rows * 4, dtype=np.float64).reshape(rows, 4) / 64)
    b = f16bits(-np.arange(1, 1 + rows * 4, dtype=np.float64).reshape(rows, 4) / 128)
    for r in range(rows):
        for c in (0, 1, 7, 8, 63, 64, 100, 255):
            q = np.zeros((rows, cols // 8), np.uint32)
            q[r, c // 8] = np.uint32(0xB) << np.uint32(4 * (c % 8))  # nibble value 11 at column c
            W = O.dequant(q, s, b)
            S = s.view(np.float16).astype(np.float64)
            B = b.view(np.float16).astype(np.float64)
            expect = np.repeat(B, 64, axis=1)
            expect[r, c] = 11 * S[r, c // 64] + B[r, c // 64]
            assert np.array_equal(W, expect), (r, c)


# ---------------------------------------------------------------- router
def test_router_integer_inputs_exact():
    w, L = tiny(d=256, E=16)
    rng = np.random.default_rng(3)
    x = rng.integers(-2, 3, size=(5, w.d)).astype(np.float32)
    got = O.OracleLayer.from_workload(w, L).logits(x)
    acc = x.astype(np.int64) @ L["router_w"].astype(np.int64).T     # exact integer matmul
    scale = L["router_scale"].view(np.float16).astype(np.float64)
    assert np.array_equal(got, acc * scale[None, :])


def test_router_bias_is_added():
    w, L = tiny(d=128, E=8, zipf=1.0)
    x = make_tokens(w, 2)
    got = O.OracleLayer.from_workload(w, L).logits(x)
    L0 = dict(L, router_bias=None)
    base = O.OracleLayer.from_workload(w, L0).logits(x)
    assert np.allclose(got - base, L["router_bias"][None, :].astype(np.float64), atol=1e-12, rtol=0)
    rank = np.round(np.exp(-L["router_bias"].astype(np.float64))).astype(int)
    assert sorted(rank) == list(range(1, w.E + 1))   # b_e = -ln(rank_e), rank a permutation


# ---------------------------------------------------------------- selection
def test_select_brute_force_sort():
    rng = np.random.default_rng(4)
    for _ in range(200):
        E = int(rng.integers(2, 40))
        K = int(rng.integers(1, E + 1))
        l = np.round(rng.standard_normal(E) * 4, 1)  # coarse values: many exact ties
        ids, w, m = O.select(l, K)
        order = sorted(range(E), key=lambda e: (-l[e], e))
        assert list(ids) == sorted(order[:K])
        assert abs(w.sum() - 1) < 1e-12
        p = np.exp(l - l.max())
        p = p / p.sum()
        assert np.allclose(w, p[ids] / p[ids].sum(), rtol=1e-12, atol=0)
        if K < E:
            assert m == l[order[K - 1]] - l[order[K]]
        else:
            assert m == np.inf


def test_select_shift_invariance_and_ties():
    l = np.array([0.5, 2.0, 2.0, -1.0, 2.0])
    ids, w, _ = O.select(l, 2)
    assert list(ids) == [1, 2]          # tie at 2.0 between 1, 2, 4: lower indices win
    ids2, w2, _ = O.select(l + 123.25, 2)
    assert list(ids2) == [1, 2] and np.allclose(w, w2, rtol=1e-12)
    ids, w, _ = O.select(np.zeros(6), 6)
    assert list(ids) == list(range(6)) and np.allclose(w, 1 / 6, rtol=1e-15)


def test_identical_router_rows_tie_to_lower_index():
    w, L = tiny(d=128, E=8, K=1)
    x = make_tokens(w, 1)
    L = dict(L)
    rw = L["router_w"].copy()
    top = np.where(x[0] >= 0, 127, -127).astype(np.int8)   # the largest possible logit
    rw[5] = top
    rw[2] = top
    L["router_w"] = rw
    OL = O.OracleLayer.from_workload(w, L)
    lg = OL.logits(x)[0]
    assert lg[2] == lg[5] == lg.max()
    y, ids, wt, m = OL.forward(x)
    assert ids[0, 0] == 2 and m[0] == 0.0


# ---------------------------------------------------------------- experts / layer
def _expert_closed_form_layer(d=128, f=64):
    """Gate and up are bias-only (scale 0), down is random: with x = e_0,
    g = 40, u = 1/2, so silu(g)*u = 20 and y = 20 * rowsum(W_down)."""
    w, L = tiny(d=d, E=1, K=1, f=f, fs=0)
    L = dict(L)
    for name, val in (("gate", 40.0), ("up", 0.5)):
        L[name + "_s"] = np.zeros_like(L[name + "_s"])
        L[name + "_b"] = np.full_like(L[name + "_b"], f16bits(val))
    return w, L


def test_expert_closed_form_pins_down_orientation():
    w, L = _expert_closed_form_layer()
    x = np.zeros(w.d, np.float32)
    x[0] = 1.0
    out = O.OracleLayer.from_workload(w, L).expert(0, x)
    q = L["down_q"][0]
    nib = np.stack([(q >> np.uint32(4 * k)) & 0xF for k in range(8)], -1).reshape(w.d, w.f).astype(np.int64)
    qsum = nib.reshape(w.d, w.f // 64, 64).sum(-1)            # integer nibble sums per group
    S = L["down_s"][0].view(np.float16).astype(np.float64)
    B = L["down_b"][0].view(np.float16).astype(np.float64)
    rowsum = (S * qsum + 64 * B).sum(-1)
    assert np.allclose(out, 20.0 * rowsum, rtol=1e-13, atol=1e-13)


def test_identical_experts_equal_one_expert():
    w, L = tiny(d=128, E=6, K=3, f=64, fs=64, zipf=1.0)
    L = dict(L)
    for n in ("gate", "up", "down"):
        for p in ("_q", "_s", "_b"):
            L[n + p] = np.repeat(L[n + p][:1], w.E, axis=0)
    x = make_tokens(w, 3)
    OL = O.OracleLayer.from_workload(w, L)
    y, ids, wt, _ = OL.forward(x)
    for t in range(3):
        one = OL.expert(0, x[t]) + OL.expert(-1, x[t])
        assert np.allclose(y[t], one, rtol=1e-12, atol=1e-12)


def test_k_equals_e_uniform_logits_gives_mean():
    w, L = tiny(d=128, E=5, K=5, f=64, fs=64)
    L = dict(L, router_w=np.zeros_like(L["router_w"]), router_bias=None)
    x = make_tokens(w, 2)
    OL = O.OracleLayer.from_workload(w, L)
    y, ids, wt, _ = OL.forward(x)
    assert np.allclose(wt, 1 / 5, rtol=1e-15)
    for t in range(2):
        mean = np.mean([OL.expert(e, x[t]) for e in range(5)], axis=0)
        assert np.allclose(y[t], OL.expert(-1, x[t]) + mean, rtol=1e-12, atol=1e-12)


def test_zero_experts_give_shared_and_zero_shared_gives_routed():
    w, L = tiny(d=128, E=4, K=2, f=64, fs=64)
    x = make_tokens(w, 2)
    Lz = dict(L)
    for n in ("down",):
        Lz[n + "_s"] = np.zeros_like(L[n + "_s"])
        Lz[n + "_b"] = np.zeros_like(L[n + "_b"])
    OL, OZ = O.OracleLayer.from_workload(w, L), O.OracleLayer.from_workload(w, Lz)
    y, *_ = OZ.forward(x)
    for t in range(2):
        assert np.array_equal(y[t], OZ.expert(-1, x[t]))
    Ls = dict(L, sh_down_s=np.zeros_like(L["sh_down_s"]), sh_down_b=np.zeros_like(L["sh_down_b"]))
    ys, ids, wt, _ = O.OracleLayer.from_workload(w, Ls).forward(x)
    for t in range(2):
        routed = sum(wt[t, k] * OL.expert(ids[t, k], x[t]) for k in range(w.K))
        assert np.allclose(ys[t], routed, rtol=1e-12, atol=1e-12)


def test_doubling_down_scale_and_bias_doubles_contribution():
    w, L = tiny(d=128, E=4, K=4, f=64, fs=64)
    x = make_tokens(w, 1)
    OL = O.OracleLayer.from_workload(w, L)
    L2 = dict(L)
    for p in ("down_s", "down_b"):
        a = L[p].view(np.float16).astype(np.float64).copy()
        a[1] *= 2                                   # exact in fp16
        L2[p] = a.astype(np.float16).view(np.uint16)
    y1, ids, wt, _ = OL.forward(x)
    y2, *_ = O.OracleLayer.from_workload(w, L2).forward(x)
    k = list(ids[0]).index(1)
    assert np.allclose(y2[0] - y1[0], wt[0, k] * OL.expert(1, x[0]), rtol=1e-11, atol=1e-12)


def test_forced_set_uses_current_logits():
    w, L = tiny(d=128, E=8, K=2, zipf=1.0)
    x = make_tokens(w, 1)
    OL = O.OracleLayer.from_workload(w, L)
    forced = np.array([[1, 6]], np.int32)
    y, ids, wt, _ = OL.forward(x, forced=forced)
    l = OL.logits(x)[0]
    p = np.exp(l[[1, 6]] - l[[1, 6]].max())
    assert list(ids[0]) == [1, 6] and np.allclose(wt[0], p / p.sum(), rtol=1e-14)
    ref = OL.expert(-1, x[0]) + wt[0, 0] * OL.expert(1, x[0]) + wt[0, 1] * OL.expert(6, x[0])
    assert np.allclose(y[0], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(20))
def test_c_oracle_matches_dense_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    d = 64 * int(rng.integers(1, 4))
    E = int(rng.integers(1, 10))
    K = int(rng.integers(1, E + 1))
    f = 64 * int(rng.integers(1, 3))
    fs = 64 * int(rng.integers(0, 3))
    zipf = None if seed % 2 else 1.0
    w, L = tiny(d=d, E=E, K=K, f=f, fs=fs, zipf=zipf, seed=seed)
    x = make_tokens(w, 3)
    y, ids, wt, _ = O.OracleLayer.from_workload(w, L).forward(x)
    yb, idb, wb = brute.layer(L, K, O.tokens_to_f64(x))
    assert np.array_equal(ids, idb)
    assert np.allclose(wt, wb, rtol=1e-12, atol=1e-15)
    assert np.max(np.abs(y - yb)) <= 1e-12 * max(1.0, np.abs(yb).max())


def test_tiny_workload_matches_brute_force():
    w = WORKLOADS[0]
    L = make_layer(w)
    x = make_tokens(w, w.T)
    y, ids, wt, m = O.OracleLayer.from_workload(w, L).forward(x)
    yb, idb, wb = brute.layer(L, w.K, O.tokens_to_f64(x))
    assert np.array_equal(ids, idb) and np.max(np.abs(y - yb)) < 1e-12


# ---------------------------------------------------------------- grouping
def test_sort_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(50):
        E = int(rng.integers(1, 40))
        K = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(0, 30))
        ids = np.array([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)], np.int32).reshape(T, K)
        counts, offsets, perm, inv = O.sort(ids, E)
        pairs = sorted((ids[t, k], t, k) for t in range(T) for k in range(K))
        assert list(perm) == [t * K + k for _, t, k in pairs]
        assert counts.sum() == T * K and offsets[-1] == T * K and np.all(np.diff(offsets) == counts)
        assert np.array_equal(perm[inv], np.arange(T * K)) if T else True


# ---------------------------------------------------------------- stack glue
def test_rmsnorm_closed_form_and_numpy():
    d = 256
    h = f32_to_bf16_bits(np.full(d, 3.0, np.float32))
    n = O.rmsnorm_bf16(h, 1e-6)   # 3 / sqrt(9 + 1e-6) rounds to 1.0 in bf16
    assert np.all(n == 0x3F80)
    rng = np.random.default_rng(5)
    hv = f32_to_bf16_bits(rng.standard_normal(d).astype(np.float32) * 4)
    hf = (hv.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = hf / np.sqrt(np.mean(hf * hf) + 1e-6)
    got = (O.rmsnorm_bf16(hv).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8)   # within half a bf16 ulp


def test_residual_rounds_once_and_keeps_h():
    """h <- RNE_bf16(h + y) with y in fp64: one rounding of the exact sum.
    y = 2^-8 + 2^-30 on h = 1 lies just above the tie between 1 and 1 + 2^-7,
    so it must round up; rounding y to bf16 first would leave the exact tie
    (2^-30 is far below a bf16 ulp of 2^-8) and give the even 1.0.  A dropped
    h, or a sign error on either term, fails every case."""
    one = np.array([0x3F80], np.uint16)
    assert O.residual_bf16(one, np.array([2.0**-8 + 2.0**-30]))[0] == 0x3F81
    assert O.residual_bf16(one, np.array([2.0**-8]))[0] == 0x3F80          # exact tie -> even
    assert O.residual_bf16(one, np.array([3 * 2.0**-8]))[0] == 0x3F82      # tie -> even (up)
    assert O.residual_bf16(one, np.array([-1.0]))[0] == 0x0000             # y = -h gives +0
    assert O.residual_bf16(one, np.array([0.0]))[0] == 0x3F80              # y = 0 keeps h
    assert O.residual_bf16(np.array([0x4040], np.uint16), np.array([-0.5]))[0] == 0x4020  # 3 - 0.5 = 2.5
    # random cases whose exact sum is representable in fp32: |h| in [2^-3, 2^3)
    # (bf16: lowest bit >= 2^-10) and y a multiple of 2^-16 below 8 in magnitude,
    # so h + y needs at most 20 significant bits; then RNE_bf16 of the fp32 sum
    # (the fp32 -> bf16 route, pinned above) is the only correct answer
    rng = np.random.default_rng(17)
    n = 4096
    hv = rng.uniform(0.125, 8.0, n) * rng.choice([-1.0, 1.0], n)
    h = f32_to_bf16_bits(hv.astype(np.float32))
    y = rng.integers(-(2**19) + 1, 2**19, n).astype(np.float64) * 2.0**-16
    hf = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s32 = (hf + y).astype(np.float32)
    assert np.array_equal(s32.astype(np.float64), hf + y)  # the sums are exact in fp32
    assert np.array_equal(O.residual_bf16(h, y), f32_to_bf16_bits(s32))


def test_stack_step_composes_layers():
    w, L0 = tiny(d=128, E=4, K=2, f=64, fs=64, zipf=1.0, seed=1)
    _, L1 = tiny(d=128, E=4, K=2, f=64, fs=64, zipf=1.0, seed=2)
    layers = [O.OracleLayer.from_workload(w, L0), O.OracleLayer.from_workload(w, L1)]
    h = make_tokens(Workload(91, "t", 128, 4, 2, 64, 64, "bf16", None, 1), 1)[0]
    got, ids = O.stack_step(layers, h)
    ref = h.copy()
    for l in layers:
        n = O.rmsnorm_bf16(ref)
        y, *_ = l.forward(n[None, :])
        ref = O.residual_bf16(ref, y[0])
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- cache policy
def test_lfu_golden_trace():
    rows = []
    for line in open(os.path.join(HERE, "golden", "lfu_trace.txt")):
        line = line.split("#")[0].strip()
        if line:
            rows.append([list(map(int, part.split())) for part in line.split("|")])
    lfu = LfuReplay(4)
    for (step,), chosen, slots, misses in rows:
        got_slots, got_miss = lfu.step(chosen)
        assert got_slots == slots, step
        assert [int(m) for m in got_miss] == misses, step
    assert (lfu.accesses, lfu.hits, lfu.misses, lfu.evictions) == (10, 2, 8, 4)


def test_lfu_prefetch_golden_trace():
    lfu = LfuReplay(4)
    for line in open(os.path.join(HERE, "golden", "lfu_prefetch_trace.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        op, experts, slots, misses = [p.strip() for p in line.split("|")]
        experts, slots = list(map(int, experts.split())), list(map(int, slots.split()))
        if op == "step":
            got_slots, got_miss = lfu.step(experts)
            assert got_slots == slots and [int(m) for m in got_miss] == list(map(int, misses.split())), line
        else:
            placed = lfu.prefetch(experts)
            assert [placed.get(e, -1) for e in experts] == slots, line
    assert (lfu.accesses, lfu.hits, lfu.misses, lfu.evictions, lfu.prefetches, lfu.prefetch_used) == \
        (6, 2, 4, 4, 4, 2)


def _lru_golden_rows():
    rows = []
    for line in open(os.path.join(HERE, "golden", "lru_pool_trace.txt")):
        line = line.split("#")[0].strip()
        if line:
            rows.append([list(map(int, part.split())) for part in line.split("|")])
    return rows


def test_lru_pool_golden_trace():
    pool = LruPoolReplay(4)
    for (step,), (layer,), chosen, slots, misses in _lru_golden_rows():
        got_slots, got_miss = pool.step(layer, chosen)
        assert got_slots == slots, step
        assert [int(m) for m in got_miss] == misses, step
    assert (pool.accesses, pool.hits, pool.misses, pool.evictions) == (13, 4, 9, 5)


@pytest.mark.parametrize("n_slots", [1, 3, 8])
def test_lru_pool_single_expert_calls_follow_stack_distance(n_slots):
    """With one expert per call nothing is protected and the policy is plain
    LRU, so an access misses exactly when its stack distance (distinct keys
    touched since its previous use, infinite on first use) is >= the slot
    count: the inclusion property of LRU (Mattson et al., 1970)."""
    rng = np.random.default_rng(n_slots)
    pool = LruPoolReplay(n_slots)
    history = []
    for step in range(600):
        layer = int(rng.integers(0, 3))
        e = int(min(rng.geometric(0.15), 40))
        key = (layer, e)
        if key in history:
            last = len(history) - 1 - history[::-1].index(key)
            dist = len(set(history[last + 1:]))
        else:
            dist = 10**9
        _, miss = pool.step(layer, [e])
        assert miss[0] == (dist >= n_slots), step
        history.append(key)


def test_prefill_steps_hand_worked():
    """Prefill through the cache, worked by hand: 3 tokens, top-2, 6 experts,
    2 slots, expert 5 cached.  Counts: e0 1, e1 2, e3 1, e4 1, e5 1.  Cached
    first: [5]; then least chosen first, ties to the lower id: 0, 3, 4, then
    1 (count 2).  Steps of 2, ids ascending: [0, 5], [3, 4], [1]."""
    from oracle.lfu import prefill_steps, LfuReplay
    ids = [[1, 5], [0, 1], [3, 4]]
    steps = prefill_steps(ids, 6, 2, cached=[5])
    assert steps == [[0, 5], [3, 4], [1]]
    r = LfuReplay(2)
    r.step([5])  # the state before the chunk
    for g in steps:
        r.step(g)
    # [0, 5]: 5 hits (count 2), 0 fills the empty slot; [3, 4]: both miss and
    # evict 0 and 5 (counts 1 and 2 are not protected: neither is chosen);
    # (4 in slot 0, 3 in slot 1); [1]: 3 and 4 tie on count and tick, so the
    # lower slot goes: the chunk's most chosen expert, 1, stays in the cache
    assert r.hits == 1 and r.misses == 5
    assert r.expert == [1, 3]
