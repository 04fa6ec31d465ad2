"""Stack glue (residual + rmsnorm between layers), the streamed expert cache
and the token->expert grouping, through the C ABI on the GPU."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, Workload, make_layer, make_tokens, make_reuse_coins
from oracle import oracle as O
from oracle.lfu import LfuReplay, LruPoolReplay, prefill_steps
from tests.helpers import GpuLayer, to_device, to_host, torch_mod

pytestmark = pytest.mark.gpu


def _bf16_ulp(v):
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0**-126)))
    return 2.0 ** (e - 7)


def _stack_layers(w, n, seed0=0):
    arrays = [make_layer(w, layer=l, seed=seed0) for l in range(n)]
    gls = [GpuLayer(w, a, 1) for a in arrays]
    ols = [O.OracleLayer.from_workload(w, a) for a in arrays]
    return arrays, gls, ols


SMALL = Workload(85, "stack-small", d=512, E=64, K=8, f=128, fs=256, act="bf16", zipf=1.0, T=1,
                 layers=4, steps=6, noise_sd=0.1)


@pytest.mark.parametrize("w", [SMALL, Workload(86, "stack-d2816", d=2816, E=128, K=8, f=704, fs=2112,
                                                act="bf16", zipf=1.0, T=1, layers=3, steps=2, noise_sd=0.1)],
                         ids=["small", "decode-shape"])
def test_stack_teacher_forced_and_composed(w):
    torch = torch_mod()
    arrays, gls, ols = _stack_layers(w, w.layers)
    stack = M.moe_stack_create([g.handle for g in gls], 1e-6)
    singles = [M.moe_stack_create([g.handle], 1e-6) for g in gls]
    h0 = make_tokens(w, 1, stream=21)
    # whole stack in one call
    h = to_device(h0)
    ids_all = torch.empty((w.layers, 1, w.K), dtype=torch.int32, device="cuda")
    M.moe_stack_forward(h, stack, 1, ids_out=ids_all)
    torch.cuda.synchronize()
    h_stack = to_host(h)
    # layer by layer, checking each layer against the oracle on the GPU's own input
    hl = to_device(h0)
    for l in range(w.layers):
        h_in = to_host(hl)
        M.moe_stack_forward(hl, singles[l], 1)
        torch.cuda.synchronize()
        h_out = to_host(hl)[0]
        n = O.rmsnorm_bf16(h_in[0])
        y_ref, ids_ref, _, margin = ols[l].forward(n[None, :])
        ref = O.residual_bf16(h_in[0], y_ref[0])
        got, want = O.tokens_to_f64(h_out), O.tokens_to_f64(ref)
        ynorm = np.linalg.norm(y_ref[0])
        slack = np.linalg.norm(_bf16_ulp(want))
        assert np.linalg.norm(got - want) <= 5e-3 * ynorm + slack, f"layer {l}"
    assert np.array_equal(h_stack, to_host(hl)), "a stack must equal its layers applied one by one"
    for s in singles:
        M.moe_stack_destroy(s)
    M.moe_stack_destroy(stack)
    for g in gls:
        g.close()


def test_stack_reuse_mask_reuses_previous_sets():
    torch = torch_mod()
    w = SMALL
    arrays, gls, ols = _stack_layers(w, 2, seed0=3)
    stack = M.moe_stack_create([g.handle for g in gls], 1e-6)
    h = to_device(make_tokens(w, 1, stream=22))
    ids1 = torch.empty((2, 1, w.K), dtype=torch.int32, device="cuda")
    ids2 = torch.empty_like(ids1)
    M.moe_stack_forward(h, stack, 1, ids_out=ids1)
    M.moe_stack_forward(h, stack, 1, reuse_mask=[1, 0], ids_out=ids2)
    torch.cuda.synchronize()
    assert np.array_equal(ids1.cpu().numpy()[0], ids2.cpu().numpy()[0])
    M.moe_stack_destroy(stack)


CACHE_W = Workload(87, "cache", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=1,
                   layers=1, steps=60, reuse_p=0.6, slots=16)


@pytest.mark.parametrize("w", [CACHE_W, Workload(88, "cache-d2048-e256", d=2048, E=256, K=8, f=512, fs=512,
                                                  act="bf16", zipf=1.1, T=1, layers=1, steps=40,
                                                  reuse_p=0.6, slots=16)],
                         ids=["small", "stream-shape"])
def test_streamed_layer_bit_identical_and_counters_replay(w):
    torch = torch_mod()
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 1)
    st = GpuLayer(w, arrays, 1, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    _, stride = M.moe_layer_bytes(st.handle)
    x = make_tokens(w, w.steps, stream=23)
    coins = make_reuse_coins(w, w.steps)[:, 0]
    replay = LfuReplay(w.slots)
    for t in range(w.steps):
        reuse = bool(coins[t])
        y_r, ids_r, w_r = res.forward(x[t:t + 1], path=M.MOE_PATH_DECODE, reuse=reuse)
        y_s, ids_s, w_s = st.forward(x[t:t + 1], path=M.MOE_PATH_DECODE, reuse=reuse)
        assert np.array_equal(y_r, y_s), f"step {t}: streamed output differs from resident"
        assert np.array_equal(ids_r, ids_s) and np.array_equal(w_r, w_s)
        replay.step(ids_s[0].tolist())
    stats = M.moe_cache_stats_get(st.handle)
    assert (stats["accesses"], stats["hits"], stats["misses"], stats["evictions"]) == \
        (replay.accesses, replay.hits, replay.misses, replay.evictions)
    assert stats["h2d_bytes"] == replay.misses * stride
    experts, counts = M.moe_cache_contents(st.handle, w.slots)
    assert list(experts) == replay.expert and list(counts) == replay.count
    # every hit of a one-token call was computed by the kernels queued before
    # the cache step
    assert stats["ahead_slots"] == replay.hits
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


def test_streamed_reuse_follows_the_stored_sets():
    """A one-token call of a streamed layer that reuses the previous sets does
    its cache step from the host's copy of the routing, without waiting for
    its kernels.  The stored sets are the last routing of the layer, also a
    route-only call's (moe_layer_route): after one, a reusing call must take
    that call's sets, like the resident layer, and run bit-identical to it."""
    torch = torch_mod()
    w = CACHE_W
    arrays = make_layer(w, seed=9)
    res = GpuLayer(w, arrays, 1)
    st = GpuLayer(w, arrays, 1, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    x = make_tokens(w, 6, stream=41)
    calls = [("fwd", False), ("fwd", True), ("fwd", True), ("route", None), ("fwd", True), ("fwd", False),
             ("fwd", True)]
    routed = None
    for i, (kind, reuse) in enumerate(calls):
        xi = x[i % 6:i % 6 + 1]
        if kind == "route":
            xd = to_device(xi)
            for g in (res, st):
                ids = torch.empty((1, w.K), dtype=torch.int32, device="cuda")
                wts = torch.empty((1, w.K), dtype=torch.float32, device="cuda")
                M.moe_layer_route(xd, g.handle, ids, wts, 1)
            torch.cuda.synchronize()
            routed = ids.cpu().numpy()
            continue
        y_r, ids_r, w_r = res.forward(xi, path=M.MOE_PATH_DECODE, reuse=reuse)
        y_s, ids_s, w_s = st.forward(xi, path=M.MOE_PATH_DECODE, reuse=reuse)
        assert np.array_equal(y_r, y_s) and np.array_equal(ids_r, ids_s), f"call {i}"
        if i == 4:
            assert np.array_equal(ids_s, routed), "a reusing call after a route-only call takes its sets"
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


def test_streamed_hits_at_once_misses_after_their_fill():
    """Forced routings whose calls mix hits and misses in every proportion
    (0 to K misses, repeated ids in a call): the hits of a one-token call are
    computed by kernels queued before its cache step, its misses after the
    fill kernel, then the down kernel.  Outputs stay bit-identical to the
    resident layer, the cache follows the replay, and the slots computed ahead
    are exactly the slots whose experts were hits."""
    w = CACHE_W
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 1)
    st = GpuLayer(w, arrays, 1, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    x = make_tokens(w, 48, stream=37)
    rng = np.random.default_rng(41)
    replay = LfuReplay(w.slots)
    want_ahead = 0
    plans = [list(range(8)), [0, 1, 2, 3, 4, 5, 8, 9], [0, 1, 2, 3, 4, 5, 6, 10], [1, 1, 2, 3, 11, 11, 12, 4],
             list(range(20, 28))]
    for t in range(48):
        cached = [e for e in replay.expert if e >= 0]
        if t < len(plans):
            ids = plans[t]
        else:  # n_miss of the K slots from experts not cached, the rest from the cache
            n_miss = int(rng.integers(0, w.K + 1)) if len(cached) >= w.K else w.K
            absent = [e for e in range(w.E) if e not in cached]
            ids = list(rng.choice(absent, n_miss, replace=False)) + list(rng.choice(cached, w.K - n_miss,
                                                                                    replace=False))
            rng.shuffle(ids)
        forced = np.array([ids], np.int32)
        y_r, ids_r, w_r = res.forward(x[t:t + 1], path=M.MOE_PATH_DECODE, forced=forced)
        y_s, ids_s, w_s = st.forward(x[t:t + 1], path=M.MOE_PATH_DECODE, forced=forced)
        assert np.array_equal(y_r, y_s), f"call {t} (routing {ids}) differs from resident"
        assert np.array_equal(ids_r, ids_s) and np.array_equal(w_r, w_s)
        want_ahead += sum(1 for e in ids if e in cached)
        replay.step(sorted(set(int(e) for e in ids)))
    stats = M.moe_cache_stats_get(st.handle)
    assert (stats["accesses"], stats["hits"], stats["misses"], stats["evictions"]) == \
        (replay.accesses, replay.hits, replay.misses, replay.evictions)
    assert replay.evictions > 0 and replay.hits > 0
    assert stats["ahead_slots"] == want_ahead
    assert stats["h2d_ns"] > 0
    experts, counts = M.moe_cache_contents(st.handle, w.slots)
    assert list(experts) == replay.expert and list(counts) == replay.count
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


def test_streamed_one_and_two_token_calls_interleave():
    """One-token calls hand the routing over through host memory and launch
    their expert kernels ahead; two-token calls copy and synchronise.  Mixed
    on one layer they stay bit-identical to a resident layer, and the cache
    follows the replay of the calls' chosen sets."""
    w = CACHE_W
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 2)
    st = GpuLayer(w, arrays, 2, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    x = make_tokens(w, 40, stream=31)
    replay = LfuReplay(w.slots)
    i = 0
    for T in [1, 2, 1, 1, 2, 2, 1, 2, 1, 1, 2, 1] * 2:
        y_r, ids_r, w_r = res.forward(x[i:i + T], path=M.MOE_PATH_DECODE)
        y_s, ids_s, w_s = st.forward(x[i:i + T], path=M.MOE_PATH_DECODE)
        assert np.array_equal(y_r, y_s), f"call at token {i} (T={T}) differs from resident"
        assert np.array_equal(ids_r, ids_s) and np.array_equal(w_r, w_s)
        replay.step(sorted(set(int(e) for e in ids_s.flatten())))
        i += T
    stats = M.moe_cache_stats_get(st.handle)
    assert (stats["accesses"], stats["hits"], stats["misses"], stats["evictions"]) == \
        (replay.accesses, replay.hits, replay.misses, replay.evictions)
    assert replay.misses > 0 and replay.hits > 0
    experts, counts = M.moe_cache_contents(st.handle, w.slots)
    assert list(experts) == replay.expert and list(counts) == replay.count
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


def test_streamed_prefill_goes_through_the_cache():
    """Prefill of a streamed layer runs the chunk's experts through the LFU
    cache group by group: outputs bit-identical to the resident prefill, cache
    state equal to the replay of the groups, and one-token calls afterwards
    still match."""
    w = Workload(89, "prefill-cache", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=96,
                 layers=1, steps=1, slots=16)
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 256)
    st = GpuLayer(w, arrays, 256, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    _, stride = M.moe_layer_bytes(st.handle)
    x = make_tokens(w, 96 + 130 + 2, stream=41)
    replay = LfuReplay(w.slots)
    for lo, hi in ((0, 96), (96, 226)):  # one chunk, then 130 tokens (chunks of 128 and 2)
        y_r, ids_r, w_r = res.forward(x[lo:hi], path=M.MOE_PATH_PREFILL)
        y_s, ids_s, w_s = st.forward(x[lo:hi], path=M.MOE_PATH_PREFILL)
        assert np.array_equal(y_r, y_s), f"prefill of tokens {lo}..{hi} differs from resident"
        assert np.array_equal(ids_r, ids_s) and np.array_equal(w_r, w_s)
        for c0 in range(0, hi - lo, 128):
            for g in prefill_steps(ids_s[c0:c0 + 128], w.E, w.slots, [e for e in replay.expert if e >= 0]):
                replay.step(g)
    stats = M.moe_cache_stats_get(st.handle)
    assert (stats["accesses"], stats["hits"], stats["misses"], stats["evictions"]) == \
        (replay.accesses, replay.hits, replay.misses, replay.evictions)
    assert stats["h2d_bytes"] == replay.misses * stride
    experts, counts = M.moe_cache_contents(st.handle, w.slots)
    assert list(experts) == replay.expert and list(counts) == replay.count
    assert replay.hits > 0  # the second call's chunks start with what the cache holds
    for t in (226, 227):  # decode after prefill, on the warmed cache
        y_r, _, _ = res.forward(x[t:t + 1], path=M.MOE_PATH_DECODE)
        y_s, ids_s, _ = st.forward(x[t:t + 1], path=M.MOE_PATH_DECODE)
        assert np.array_equal(y_r, y_s)
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


def test_streamed_stack_equals_resident_stack_on_the_same_path():
    """A stack of streamed layers (16-slot LFU caches, fills on a side stream)
    ends in exactly the state of the same stack with every expert resident,
    both on the split kernels, over steps with forced reuse."""
    torch = torch_mod()
    w = Workload(91, "stream-stack-small", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=1,
                 layers=3, steps=12, reuse_p=0.6, slots=16, noise_sd=0.1)
    arrays = [make_layer(w, layer=l, seed=7) for l in range(w.layers)]
    res = [GpuLayer(w, a, 1) for a in arrays]
    st = [GpuLayer(w, a, 1, residency=M.MOE_STREAMED) for a in arrays]
    for g in res:
        M.moe_layer_set_default_path(g.handle, M.MOE_PATH_DECODE)
    for g in st:
        M.moe_cache_attach(g.handle, w.slots)
    coins = make_reuse_coins(w, w.steps).astype(np.uint8)
    finals = []
    for layers in (res, st):
        stack = M.moe_stack_create([g.handle for g in layers], 1e-6)
        h = to_device(make_tokens(w, 1, stream=26))
        for t in range(w.steps):
            M.moe_stack_forward(h, stack, 1, reuse_mask=coins[t])
        torch.cuda.synchronize()
        finals.append(to_host(h))
        M.moe_stack_destroy(stack)
    assert np.array_equal(finals[0], finals[1]), "streamed stack differs from the resident stack"
    assert sum(M.moe_cache_stats_get(g.handle)["misses"] for g in st) > 0, "no fills happened"
    with pytest.raises(M.MoeError):
        M.moe_layer_set_default_path(res[0].handle, 7)
    for g in res + st:
        g.close()


def test_stack_prefetch_equals_resident_and_replays():
    """Fetch-ahead in a streamed stack (each layer prefetches the next
    layer's historically most chosen absent experts): outputs stay exactly the
    resident stack's, and every layer's counters, prefetches included, equal
    the oracle replay with the same predictor on the recorded routing."""
    torch = torch_mod()
    w = Workload(93, "prefetch-stack-small", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=1,
                 layers=3, steps=16, reuse_p=0.6, slots=16, noise_sd=0.1)
    depth = 6
    arrays = [make_layer(w, layer=l, seed=11) for l in range(w.layers)]
    res = [GpuLayer(w, a, 1) for a in arrays]
    st = [GpuLayer(w, a, 1, residency=M.MOE_STREAMED) for a in arrays]
    for g in res:
        M.moe_layer_set_default_path(g.handle, M.MOE_PATH_DECODE)
    for g in st:
        M.moe_cache_attach(g.handle, w.slots)
    _, eb = M.moe_layer_bytes(st[0].handle)
    coins = make_reuse_coins(w, w.steps).astype(np.uint8)
    xs = make_tokens(w, w.steps, stream=29)  # a fresh token every step: misses to predict
    s_res = M.moe_stack_create([g.handle for g in res], 1e-6)
    s_st = M.moe_stack_create([g.handle for g in st], 1e-6)
    M.moe_stack_set_prefetch(s_st, depth)
    ref = [LfuReplay(w.slots) for _ in range(w.layers)]
    hist = np.zeros((w.layers, w.E), np.int64)

    def guess(l):
        cand = [e for e in range(w.E) if hist[l][e] > 0 and e not in ref[l].expert]
        return sorted(cand, key=lambda e: (-hist[l][e], e))[:depth]

    ids = torch.empty((w.layers, 1, w.K), dtype=torch.int32, device="cuda")
    for t in range(w.steps):
        ha, hb = to_device(xs[t:t + 1]), to_device(xs[t:t + 1])
        M.moe_stack_forward(ha, s_res, 1, reuse_mask=coins[t])
        M.moe_stack_forward(hb, s_st, 1, reuse_mask=coins[t], ids_out=ids)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ha), to_host(hb)), f"step {t}: streamed with prefetch differs"
        for l, row in enumerate(ids.cpu().numpy()[:, 0]):
            chosen = sorted(set(row.tolist()))
            ref[l].step(chosen)
            hist[l][chosen] += 1
            if l + 1 < w.layers:
                ref[l + 1].prefetch(guess(l + 1))
    used = 0
    for g, r in zip(st, ref):
        s = M.moe_cache_stats_get(g.handle)
        assert (s["accesses"], s["hits"], s["misses"], s["evictions"], s["prefetches"], s["prefetch_used"]) == \
            (r.accesses, r.hits, r.misses, r.evictions, r.prefetches, r.prefetch_used)
        assert s["h2d_bytes"] == (r.misses + r.prefetches) * eb
        used += r.prefetch_used
    assert used > 0, "no prefetch was ever used"
    with pytest.raises(M.MoeError):
        M.moe_stack_set_prefetch(s_st, 65)
    M.moe_stack_destroy(s_res)
    M.moe_stack_destroy(s_st)
    for g in res + st:
        assert M.moe_layer_check_errors(g.handle) == 0
        g.close()


def test_pooled_lru_stack_equals_resident_and_replays():
    """Three streamed layers share one LRU pool smaller than their combined
    working sets: the stack ends in exactly the resident stack's state (same
    split kernels), the pool's contents and counters equal the oracle's
    replay of the recorded routing, and the layers can then be detached and
    given per-layer caches."""
    torch = torch_mod()
    w = Workload(92, "pool-stack-small", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=1,
                 layers=3, steps=14, reuse_p=0.6, slots=16, noise_sd=0.1)
    arrays = [make_layer(w, layer=l, seed=9) for l in range(w.layers)]
    res = [GpuLayer(w, a, 1) for a in arrays]
    st = [GpuLayer(w, a, 1, residency=M.MOE_STREAMED) for a in arrays]
    for g in res:
        M.moe_layer_set_default_path(g.handle, M.MOE_PATH_DECODE)
    _, eb = M.moe_layer_bytes(st[0].handle)
    n_slots = 20
    pool = M.moe_cache_pool_create(n_slots * eb + eb // 2, eb)  # the budget's remainder holds no expert
    for g in st:
        M.moe_cache_attach_pool(g.handle, pool)
    coins = make_reuse_coins(w, w.steps).astype(np.uint8)
    replay = LruPoolReplay(n_slots)
    finals = []
    for layers in (res, st):
        stack = M.moe_stack_create([g.handle for g in layers], 1e-6)
        h = to_device(make_tokens(w, 1, stream=27))
        ids = torch.empty((w.layers, 1, w.K), dtype=torch.int32, device="cuda")
        for t in range(w.steps):
            M.moe_stack_forward(h, stack, 1, reuse_mask=coins[t], ids_out=ids)
            if layers is st:
                for l, row in enumerate(ids.cpu().numpy()[:, 0]):
                    replay.step(l, sorted(set(row.tolist())))
        torch.cuda.synchronize()
        finals.append(to_host(h))
        M.moe_stack_destroy(stack)
    assert np.array_equal(finals[0], finals[1]), "pooled streamed stack differs from the resident stack"
    tot = M.moe_cache_pool_stats(pool)
    assert (tot["accesses"], tot["hits"], tot["misses"], tot["evictions"]) == \
        (replay.accesses, replay.hits, replay.misses, replay.evictions)
    assert replay.evictions > 0, "the pool never filled up"
    assert tot["h2d_bytes"] == replay.misses * eb
    per = [M.moe_cache_stats_get(g.handle) for g in st]
    assert sum(p["misses"] for p in per) == replay.misses
    lay, exp = M.moe_cache_pool_contents(pool, n_slots)
    want = [k if k is not None else (-1, -1) for k in replay.key]
    assert [(int(a), int(b)) for a, b in zip(lay, exp)] == want
    with pytest.raises(M.MoeError):
        M.moe_cache_attach(st[0].handle, 16)  # already cached by the pool
    for g in st:
        M.moe_cache_detach(g.handle)
        M.moe_cache_attach(g.handle, 16)
    y_r, _, _ = res[0].forward(make_tokens(w, 1, stream=28), path=M.MOE_PATH_DECODE)
    y_s, _, _ = st[0].forward(make_tokens(w, 1, stream=28), path=M.MOE_PATH_DECODE)
    assert np.array_equal(y_r, y_s)
    M.moe_cache_pool_destroy(pool)
    for g in res + st:
        assert M.moe_layer_check_errors(g.handle) == 0
        g.close()


def test_streamed_fault_injection_leaves_state_unchanged():
    w = CACHE_W
    arrays = make_layer(w)
    st = GpuLayer(w, arrays, 1, residency=M.MOE_STREAMED)
    with pytest.raises(M.MoeError) as ei:
        st.forward(make_tokens(w, 1, stream=24), path=M.MOE_PATH_DECODE)
    assert ei.value.status == M.MOE_ERR_STATE  # no cache attached yet
    M.moe_cache_attach(st.handle, w.slots)
    x = make_tokens(w, 3, stream=25)
    _, ids, _ = st.forward(x[:1], path=M.MOE_PATH_DECODE)
    before = M.moe_cache_contents(st.handle, w.slots)
    stats0 = M.moe_cache_stats_get(st.handle)
    # make every expert that is not cached unreadable, then route a fresh token
    cached = set(int(e) for e in before[0] if e >= 0)
    for e in range(w.E):
        if e not in cached:
            M.moe_cache_fail_expert(st.handle, e, True)
    with pytest.raises(M.MoeError) as ei:
        st.forward(x[1:2], path=M.MOE_PATH_DECODE, forced=np.array([[e for e in range(w.E) if e not in cached][:w.K]]))
    assert ei.value.status == M.MOE_ERR_IO
    after = M.moe_cache_contents(st.handle, w.slots)
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    assert M.moe_cache_stats_get(st.handle)["misses"] == stats0["misses"]
    for e in range(w.E):
        M.moe_cache_fail_expert(st.handle, e, False)
    y_s, _, _ = st.forward(x[2:3], path=M.MOE_PATH_DECODE)  # recovers
    res = GpuLayer(w, arrays, 1)
    y_r, _, _ = res.forward(x[2:3], path=M.MOE_PATH_DECODE)
    assert np.array_equal(y_r, y_s)
    # the failed call's kernels queued before the cache step found no chosen
    # expert in the table: they computed nothing and raised no flag
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


@pytest.mark.parametrize("T", [0, 1, 37, 128, 512])
def test_sort_bit_exact(T):
    torch = torch_mod()
    w = WORKLOADS[3]
    wl = Workload(89, "sort", d=256, E=w.E, K=w.K, f=64, fs=64, act="bf16", zipf=1.0, T=max(T, 1))
    gl = GpuLayer(wl, make_layer(wl), max(T, 1))
    rng = np.random.default_rng(T)
    ids = np.array([np.sort(rng.choice(wl.E, wl.K, replace=False)) for _ in range(T)], np.int32).reshape(T, wl.K)
    di = torch.from_numpy(ids).cuda() if T else torch.zeros((1, wl.K), dtype=torch.int32, device="cuda")
    counts = torch.empty(wl.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(wl.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(max(T, 1) * wl.K, dtype=torch.int32, device="cuda")
    inv = torch.empty_like(perm)
    M.moe_layer_sort(di, gl.handle, T, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    c, o, p, iv = O.sort(ids, wl.E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy()[:T * wl.K], p)
    assert np.array_equal(inv.cpu().numpy()[:T * wl.K], iv)
    gl.close()


def test_decode_stack30_trajectory_teacher_forced():
    """The 30-layer decode stack (d_model 2816, 128 experts, top-8, all
    weights resident) driven for 16 steps of its recurrence, next input =
    output + N(0, 0.1): every step of the production call equals its layers
    run one by one, and nine sampled (step, layer) pairs, first and last
    layer included, match the oracle on the GPU's own input."""
    from gen.workloads import make_noise
    from tests.helpers import check_stack_layer
    torch = torch_mod()
    w = WORKLOADS[2]
    steps = 16
    pairs = {(0, 0), (1, 29), (3, 7), (5, 14), (8, 21), (10, 3), (13, 26), (15, 11), (15, 29)}
    keep = {l for _, l in pairs}
    gls, ols = [], {}
    for l in range(w.layers):
        arrays = make_layer(w, layer=l)
        gls.append(GpuLayer(w, arrays, 1))
        if l in keep:
            ols[l] = O.OracleLayer.from_workload(w, arrays)
        del arrays
    stack = M.moe_stack_create([g.handle for g in gls], 1e-6)
    singles = [M.moe_stack_create([g.handle], 1e-6) for g in gls]
    noise = torch.from_numpy(make_noise(w, steps)).cuda()
    h = to_device(make_tokens(w, 1, stream=5))
    hs = h.clone()
    ids = torch.empty((1, 1, w.K), dtype=torch.int32, device="cuda")
    checked = 0
    for t in range(steps):
        M.moe_stack_forward(h, stack, 1)
        for l in range(w.layers):
            if (t, l) in pairs:
                torch.cuda.synchronize()
                h_in = to_host(hs)[0]
                M.moe_stack_forward(hs, singles[l], 1, ids_out=ids)
                torch.cuda.synchronize()
                rel = check_stack_layer(ols[l], w.K, h_in, to_host(hs)[0], ids.cpu().numpy())
                print(f"step {t} layer {l}: rel err {rel:.3e}")
                checked += 1
            else:
                M.moe_stack_forward(hs, singles[l], 1)
        torch.cuda.synchronize()
        assert torch.equal(h, hs), f"step {t}: the stack call differs from its layers"
        h.copy_((h.float() + noise[t]).to(torch.bfloat16))
        hs.copy_(h)
    assert checked == len(pairs)
    assert bool(torch.isfinite(h.float()).all())
    for g in gls:
        assert M.moe_layer_check_errors(g.handle) == 0
    for s in singles:
        M.moe_stack_destroy(s)
    M.moe_stack_destroy(stack)
    for g in gls:
        g.close()
