"""Checks of the device weight layout, the error flags and host-side
fallbacks, and stacks of layers with different shapes, through the C ABI on
the GPU."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import Workload, f32_to_bf16_bits, make_layer, make_tokens
from oracle import oracle as O
from oracle.lfu import LfuReplay
from tests.helpers import GpuLayer, check_layer, check_stack_layer, to_device, to_host, torch_mod

pytestmark = pytest.mark.gpu

LAYOUT_W = Workload(70, "layout", d=256, E=4, K=2, f=128, fs=192, act="bf16", zipf=None, T=1)


def _f16(a):
    return a.view(np.float16).astype(np.float64)


def _patterned_layout_arrays():
    """Expert 1's gate holds q = 8 everywhere; row r < 8 of expert 2's up holds
    a single nonzero nibble (11) at column ONE_HOT[r], all others 0."""
    w = LAYOUT_W
    arrays = make_layer(w)
    gq = arrays["gate_q"].copy()
    gq[1] = 0x88888888
    uq = arrays["up_q"].copy()
    uq[2] = 0
    for r, c in enumerate(ONE_HOT):
        uq[2, r, c // 8] = np.uint32(0xB) << np.uint32(4 * (c % 8))
    arrays["gate_q"], arrays["up_q"] = gq, uq
    return arrays


ONE_HOT = (0, 1, 7, 8, 63, 64, 100, 255)


@pytest.mark.parametrize("residency", [M.MOE_RESIDENT, M.MOE_STREAMED], ids=["resident", "streamed"])
def test_device_layout_dequantises_to_the_canonical_weights(residency):
    """The GPU reads every weight of the device repack back through the GEMV
    kernels' addressing: fma(scale, q, bias) in fp32 is the fp32 rounding of
    the exact affine weight, so it must equal the fp64 dequantisation rounded
    once to fp32, element for element."""
    w = LAYOUT_W
    arrays = _patterned_layout_arrays()
    gl = GpuLayer(w, arrays, 1, residency=residency)
    mats = (("gate", w.f, w.d), ("up", w.f, w.d), ("down", w.d, w.f))
    for which, (name, rows, cols) in enumerate(mats):
        for e in (-1, 0, 1, 2, w.E - 1):
            pre = "sh_" if e < 0 else ""
            srows = (w.fs if name != "down" else w.d) if e < 0 else rows
            scols = (w.fs if name == "down" else w.d) if e < 0 else cols
            q, s, b = (arrays[pre + name + "_" + k] for k in "qsb")
            if e >= 0:
                q, s, b = q[e], s[e], b[e]
            got = M.moe_debug_dequant(gl.handle, which, e, srows, scols)
            assert np.array_equal(got, O.dequant(q, s, b).astype(np.float32)), (name, e)
    # closed forms, independent of the oracle
    S, B = _f16(arrays["gate_s"][1]), _f16(arrays["gate_b"][1])
    got = M.moe_debug_dequant(gl.handle, 0, 1, w.f, w.d)
    assert np.array_equal(got, np.repeat(8.0 * S + B, 64, axis=1).astype(np.float32))  # all-q = 8 -> 8 s + b
    S, B = _f16(arrays["up_s"][2]), _f16(arrays["up_b"][2])
    got = M.moe_debug_dequant(gl.handle, 1, 2, w.f, w.d)
    expect = np.repeat(B, 64, axis=1)
    for r, c in enumerate(ONE_HOT):
        expect[r, c] = 11.0 * S[r, c // 64] + B[r, c // 64]
    assert np.array_equal(got, expect.astype(np.float32))
    gl.close()


RANGE_W = Workload(71, "range", d=512, E=16, K=2, f=128, fs=128, act="bf16", zipf=1.0, T=16)


def test_fp16_handoff_range_is_flagged():
    """Tokens scaled by 1000 drive |silu(g) u| far past 65504: the decode and
    fused paths (fp16 hand-off of the activations) must raise bit 3; the
    prefill path keeps them in bf16, so it still matches the oracle, unflagged."""
    w = RANGE_W
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 16)
    OL = O.OracleLayer.from_workload(w, arrays)
    x = make_tokens(w, 16, stream=40)
    big = f32_to_bf16_bits(O.tokens_to_f64(x).astype(np.float32) * np.float32(1000.0))
    gl.forward(x[:1], path=M.MOE_PATH_FUSED)
    gl.forward(x, path=M.MOE_PATH_DECODE)
    assert M.moe_layer_check_errors(gl.handle) == 0
    gl.forward(big[:1], path=M.MOE_PATH_FUSED)
    assert M.moe_layer_check_errors(gl.handle) & 8
    gl.forward(big, path=M.MOE_PATH_DECODE)
    assert M.moe_layer_check_errors(gl.handle) & 8
    y, ids, wt = gl.forward(big, path=M.MOE_PATH_PREFILL)
    assert M.moe_layer_check_errors(gl.handle) == 0
    check_layer(gl, OL, big, y, ids, wt)
    gl.close()


FALLBACK_W = Workload(72, "fallback", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.1, T=1,
                      steps=24, reuse_p=0.6, slots=16)


def test_streamed_call_without_host_spin_matches_resident():
    """A streamed one-token call whose host spin for the routing runs out at
    once falls back to waiting for the stream (which then also holds its hits,
    computed by the kernels queued before the cache step); its misses still
    run after their fill, so every call equals the resident layer bit for
    bit, flags stay clear and the counters replay."""
    w = FALLBACK_W
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 1)
    st = GpuLayer(w, arrays, 1, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    M.moe_debug_host_wait(st.handle, 0)
    x = make_tokens(w, w.steps, stream=41)
    replay = LfuReplay(w.slots)
    for t in range(w.steps):
        y_r, ids_r, w_r = res.forward(x[t:t + 1], path=M.MOE_PATH_DECODE)
        y_s, ids_s, w_s = st.forward(x[t:t + 1], path=M.MOE_PATH_DECODE)
        assert np.array_equal(y_r, y_s), t
        assert np.array_equal(ids_r, ids_s) and np.array_equal(w_r, w_s)
        replay.step(ids_s[0].tolist())
    stats = M.moe_cache_stats_get(st.handle)
    assert (stats["accesses"], stats["hits"], stats["misses"]) == (replay.accesses, replay.hits, replay.misses)
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()


MIXED = [Workload(73, "mix-a", d=512, E=64, K=8, f=128, fs=256, act="bf16", zipf=1.0, T=1),
         Workload(74, "mix-b", d=512, E=32, K=4, f=192, fs=128, act="bf16", zipf=1.0, T=1),
         Workload(75, "mix-c", d=512, E=16, K=2, f=64, fs=0, act="bf16", zipf=None, T=1)]


def test_stack_of_mixed_shapes_equals_its_layers():
    """A stack whose layers differ in experts, top-K, d_ff and shared d_ff
    (shapes a, b, a, c, b): the fused launches of each shape keep their own
    counters, so the stack equals its layers run one by one, every layer
    matches the oracle on its own input, and no wait runs out."""
    torch = torch_mod()
    order = [0, 1, 0, 2, 1]
    ws = [MIXED[i] for i in order]
    arrays = [make_layer(w, layer=l) for l, w in enumerate(ws)]
    gls = [GpuLayer(w, a, 1) for w, a in zip(ws, arrays)]
    ols = [O.OracleLayer.from_workload(w, a) for w, a in zip(ws, arrays)]
    stack = M.moe_stack_create([g.handle for g in gls], 1e-6)
    singles = [M.moe_stack_create([g.handle], 1e-6) for g in gls]
    h = to_device(make_tokens(ws[0], 1, stream=42))
    hs = h.clone()
    for step in range(3):
        M.moe_stack_forward(h, stack, 1)
        for l, g in enumerate(gls):
            h_in = to_host(hs)[0]
            ids = torch.empty((1, 1, ws[l].K), dtype=torch.int32, device="cuda")
            M.moe_stack_forward(hs, singles[l], 1, ids_out=ids)
            torch.cuda.synchronize()
            check_stack_layer(ols[l], ws[l].K, h_in, to_host(hs)[0], ids.cpu().numpy())
        torch.cuda.synchronize()
        assert torch.equal(h, hs), step
    for g in gls:
        assert M.moe_layer_check_errors(g.handle) == 0
    for s in singles:
        M.moe_stack_destroy(s)
    M.moe_stack_destroy(stack)
    for g in gls:
        g.close()
