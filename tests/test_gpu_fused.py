"""Single-launch decode kernel: parity with the fp64 oracle, agreement with
the three-kernel decode path (same routing bit for bit; outputs equal up to
the fp32 summation order of the down projection, which the fused kernel
takes phase by phase), repeated launches and graph replays (its
cross-workgroup counters need no reset), and the cases it must refuse."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, Workload, f32_to_bf16_bits, make_layer, make_tokens
from oracle import oracle as O
from tests.helpers import GpuLayer, check_layer, empty_like_act, to_device, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def decode_layer():
    w = WORKLOADS[1]
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 4)
    yield w, gl, O.OracleLayer.from_workload(w, arrays)
    gl.close()


def _agree(fused, split):
    """Identical expert sets and weights; outputs within a few bf16 ulps plus
    the fused kernel's rounding of the intermediate activations to 9
    mantissa bits (its tenth bit tags the launch), about 4e-3 of the rms."""
    assert np.array_equal(fused[1], split[1])
    assert np.array_equal(fused[2], split[2])
    yf, ys = O.tokens_to_f64(fused[0]), O.tokens_to_f64(split[0])
    rms = np.sqrt(np.mean(ys * ys, axis=-1, keepdims=True))
    assert np.all(np.abs(yf - ys) <= 2.0 ** -7 * np.abs(ys) + 4e-3 * rms), np.abs(yf - ys).max()


def test_fused_decode_layer_tokens(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 16, stream=21)
    worst = 0.0
    for t in range(16):
        got = gl.forward(x[t:t + 1], path=M.MOE_PATH_FUSED)
        worst = max(worst, check_layer(gl, OL, x[t:t + 1], *got))
        _agree(got, gl.forward(x[t:t + 1], path=M.MOE_PATH_DECODE))
    print(f"fused: worst rel L2 over 16 tokens {worst:.3e}")
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_fused_router_integer_inputs_bit_exact(decode_layer):
    """The fused kernel's router workgroups on integer-valued tokens: exact
    fp32 sums, so the chosen sets equal the oracle's with no tie band."""
    w, gl, OL = decode_layer
    rng = np.random.default_rng(13)
    x = f32_to_bf16_bits(rng.integers(-2, 3, size=(12, w.d)).astype(np.float32))
    logits = OL.logits(x)
    for t in range(12):
        _, ids, wt = gl.forward(x[t:t + 1], path=M.MOE_PATH_FUSED)
        ids_ref, w_ref, _ = O.select(logits[t], w.K)
        assert np.array_equal(ids[0], ids_ref), t
        assert np.allclose(wt[0], w_ref, rtol=2e-5, atol=1e-7)
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_auto_takes_fused_for_one_token(decode_layer):
    w, gl, OL = decode_layer
    M.moe_layer_profile(gl.handle, True)
    x = make_tokens(w, 1, stream=22)
    gl.forward(x)
    rec = M.moe_layer_profile_read(gl.handle)
    M.moe_layer_profile(gl.handle, False)
    assert set(rec) == {"fused_layer"}, rec


SHAPES = [  # (d, E, K, f, fs): one expert, no shared expert, K = E, E > 256, ragged groups
    (64, 1, 1, 64, 0),
    (192, 3, 3, 64, 64),
    (1088, 17, 4, 192, 128),
    (512, 300, 9, 64, 0),
    (2048, 256, 8, 512, 512),
    (4096, 8, 2, 128, 64),
    (256, 64, 64, 64, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_fused_shapes(shape):
    d, E, K, f, fs = shape
    w = Workload(82, "shape", d=d, E=E, K=K, f=f, fs=fs, act="bf16", zipf=1.0, T=4)
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 1)
    OL = O.OracleLayer.from_workload(w, arrays)
    x = make_tokens(w, 4, stream=5)
    for t in range(4):
        got = gl.forward(x[t:t + 1], path=M.MOE_PATH_FUSED)
        check_layer(gl, OL, x[t:t + 1], *got)
        _agree(got, gl.forward(x[t:t + 1], path=M.MOE_PATH_DECODE))
    assert M.moe_layer_check_errors(gl.handle) == 0
    gl.close()


@pytest.mark.parametrize("seed", range(6))
def test_fused_forced_sets_on_random_shapes(seed):
    """Seeded random shapes within the fused kernel's limits, each with a
    forced set of distinct experts given in shuffled order (the routed
    gate/up workgroups then skip the logits): the oracle on the same set, and
    the three-kernel path on it."""
    rng = np.random.default_rng(1000 + seed)
    while True:
        d = 64 * int(rng.integers(1, 65))
        E = int(rng.integers(1, 301))
        K = int(rng.integers(1, min(E, 16) + 1))
        f = 64 * int(rng.integers(1, 13))
        fs = 64 * int(rng.integers(0, 9))
        if K * (f // 64) <= 128:
            break
    print(f"shape d={d} E={E} K={K} f={f} fs={fs}", flush=True)
    w = Workload(124 + seed, "forced-shape", d=d, E=E, K=K, f=f, fs=fs, act="bf16", zipf=1.0, T=2)
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 1)
    OL = O.OracleLayer.from_workload(w, arrays)
    x = make_tokens(w, 2, stream=6)
    for t in range(2):
        chosen = np.sort(rng.choice(E, size=K, replace=False)).astype(np.int32)
        shuffled = rng.permutation(chosen).astype(np.int32)[None, :]
        got = gl.forward(x[t:t + 1], path=M.MOE_PATH_FUSED, forced=shuffled)
        check_layer(gl, OL, x[t:t + 1], *got, forced=chosen[None, :])
        _agree(got, gl.forward(x[t:t + 1], path=M.MOE_PATH_DECODE, forced=chosen[None, :]))
    assert M.moe_layer_check_errors(gl.handle) == 0
    gl.close()


def test_fused_many_launches_and_graph_replays(decode_layer):
    """Back-to-back launches, then a captured graph of 8 calls replayed 4
    times with eager work in between; every replay equals the eager result."""
    w, gl, OL = decode_layer
    torch = torch_mod()
    n = 8
    x = make_tokens(w, n, stream=23)
    xd = [to_device(x[i:i + 1]) for i in range(n)]
    ref = []
    for i in range(n):
        ref.append(gl.forward(x[i:i + 1], path=M.MOE_PATH_FUSED)[0])
    for rep in range(3):  # 3 x 8 eager launches without a sync between them
        outs = [empty_like_act(w, 1) for _ in range(n)]
        for i in range(n):
            M.moe_layer_forward(xd[i], gl.handle, outs[i], 1, None)
        torch.cuda.synchronize()
        for i in range(n):
            assert np.array_equal(to_host(outs[i]), ref[i]), (rep, i)
    outs = [empty_like_act(w, 1) for _ in range(n)]
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(n):
            M.moe_layer_forward(xd[i], gl.handle, outs[i], 1, cap.cuda_stream)
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            assert np.array_equal(to_host(outs[i]), ref[i]), (rep, i)
        gl.forward(x[rep:rep + 1], path=M.MOE_PATH_DECODE)  # eager work between replays
    del g
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_fused_forced_and_reused(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 2, stream=24)
    forced = np.array([[3, 7, 11, 50, 51, 90, 100, 126]], np.int32)
    got = gl.forward(x[:1], path=M.MOE_PATH_FUSED, forced=forced)
    check_layer(gl, OL, x[:1], *got, forced=forced)
    got2 = gl.forward(x[1:2], path=M.MOE_PATH_FUSED, reuse=True)
    check_layer(gl, OL, x[1:2], *got2, forced=forced)
    _agree(got2, gl.forward(x[1:2], path=M.MOE_PATH_DECODE, forced=forced))
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_fused_forced_set_in_any_order(decode_layer):
    """A forced set names its experts in any order: the routed gate/up
    workgroups take the k-th smallest id without waiting for the logits, and
    the result is bit-identical to the same set given in ascending order."""
    w, gl, OL = decode_layer
    x = make_tokens(w, 1, stream=27)
    ordered = np.array([[3, 7, 11, 50, 51, 90, 100, 126]], np.int32)
    shuffled = np.array([[126, 3, 90, 7, 51, 11, 100, 50]], np.int32)
    a = gl.forward(x, path=M.MOE_PATH_FUSED, forced=ordered)
    b = gl.forward(x, path=M.MOE_PATH_FUSED, forced=shuffled)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    check_layer(gl, OL, x, *b, forced=ordered)
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_fused_bad_forced_id_is_flagged(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 1, stream=25)
    gl.forward(x, path=M.MOE_PATH_FUSED, forced=np.array([[0, 1, 2, 3, 4, 5, 6, 999]], np.int32))
    assert M.moe_layer_check_errors(gl.handle) == 1
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_fused_refuses_what_it_does_not_serve(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 2, stream=26)
    with pytest.raises(M.MoeError):  # two tokens
        gl.forward(x, path=M.MOE_PATH_FUSED)
    wf = WORKLOADS[0]
    g32 = GpuLayer(wf, make_layer(wf), 1)
    with pytest.raises(M.MoeError):  # fp32 activations
        g32.forward(make_tokens(wf, 1), path=M.MOE_PATH_FUSED)
    g32.close()
    wd = Workload(83, "wide", d=4160, E=8, K=2, f=128, fs=64, act="bf16", zipf=1.0, T=1)
    gwide = GpuLayer(wd, make_layer(wd), 1)
    with pytest.raises(M.MoeError):  # d_model above 4096
        gwide.forward(make_tokens(wd, 1), path=M.MOE_PATH_FUSED)
    gwide.forward(make_tokens(wd, 1))  # AUTO falls back to the three-kernel path
    gwide.close()
