"""Decode-path parity: the HIP kernels through the C ABI against the fp64
oracle, element by element, on seeded inputs."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, Workload, make_layer, make_tokens, f32_to_bf16_bits
from oracle import oracle as O
from tests.helpers import GpuLayer, check_layer, to_device, torch_mod

pytestmark = pytest.mark.gpu


def _layer(w, max_tokens=8, arrays=None):
    arrays = make_layer(w) if arrays is None else arrays
    return GpuLayer(w, arrays, max_tokens), O.OracleLayer.from_workload(w, arrays), arrays


def test_tiny_f32_workload():
    w = WORKLOADS[0]
    gl, OL, _ = _layer(w, max_tokens=w.T)
    x = make_tokens(w, w.T)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_DECODE)
    check_layer(gl, OL, x, y, ids, wt)
    assert M.moe_layer_check_errors(gl.handle) == 0


@pytest.fixture(scope="module")
def decode_layer():
    w = WORKLOADS[1]
    gl, OL, arrays = _layer(w, max_tokens=8)
    yield w, gl, OL
    gl.close()


def test_decode_layer_batch1_tokens(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 12, stream=7)
    worst = 0.0
    for t in range(12):
        y, ids, wt = gl.forward(x[t:t + 1], path=M.MOE_PATH_DECODE)
        worst = max(worst, check_layer(gl, OL, x[t:t + 1], y, ids, wt))
    print(f"worst rel L2 over 12 batch-1 tokens: {worst:.3e}")
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_decode_layer_multi_token_call(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 8, stream=8)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_DECODE)
    check_layer(gl, OL, x, y, ids, wt)


def test_repeat_is_bit_identical(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 3, stream=9)
    a = gl.forward(x, path=M.MOE_PATH_DECODE)
    b = gl.forward(x, path=M.MOE_PATH_DECODE)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_zero_tokens_is_noop(decode_layer):
    w, gl, OL = decode_layer
    torch = torch_mod()
    x = torch.zeros((1, w.d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, w.d), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_layer_forward(x, gl.handle, out, 0)
    torch.cuda.synchronize()
    assert float(out.float().min()) == 7.0
    with pytest.raises(M.MoeError):
        M.moe_layer_forward(x, gl.handle, out, 9)  # above max_tokens


SHAPES = [  # (d, E, K, f, fs, act): ragged group counts, K = E, no shared expert, one expert
    (64, 1, 1, 64, 0, "f32"),
    (192, 3, 3, 64, 64, "bf16"),
    (1088, 17, 4, 192, 128, "bf16"),
    (1088, 17, 4, 192, 128, "f32"),
    (512, 300, 9, 64, 0, "bf16"),
    (4160, 8, 2, 128, 64, "bf16"),
    (256, 64, 64, 64, 64, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_random_shapes(shape):
    d, E, K, f, fs, act = shape
    w = Workload(80, "shape", d=d, E=E, K=K, f=f, fs=fs, act=act, zipf=1.0, T=5)
    gl, OL, _ = _layer(w, max_tokens=5)
    x = make_tokens(w, 5, stream=3)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_DECODE)
    check_layer(gl, OL, x, y, ids, wt)
    gl.close()


def test_integer_inputs_route_bit_exact():
    """Integer-valued inputs make the router sums exact in fp32, so the chosen
    sets must equal the oracle's with no tie band (exact ties included)."""
    w = WORKLOADS[1]
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 8)
    OL = O.OracleLayer.from_workload(w, arrays)
    rng = np.random.default_rng(11)
    torch = torch_mod()
    for rep in range(4):
        xi = rng.integers(-2, 3, size=(8, w.d)).astype(np.float32)
        x = f32_to_bf16_bits(xi)
        ids = torch.empty((8, w.K), dtype=torch.int32, device="cuda")
        wt = torch.empty((8, w.K), dtype=torch.float32, device="cuda")
        M.moe_layer_route(to_device(x), gl.handle, ids, wt, 8)
        torch.cuda.synchronize()
        _, ids_ref, w_ref, _ = OL.forward(x)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.allclose(wt.cpu().numpy(), w_ref, rtol=2e-5, atol=1e-7)
    gl.close()


def test_exact_ties_go_to_lower_index():
    w = Workload(81, "ties", d=128, E=8, K=2, f=64, fs=64, act="bf16", zipf=None, T=2)
    arrays = make_layer(w)
    x = make_tokens(w, 2)
    top = np.where(O.tokens_to_f64(x[0]) >= 0, 127, -127).astype(np.int8)
    rw = arrays["router_w"].copy()
    rw[6] = top
    rw[3] = top
    rw[5] = top
    arrays["router_w"] = rw
    gl, OL, _ = _layer(w, max_tokens=2, arrays=arrays)
    y, ids, wt = gl.forward(x[:1], path=M.MOE_PATH_DECODE)
    assert list(ids[0]) == [3, 5]
    check_layer(gl, OL, x[:1], y, ids, wt)
    gl.close()


def test_forced_and_reused_sets(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 2, stream=12)
    forced = np.array([[1, 5, 9, 20, 40, 64, 100, 127], [0, 2, 3, 4, 5, 6, 7, 8]], np.int32)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_DECODE, forced=forced)
    check_layer(gl, OL, x, y, ids, wt, forced=forced)
    x2 = make_tokens(w, 2, stream=13)
    y2, ids2, wt2 = gl.forward(x2, path=M.MOE_PATH_DECODE, reuse=True)
    check_layer(gl, OL, x2, y2, ids2, wt2, forced=forced)
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_bad_forced_id_is_flagged(decode_layer):
    w, gl, OL = decode_layer
    x = make_tokens(w, 1, stream=14)
    forced = np.array([[1, 2, 3, 4, 5, 6, 7, 500]], np.int32)
    gl.forward(x, path=M.MOE_PATH_DECODE, forced=forced)
    assert M.moe_layer_check_errors(gl.handle) & 1
    assert M.moe_layer_check_errors(gl.handle) == 0
