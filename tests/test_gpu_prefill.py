"""Prefill-path parity: token->expert grouping + grouped bf16 MFMA GEMMs
against the fp64 oracle, including multi-chunk calls and ragged shapes."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, Workload, f32_to_bf16_bits, make_layer, make_tokens
from oracle import oracle as O
from tests.helpers import GpuLayer, check_layer, check_selection, to_device, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prefill_layer():
    w = WORKLOADS[3]
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 2048)
    yield w, gl, O.OracleLayer.from_workload(w, arrays)
    gl.close()


def _oracle_selection(OL, x, K):
    """The oracle's logits, sets, coefficients and margins of every token
    (router and selection only)."""
    logits = OL.logits(x)
    ids = np.empty((x.shape[0], K), np.int32)
    wts = np.empty((x.shape[0], K))
    margin = np.empty(x.shape[0])
    for t in range(x.shape[0]):
        ids[t], wts[t], margin[t] = O.select(logits[t], K)
    return logits, ids, wts, margin


def test_prefill_chunk_128_full(prefill_layer):
    w, gl, OL = prefill_layer
    x = make_tokens(w, 128, stream=31)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    worst = check_layer(gl, OL, x, y, ids, wt)
    print(f"prefill chunk: worst rel L2 {worst:.3e}")


def test_prefill_512_as_four_chunks_full(prefill_layer):
    """The 512-token run of the prefill workload (four 128-token chunks in
    one call), every token against the oracle."""
    w, gl, OL = prefill_layer
    x = make_tokens(w, 512, stream=32)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    worst = check_layer(gl, OL, x, y, ids, wt)
    print(f"prefill 512: worst rel L2 {worst:.3e}")


def test_prefill_2048_as_sixteen_chunks(prefill_layer):
    """The 2048-token run (sixteen chunks in one call): every token's expert
    set against the oracle's selection, and outputs on the first two and last
    two tokens of every chunk plus one inside it (80 tokens, every chunk edge)."""
    w, gl, OL = prefill_layer
    x = make_tokens(w, 2048, stream=36)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    logits, ids_ref, _, margin = _oracle_selection(OL, x, w.K)
    check_selection(ids, ids_ref, logits, margin, w.K)
    sample = np.concatenate([c * 128 + np.array([0, 1, 61, 126, 127]) for c in range(16)])
    worst = check_layer(gl, OL, x[sample], y[sample], ids[sample], wt[sample])
    print(f"prefill 2048: worst rel L2 on {len(sample)} sampled tokens {worst:.3e}")


def test_prefill_sort_outputs(prefill_layer):
    """Grouping outputs of a two-chunk call: one row of offsets per chunk and
    each chunk's pairs (chunk-local token index) in its part of the perm."""
    w, gl, OL = prefill_layer
    torch = torch_mod()
    T = 200
    x = make_tokens(w, T, stream=33)
    out = torch.empty((T, w.d), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    offs = torch.empty((2, w.E + 1), dtype=torch.int32, device="cuda")
    perm = torch.empty(T * w.K, dtype=torch.int32, device="cuda")
    o = M.fwd_opts(topk_ids=ids, path=M.MOE_PATH_PREFILL, sort_offsets=offs, sort_perm=perm)
    M.moe_layer_forward_ex(to_device(x), gl.handle, out, T, o)
    torch.cuda.synchronize()
    ids_h, offs_h, perm_h = ids.cpu().numpy(), offs.cpu().numpy(), perm.cpu().numpy()
    for c, (t0, t1) in enumerate(((0, 128), (128, T))):
        _, off_ref, perm_ref, _ = O.sort(ids_h[t0:t1], w.E)
        assert np.array_equal(offs_h[c], off_ref), c
        assert np.array_equal(perm_h[t0 * w.K:t1 * w.K], perm_ref), c


def test_reuse_previous_after_multichunk_prefill(prefill_layer):
    """A 256-token prefill call, then calls that reuse its expert sets (prefill
    and decode paths): every chunk's sets come back, with coefficients from
    the new logits, and outputs match the oracle forced to those sets."""
    w, gl, OL = prefill_layer
    T = 256
    x1 = make_tokens(w, T, stream=37)
    _, ids1, _ = gl.forward(x1, path=M.MOE_PATH_PREFILL)
    x2 = make_tokens(w, T, stream=38)
    y2, ids2, wt2 = gl.forward(x2, path=M.MOE_PATH_PREFILL, reuse=True)
    assert np.array_equal(ids2, ids1)
    sample = np.r_[0:4, 124:132, 252:256]
    check_layer(gl, OL, x2[sample], y2[sample], ids2[sample], wt2[sample], forced=ids1[sample])
    y3, ids3, wt3 = gl.forward(x2, path=M.MOE_PATH_DECODE, reuse=True)
    assert np.array_equal(ids3, ids1)
    check_layer(gl, OL, x2[sample], y3[sample], ids3[sample], wt3[sample], forced=ids1[sample])
    assert M.moe_layer_check_errors(gl.handle) == 0


def test_prefill_router_integer_inputs_bit_exact(prefill_layer):
    """Integer-valued tokens make every matrix-core router sum an exact
    integer in fp32, so each logit is the fp32 rounding of the oracle's and
    the chosen sets must equal the oracle's with no tie band."""
    w, gl, OL = prefill_layer
    rng = np.random.default_rng(12)
    for rep in range(2):
        x = f32_to_bf16_bits(rng.integers(-2, 3, size=(128, w.d)).astype(np.float32))
        _, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
        _, ids_ref, w_ref, _ = _oracle_selection(OL, x, w.K)
        assert np.array_equal(ids, ids_ref), rep
        assert np.allclose(wt, w_ref, rtol=2e-5, atol=1e-7)


PSHAPES = [  # (d, E, K, f, fs, T)
    (512, 16, 4, 128, 0, 37),
    (512, 16, 16, 64, 192, 20),
    (1024, 300, 8, 256, 128, 130),
    (2816, 128, 8, 704, 2112, 24),
    (256, 1, 1, 64, 64, 16),
    (512, 4, 2, 128, 64, 128),     # every routed expert has about 64 rows (four 16-row tiles)
    (1024, 8, 8, 128, 128, 200),   # K = E: every expert takes every row (128, then 72)
    (192, 8, 2, 64, 64, 40),       # 3 groups per gate/up row, 1 per down row: the scale batches of 4 clamp
    (320, 16, 4, 192, 0, 17),      # 5 and 3 groups per row, no shared expert, ragged last tile
]


@pytest.mark.parametrize("shape", PSHAPES, ids=[str(s) for s in PSHAPES])
def test_prefill_shapes(shape):
    d, E, K, f, fs, T = shape
    w = Workload(84, "pshape", d=d, E=E, K=K, f=f, fs=fs, act="bf16", zipf=1.0, T=T)
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, T)
    x = make_tokens(w, T, stream=34)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    check_layer(gl, O.OracleLayer.from_workload(w, arrays), x, y, ids, wt)
    gl.close()


def test_prefill_and_decode_paths_agree(prefill_layer):
    """Same expert sets; coefficients equal up to the fp32 summation order of
    the router (matrix-core tiles in prefill, one wavefront per row in
    decode), which moves logits by ~1e-6."""
    w, gl, OL = prefill_layer
    x = make_tokens(w, 16, stream=35)
    yp, idp, wp = gl.forward(x, path=M.MOE_PATH_PREFILL)
    yd, idd, wd = gl.forward(x, path=M.MOE_PATH_DECODE)
    assert np.array_equal(idp, idd)
    assert np.max(np.abs(wp - wd)) < 1e-5
    a, b = O.tokens_to_f64(yp), O.tokens_to_f64(yd)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 5e-3


def _mixed_forced(w, T, seed):
    """Forced sets: the first half of the tokens choose experts 0..K-1 (so
    those experts have at least T/2 rows: several 16-row tiles each), the
    rest random distinct sets (a few rows per expert)."""
    rng = np.random.default_rng(seed)
    ids = np.empty((T, w.K), np.int32)
    for t in range(T):
        ids[t] = np.arange(w.K) if t < T // 2 else np.sort(rng.choice(w.E, w.K, replace=False))
    return ids


def test_prefill_busy_and_sparse_experts_in_one_chunk(prefill_layer):
    """Experts with many rows (several 16-row tiles, a ragged last one)
    beside experts with a few rows and the shared expert, in one 128-token
    chunk and in a 300-token call, against the oracle forced to the same
    sets."""
    w, gl, OL = prefill_layer
    for T, seed in ((128, 51), (300, 52)):
        x = make_tokens(w, T, stream=seed)
        forced = _mixed_forced(w, T, seed)
        y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL, forced=forced)
        worst = check_layer(gl, OL, x, y, ids, wt, forced=forced)
        print(f"mixed forced T={T}: worst rel L2 {worst:.3e}")


def test_prefill_dense_routing_matches_oracle(prefill_layer):
    """The dense-routing case of the prefill benchmark (every token on
    experts 0..K-1: eight full 16-row tiles per chosen expert)."""
    w, gl, OL = prefill_layer
    x = make_tokens(w, 128, stream=53)
    forced = np.tile(np.arange(w.K, dtype=np.int32), (128, 1))
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL, forced=forced)
    worst = check_layer(gl, OL, x, y, ids, wt, forced=forced)
    print(f"dense routing: worst rel L2 {worst:.3e}")


def test_streamed_prefill_busy_experts_equals_resident():
    """A streamed layer's prefill with busy experts (many tiles each, inside
    the cache groups) stays bit-identical to the resident layer."""
    w = Workload(89, "pf-stream-wide", d=512, E=64, K=8, f=128, fs=128, act="bf16", zipf=1.0, T=1, slots=16)
    arrays = make_layer(w)
    res = GpuLayer(w, arrays, 256)
    st = GpuLayer(w, arrays, 256, residency=M.MOE_STREAMED)
    M.moe_cache_attach(st.handle, w.slots)
    for T, seed in ((128, 54), (256, 55)):
        x = make_tokens(w, T, stream=seed)
        forced = _mixed_forced(w, T, seed)
        y_r, ids_r, w_r = res.forward(x, path=M.MOE_PATH_PREFILL, forced=forced)
        y_s, ids_s, w_s = st.forward(x, path=M.MOE_PATH_PREFILL, forced=forced)
        assert np.array_equal(y_r, y_s), f"T={T}: streamed prefill differs from resident"
        assert np.array_equal(w_r, w_s)
    check_layer(res, O.OracleLayer.from_workload(w, arrays), x, y_r, ids_r, w_r, forced=forced)
    assert M.moe_layer_check_errors(st.handle) == 0
    res.close()
    st.close()
