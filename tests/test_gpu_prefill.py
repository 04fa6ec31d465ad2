"""Prefill-path parity: token->expert grouping + grouped bf16 MFMA GEMMs
against the fp64 oracle, including multi-chunk calls and ragged shapes."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, Workload, make_layer, make_tokens
from oracle import oracle as O
from tests.helpers import GpuLayer, check_layer, to_device, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prefill_layer():
    w = WORKLOADS[3]
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 512)
    yield w, gl, O.OracleLayer.from_workload(w, arrays)
    gl.close()


def test_prefill_chunk_128_full(prefill_layer):
    w, gl, OL = prefill_layer
    x = make_tokens(w, 128, stream=31)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    worst = check_layer(gl, OL, x, y, ids, wt)
    print(f"prefill chunk: worst rel L2 {worst:.3e}")


def test_prefill_512_as_four_chunks_sampled(prefill_layer):
    w, gl, OL = prefill_layer
    x = make_tokens(w, 512, stream=32)
    y, ids, wt = gl.forward(x, path=M.MOE_PATH_PREFILL)
    sample = np.r_[0:3, 125:131, 254:258, 380:384, 509:512]
    check_layer(gl, OL, x[sample], y[sample], ids[sample], wt[sample])


def test_prefill_sort_outputs(prefill_layer):
    w, gl, OL = prefill_layer
    torch = torch_mod()
    x = make_tokens(w, 100, stream=33)
    out = torch.empty((100, w.d), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((100, w.K), dtype=torch.int32, device="cuda")
    offs = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(100 * w.K, dtype=torch.int32, device="cuda")
    o = M.fwd_opts(topk_ids=ids, path=M.MOE_PATH_PREFILL, sort_offsets=offs, sort_perm=perm)
    M.moe_layer_forward_ex(to_device(x), gl.handle, out, 100, o)
    torch.cuda.synchronize()
    c, off_ref, perm_ref, _ = O.sort(ids.cpu().numpy(), w.E)
    assert np.array_equal(offs.cpu().numpy(), off_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)


PSHAPES = [  # (d, E, K, f, fs, T)
    (512, 16, 4, 128, 0, 37),
    (512, 16, 16, 64, 192, 20),
    (1024, 300, 8, 256, 128, 130),
    (2816, 128, 8, 704, 2112, 24),
    (256, 1, 1, 64, 64, 16),
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
