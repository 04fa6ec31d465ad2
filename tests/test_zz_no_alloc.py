"""The allocation-free forward (moe_layer_forward_noalloc) against the
existing forward on the same kernels: bit-identical outputs on two calls in a
row, the second with fewer tokens, plus the oracle on its own routing, and a
clear refusal past its workspace."""
import numpy as np
import pytest

import routed_expert_ffn_int8_amd as M
from gen.workloads import WORKLOADS, make_layer, make_tokens
from oracle import oracle as O
from tests.helpers import GpuLayer, check_layer, empty_like_act, to_device, to_host, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wid", [1, 3], ids=["decode-layer", "prefill-shape"])
def test_noalloc_forward_equals_forward(wid):
    torch = torch_mod()
    w = WORKLOADS[wid]
    arrays = make_layer(w)
    gl = GpuLayer(w, arrays, 64)
    OL = O.OracleLayer.from_workload(w, arrays)
    for n, stream in ((40, 61), (3, 62)):  # the second call is smaller
        x = make_tokens(w, n, stream=stream)
        y_ref, ids, wt = gl.forward(x, path=M.MOE_PATH_DECODE)
        xd = to_device(x)
        out = empty_like_act(w, n)
        out.fill_(7)
        M.moe_layer_forward_noalloc(xd, gl.handle, out, n)
        torch.cuda.synchronize()
        y = to_host(out)
        assert np.array_equal(y, y_ref), f"{n} tokens: outputs differ from moe_layer_forward"
        sample = np.arange(min(n, 6))
        check_layer(gl, OL, x[sample], y[sample], ids[sample], wt[sample])
    assert M.moe_layer_check_errors(gl.handle) == 0
    gl.close()


def test_noalloc_forward_refuses_what_does_not_fit():
    w = WORKLOADS[1]
    gl = GpuLayer(w, make_layer(w), 600)
    x = to_device(make_tokens(w, 600, stream=63))
    out = empty_like_act(w, 600)
    with pytest.raises(M.MoeError):  # about 16 KB per token: 600 tokens exceed 8 MiB
        M.moe_layer_forward_noalloc(x, gl.handle, out, 600)
    M.moe_layer_forward_noalloc(x, gl.handle, out, 400)  # this one fits
    torch_mod().cuda.synchronize()
    assert M.moe_layer_check_errors(gl.handle) == 0
    gl.close()
