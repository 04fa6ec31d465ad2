"""Shared helpers of the GPU parity tests: move canonical arrays through the
C ABI, run the HIP path, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import routed_expert_ffn_int8_amd as M
from gen.workloads import Workload
from oracle import oracle as O

TIE_BAND = 1e-4


def torch_mod():
    import torch
    return torch


def to_device(x: np.ndarray):
    torch = torch_mod()
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_like_act(w: Workload, T: int):
    torch = torch_mod()
    return torch.empty((T, w.d), dtype=torch.bfloat16 if w.act == "bf16" else torch.float32, device="cuda")


class GpuLayer:
    def __init__(self, w: Workload, arrays: dict, max_tokens: int, residency=M.MOE_RESIDENT):
        act = M.MOE_ACT_BF16 if w.act == "bf16" else M.MOE_ACT_F32
        desc, keep = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, act, max_tokens, residency)
        self.w = w
        self.handle = M.moe_layer_create(desc)
        del keep

    def forward(self, x: np.ndarray, path=M.MOE_PATH_AUTO, forced=None, reuse=False, stream=None):
        torch = torch_mod()
        T = x.shape[0]
        xd = to_device(x)
        out = empty_like_act(self.w, T)
        ids = torch.empty((T, self.w.K), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, self.w.K), dtype=torch.float32, device="cuda")
        fz = None if forced is None else torch.from_numpy(np.ascontiguousarray(forced, np.int32)).cuda()
        opts = M.fwd_opts(topk_ids=ids, topk_w=wts, forced_ids=fz, reuse_previous=reuse, path=path)
        M.moe_layer_forward_ex(xd, self.handle, out, T, opts, stream)
        torch.cuda.synchronize()
        return to_host(out), ids.cpu().numpy(), wts.cpu().numpy()

    def close(self):
        if self.handle:
            M.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tolerances(act: str):
    """(relative L2, max-abs as a multiple of rms(ref)) per token."""
    return (1e-5, 1e-4) if act == "f32" else (5e-3, 3e-2)


def check_selection(ids_gpu, ids_ref, logits, margin, K):
    """Bit-exact sets where the K-th/(K+1)-th margin exceeds the tie band;
    inside the band, the GPU set may swap experts whose logits lie within the
    band of the K-th largest.  Returns the list of tokens that took a swap."""
    swapped = []
    for t in range(ids_ref.shape[0]):
        a, b = set(ids_gpu[t].tolist()), set(ids_ref[t].tolist())
        assert list(ids_gpu[t]) == sorted(ids_gpu[t].tolist()), "ids must be ascending"
        if a == b:
            continue
        assert margin[t] <= TIE_BAND, f"token {t}: sets differ with margin {margin[t]}"
        lk = np.sort(logits[t])[::-1][K - 1]
        for e in a ^ b:
            assert abs(logits[t][e] - lk) <= TIE_BAND, f"token {t}: expert {e} outside the tie band"
        swapped.append(t)
    return swapped


def check_layer(gl: GpuLayer, OL: O.OracleLayer, x: np.ndarray, y_gpu, ids_gpu, w_gpu, forced=None):
    """Compare GPU outputs with the oracle token by token; returns worst rel L2."""
    w = gl.w
    y_ref, ids_ref, w_ref, margin = OL.forward(x, forced=forced)
    logits = OL.logits(x)
    if forced is None:
        swapped = check_selection(ids_gpu, ids_ref, logits, margin, w.K)
    else:
        assert np.array_equal(ids_gpu, np.asarray(forced)), "forced sets must be used as given"
        swapped = []
    if swapped:  # re-derive the oracle on the GPU's (equally valid) sets
        y_f, _, w_f, _ = OL.forward(x, forced=ids_gpu)
        y_ref[swapped], w_ref[swapped] = y_f[swapped], w_f[swapped]
    assert np.allclose(w_gpu, w_ref, rtol=2e-5, atol=1e-6), np.abs(w_gpu - w_ref).max()
    rel_tol, abs_tol = tolerances(w.act)
    yg = O.tokens_to_f64(y_gpu)
    worst = 0.0
    for t in range(x.shape[0]):
        ref = y_ref[t]
        rms = np.sqrt(np.mean(ref * ref))
        rel = np.linalg.norm(yg[t] - ref) / np.linalg.norm(ref)
        mx = np.abs(yg[t] - ref).max()
        assert rel <= rel_tol, f"token {t}: rel L2 {rel:.3e} > {rel_tol}"
        assert mx <= abs_tol * rms, f"token {t}: max abs {mx:.3e} > {abs_tol} * rms {rms:.3e}"
        worst = max(worst, rel)
    return worst


def _bf16_ulp(v):
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0**-126)))
    return 2.0 ** (e - 7)


def check_stack_layer(OL: O.OracleLayer, K: int, h_in: np.ndarray, h_out: np.ndarray, ids_gpu: np.ndarray):
    """Teacher forcing of one stack layer on the GPU's own input h_in (bf16
    bits [d]): the oracle takes n = bf16(rmsnorm(h_in)), routes it (the GPU's
    set must be the oracle's outside the tie band; inside it the oracle is
    forced to the GPU's set) and forms bf16(h_in + MoE(n)); the GPU's h_out
    must lie within the layer tolerance of that, plus one bf16 ulp of the
    result for its final rounding.  Returns the relative error."""
    n = O.rmsnorm_bf16(h_in)
    logits = OL.logits(n[None, :])
    y_ref, ids_ref, _, margin = OL.forward(n[None, :])
    swapped = check_selection(ids_gpu.reshape(1, K), ids_ref, logits, margin, K)
    if swapped:
        y_ref, *_ = OL.forward(n[None, :], forced=ids_gpu.reshape(1, K))
    ref = O.residual_bf16(h_in, y_ref[0])
    got, want = O.tokens_to_f64(h_out), O.tokens_to_f64(ref)
    ynorm = np.linalg.norm(y_ref[0])
    err = np.linalg.norm(got - want)
    assert err <= 5e-3 * ynorm + np.linalg.norm(_bf16_ulp(want)), (err, ynorm)
    return err / ynorm
