"""Dense numpy brute force of the MoE layer, written independently of moe_oracle.c.

TEST INFRASTRUCTURE ONLY.  Differs in structure from the C oracle on purpose:
it dequantises whole matrices with array operations, evaluates EVERY routed
expert densely, forms the gate coefficients as a softmax over all E experts
that is then masked to the top-K (chosen by a lexicographic sort) and
renormalised, and combines with a 0/w mask.  For tiny layers only.
"""
from __future__ import annotations

import numpy as np


def f16(a):
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(q, s, b):
    q = np.asarray(q, dtype=np.uint32)
    shifts = (np.arange(8, dtype=np.uint32) * 4)
    nib = ((q[..., :, None] >> shifts) & 0xF).reshape(q.shape[:-1] + (q.shape[-1] * 8,)).astype(np.float64)
    S = np.repeat(f16(s), 64, axis=-1)
    B = np.repeat(f16(b), 64, axis=-1)
    return S * nib + B


def silu(z):
    return z / (1.0 + np.exp(-z))


def ffn(Wg, Wu, Wd, x):
    return Wd @ (silu(Wg @ x) * (Wu @ x))


def layer(arrays: dict, K: int, x64: np.ndarray):
    """x64: [T, d] float64.  Returns y [T, d], ids [T, K] ascending, w [T, K]."""
    a = arrays
    Wr = a["router_w"].astype(np.float64) * f16(a["router_scale"])[:, None]
    bias = 0.0 if a.get("router_bias") is None else a["router_bias"].astype(np.float64)
    E = Wr.shape[0]
    Wg, Wu, Wd = dequant(a["gate_q"], a["gate_s"], a["gate_b"]), dequant(a["up_q"], a["up_s"], a["up_b"]), \
        dequant(a["down_q"], a["down_s"], a["down_b"])
    has_shared = a.get("sh_gate_q") is not None
    if has_shared:
        Sg, Su, Sd = (dequant(a[p + "_q"], a[p + "_s"], a[p + "_b"]) for p in ("sh_gate", "sh_up", "sh_down"))
    T = x64.shape[0]
    ys, idss, ws = [], [], []
    for t in range(T):
        x = x64[t]
        logits = Wr @ x + bias
        order = np.lexsort((np.arange(E), -logits))  # logit descending, index ascending
        mask = np.zeros(E)
        mask[order[:K]] = 1.0
        p = np.exp(logits - logits.max())
        p = p / p.sum()
        wfull = mask * p / (mask * p).sum()
        outs = np.stack([ffn(Wg[e], Wu[e], Wd[e], x) for e in range(E)])
        y = (wfull[:, None] * outs).sum(axis=0)
        if has_shared:
            y = y + ffn(Sg, Su, Sd, x)
        ids = np.sort(order[:K]).astype(np.int32)
        ys.append(y)
        idss.append(ids)
        ws.append(wfull[ids])
    return np.array(ys), np.array(idss), np.array(ws)
