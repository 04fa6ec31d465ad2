"""Workload shapes and seeded generators.

Canonical host layout of one 4-bit affine matrix with `rows` output rows and
`cols` input columns (groups of 64 run along the input dimension):

* packed  uint32 [rows][cols/8]   nibble k of word j is q[row][8j+k], low nibble first
* scale   uint16 [rows][cols/64]  fp16 bit patterns
* bias    uint16 [rows][cols/64]  fp16 bit patterns

Routed experts are stacked along a leading expert axis.  Gate and up matrices
have rows = d_ff, cols = d_model; down has rows = d_model, cols = d_ff.  The
router is int8 [E][d_model] with one fp16 scale per row and an optional fp32
per-expert logit bias.

Value recipe (all drawn from numpy PCG64DXSM streams keyed by
SeedSequence([seed, workload, layer, tensor])):

* packed words uniform over uint32 (equivalent to iid q ~ U{0..15});
* scale ~ U(0.002, 0.02) rounded to fp16;
* bias = fp16(-8 * scale + N(0, sd=1e-4)), using the already-rounded scale;
* router weights ~ U{-127..127}; router scale = fp16(1e-3);
* Zipf-skewed routing: logit bias b_e = -s * ln(rank_e), rank a seeded
  permutation of 1..E, stored as fp32 (absent when s is None);
* tokens x ~ N(0, 1), stored as fp32 or as bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import numpy as np

GROUP = 64

# tensor ids inside the seed sequence
_T_ROUTER_W, _T_ROUTER_PERM = 0, 1
_T_MATS = {  # (q, scale, bias-noise) per matrix name
    "gate": (2, 3, 4), "up": (5, 6, 7), "down": (8, 9, 10),
    "sh_gate": (11, 12, 13), "sh_up": (14, 15, 16), "sh_down": (17, 18, 19),
}
_T_TOKENS, _T_NOISE, _T_REUSE = 20, 21, 22


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    d: int            # d_model
    E: int            # routed experts
    K: int            # experts per token
    f: int            # routed expert d_ff
    fs: int           # shared expert d_ff
    act: str          # "f32" or "bf16"
    zipf: float | None
    T: int            # tokens per call
    layers: int = 1
    steps: int = 1    # calls (tokens for decode, steps for stacks)
    noise_sd: float = 0.0
    reuse_p: float = 0.0
    slots: int = 0
    extra_T: tuple = ()


WORKLOADS = {
    0: Workload(0, "tiny-f32", d=256, E=16, K=2, f=128, fs=128, act="f32", zipf=None, T=4),
    1: Workload(1, "decode-layer-d2816-e128", d=2816, E=128, K=8, f=704, fs=2112, act="bf16",
                zipf=1.0, T=1, steps=1000),
    2: Workload(2, "decode-stack30-d2816-e128", d=2816, E=128, K=8, f=704, fs=2112, act="bf16",
                zipf=1.0, T=1, layers=30, steps=256, noise_sd=0.1),
    3: Workload(3, "prefill-chunk128-d2048-e256", d=2048, E=256, K=8, f=512, fs=512, act="bf16",
                zipf=1.0, T=128, extra_T=(512, 2048)),
    4: Workload(4, "stream-stack40-d2048-e256-lfu16", d=2048, E=256, K=8, f=512, fs=512, act="bf16",
                zipf=1.1, T=1, layers=40, steps=256, noise_sd=0.1, reuse_p=0.6, slots=16),
}


def _rng(seed, wid, layer, tensor):
    return np.random.Generator(np.random.PCG64DXSM(np.random.SeedSequence([seed, wid, layer, tensor])))


def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN-free inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _matrix(seed, wid, layer, name, lead, rows, cols):
    tq, ts, tb = _T_MATS[name]
    shape = tuple(lead) + (rows,)
    n_words = int(np.prod(shape)) * (cols // 8)
    q = (_rng(seed, wid, layer, tq).integers(0, 2**64 - 1, size=(n_words + 1) // 2, dtype=np.uint64,
                                            endpoint=True).view(np.uint32)[:n_words].reshape(shape + (cols // 8,)))
    s = _rng(seed, wid, layer, ts).uniform(0.002, 0.02, size=shape + (cols // GROUP,)).astype(np.float16)
    noise = _rng(seed, wid, layer, tb).normal(0.0, 1e-4, size=s.shape)
    b = (-8.0 * s.astype(np.float64) + noise).astype(np.float16)
    return q, s.view(np.uint16), b.view(np.uint16)


def make_layer(w: Workload, layer: int = 0, seed: int = 0, zipf: float | None = "default") -> dict:
    """All canonical host arrays of one layer (numpy, C-contiguous)."""
    if zipf == "default":
        zipf = w.zipf
    d, E, f, fs = w.d, w.E, w.f, w.fs
    out = {}
    out["router_w"] = _rng(seed, w.wid, layer, _T_ROUTER_W).integers(-127, 128, size=(E, d), dtype=np.int8)
    out["router_scale"] = np.full((E,), 1e-3, dtype=np.float16).view(np.uint16)
    if zipf is None:
        out["router_bias"] = None
    else:
        rank = _rng(seed, w.wid, layer, _T_ROUTER_PERM).permutation(E) + 1
        out["router_bias"] = (-float(zipf) * np.log(rank.astype(np.float64))).astype(np.float32)
    for name, rows, cols in (("gate", f, d), ("up", f, d), ("down", d, f)):
        q, s, b = _matrix(seed, w.wid, layer, name, (E,), rows, cols)
        out[name + "_q"], out[name + "_s"], out[name + "_b"] = q, s, b
    for name, rows, cols in (("sh_gate", fs, d), ("sh_up", fs, d), ("sh_down", d, fs)):
        if fs == 0:
            out[name + "_q"] = out[name + "_s"] = out[name + "_b"] = None
            continue
        q, s, b = _matrix(seed, w.wid, layer, name, (), rows, cols)
        out[name + "_q"], out[name + "_s"], out[name + "_b"] = q, s, b
    return out


def make_tokens(w: Workload, n: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    """n x d tokens ~ N(0,1): float32 array, or uint16 bf16 bit patterns."""
    x = _rng(seed, w.wid, 1000 + stream, _T_TOKENS).standard_normal((n, w.d), dtype=np.float32)
    return x if w.act == "f32" else f32_to_bf16_bits(x)


def make_noise(w: Workload, steps: int, seed: int = 0) -> np.ndarray:
    """Per-step additive noise N(0, noise_sd) for the stack recurrences, fp32 [steps][d]."""
    g = _rng(seed, w.wid, 2000, _T_NOISE)
    return (g.standard_normal((steps, w.d), dtype=np.float32) * np.float32(w.noise_sd)).astype(np.float32)


def make_reuse_coins(w: Workload, steps: int, seed: int = 0) -> np.ndarray:
    """bool [steps][layers]: True where a step reuses the previous step's expert set
    at that layer (probability reuse_p; step 0 never reuses)."""
    g = _rng(seed, w.wid, 3000, _T_REUSE)
    c = g.random((steps, w.layers)) < w.reuse_p
    c[0, :] = False
    return c


def matrix_bytes(rows: int, cols: int) -> int:
    return rows * cols // 2 + rows * (cols // GROUP) * 4


def expert_bytes(w: Workload) -> int:
    return 2 * matrix_bytes(w.f, w.d) + matrix_bytes(w.d, w.f)


def shared_bytes(w: Workload) -> int:
    return 0 if w.fs == 0 else 2 * matrix_bytes(w.fs, w.d) + matrix_bytes(w.d, w.fs)


def router_bytes(w: Workload) -> int:
    return w.E * w.d + w.E * 2 + (w.E * 4 if w.zipf is not None else 0)


def layer_bytes(w: Workload) -> int:
    return w.E * expert_bytes(w) + shared_bytes(w) + router_bytes(w)
