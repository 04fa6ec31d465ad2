"""ctypes front-end of the plain-C fp64 oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the benchmark).
Inputs are the canonical host arrays of one layer; stored bf16/fp32 tokens are
widened exactly to fp64 before the call.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (plain C, OpenMP over output rows)."""
    src = os.path.join(_HERE, "moe_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("d", "E", "K", "f", "fs")] + [
        ("router_w", C.c_void_p), ("router_scale", C.c_void_p), ("router_bias", C.c_void_p),
        ("gate_q", C.c_void_p), ("up_q", C.c_void_p), ("down_q", C.c_void_p),
        ("gate_s", C.c_void_p), ("gate_b", C.c_void_p), ("up_s", C.c_void_p), ("up_b", C.c_void_p),
        ("down_s", C.c_void_p), ("down_b", C.c_void_p),
        ("sh_gate_q", C.c_void_p), ("sh_up_q", C.c_void_p), ("sh_down_q", C.c_void_p),
        ("sh_gate_s", C.c_void_p), ("sh_gate_b", C.c_void_p), ("sh_up_s", C.c_void_p),
        ("sh_up_b", C.c_void_p), ("sh_down_s", C.c_void_p), ("sh_down_b", C.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P, I = C.c_void_p, C.c_int
        L.oracle_threads.restype = C.c_int
        L.oracle_threads.argtypes = []
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_f16_to_f64.restype = C.c_double
        L.oracle_f16_to_f64.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f64.restype = C.c_double
        L.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.oracle_f64_to_bf16.restype = C.c_uint16
        L.oracle_f64_to_bf16.argtypes = [C.c_double]
        L.oracle_dequant.argtypes = [P, P, P, I, I, P]
        L.oracle_router_logits.argtypes = [P, P, I, P]
        L.oracle_select_one.argtypes = [P, I, I, P, P, P]
        L.oracle_weights_for_set.argtypes = [P, P, I, P]
        L.oracle_expert.argtypes = [P, I, P, P]
        L.oracle_layer_forward.argtypes = [P, P, I, P, P, P, P, P]
        L.oracle_sort.argtypes = [P, I, I, I, P, P, P, P]
        L.oracle_rmsnorm_bf16.argtypes = [P, I, C.c_double, P]
        L.oracle_residual_bf16.argtypes = [P, P, I, P]
        L.oracle_stack_step.argtypes = [P, I, C.c_double, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def tokens_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of stored tokens: float32 as is, uint16 as bf16 bit patterns."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


class OracleLayer:
    """Holds one layer's canonical arrays and the C descriptor pointing at them."""

    def __init__(self, arrays: dict, d: int, E: int, K: int, f: int, fs: int):
        self.arrays = {k: (None if v is None else np.ascontiguousarray(v)) for k, v in arrays.items()}
        a = self.arrays
        self.d, self.E, self.K, self.f, self.fs = d, E, K, f, fs
        s = _Layer(d, E, K, f, fs)
        for name, _ in _Layer._fields_[5:]:
            setattr(s, name, _p(a.get(name)))
        self.struct = s

    @classmethod
    def from_workload(cls, w, arrays):
        return cls(arrays, w.d, w.E, w.K, w.f, w.fs)

    @property
    def ptr(self):
        return C.addressof(self.struct)

    def logits(self, x):
        x64 = np.ascontiguousarray(tokens_to_f64(x).reshape(-1, self.d))
        out = np.empty((x64.shape[0], self.E), np.float64)
        lib().oracle_router_logits(self.ptr, _p(x64), x64.shape[0], _p(out))
        return out

    def expert(self, e, x):
        x64 = np.ascontiguousarray(tokens_to_f64(x).reshape(self.d))
        out = np.empty(self.d, np.float64)
        lib().oracle_expert(self.ptr, int(e), _p(x64), _p(out))
        return out

    def forward(self, x, forced=None):
        """Returns (y fp64 [T,d], ids int32 [T,K], w fp64 [T,K], margin fp64 [T])."""
        x64 = np.ascontiguousarray(tokens_to_f64(x).reshape(-1, self.d))
        T = x64.shape[0]
        y = np.empty((T, self.d), np.float64)
        ids = np.empty((T, self.K), np.int32)
        w = np.empty((T, self.K), np.float64)
        m = np.empty((T,), np.float64)
        fz = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32).reshape(T, self.K)
        rc = lib().oracle_layer_forward(self.ptr, _p(x64), T, _p(fz), _p(y), _p(ids), _p(w), _p(m))
        if rc:
            raise ValueError("oracle_layer_forward rejected the layer shape")
        return y, ids, w, m


def select(logits_row: np.ndarray, K: int):
    l = np.ascontiguousarray(logits_row, dtype=np.float64)
    ids = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    m = np.empty(1, np.float64)
    lib().oracle_select_one(_p(l), l.shape[0], K, _p(ids), _p(w), _p(m))
    return ids, w, float(m[0])


def dequant(q, s, b):
    rows, cols = q.shape[0], q.shape[1] * 8
    W = np.empty((rows, cols), np.float64)
    lib().oracle_dequant(_p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)), _p(np.ascontiguousarray(b)),
                         rows, cols, _p(W))
    return W


def sort(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    inv = np.empty(T * K, np.int32)
    lib().oracle_sort(_p(ids), T, K, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(int(h))


def f64_to_bf16(v: float) -> int:
    return lib().oracle_f64_to_bf16(float(v))


def rmsnorm_bf16(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    n = np.empty_like(h)
    lib().oracle_rmsnorm_bf16(_p(h), h.shape[0], eps, _p(n))
    return n


def residual_bf16(h: np.ndarray, y: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty_like(h)
    lib().oracle_residual_bf16(_p(h), _p(y), h.shape[0], _p(out))
    return out


def stack_step(layers: list, h: np.ndarray, eps: float = 1e-6, forced=None):
    """One token through all layers: h <- bf16(h + MoE(bf16(rmsnorm(h)))).
    Returns (new h bf16 bits, ids [n_layers][K])."""
    n = len(layers)
    arr = (_Layer * n)(*[l.struct for l in layers])
    h = np.array(h, dtype=np.uint16, copy=True)
    K = layers[0].K
    ids = np.empty((n, K), np.int32)
    fz = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32).reshape(n, K)
    rc = lib().oracle_stack_step(C.addressof(arr), n, eps, _p(h), _p(fz), _p(ids))
    if rc:
        raise ValueError("oracle_stack_step failed")
    return h, ids
