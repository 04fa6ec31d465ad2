"""Python binding of libmoe.so, the gfx950 routed-expert MoE FFN library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions keep the C names of include/moe.h.  Device buffers are
passed as torch tensors (only their data pointers are used) or raw integer
addresses; streams as torch streams, raw hipStream_t integers or None.
The library must have been built (routed_expert_ffn_int8_amd/build.py); if the
shared object is missing and cannot be built, importing fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_NOMEM, MOE_ERR_HIP, MOE_ERR_IO, MOE_ERR_STATE = range(6)
MOE_ACT_F32, MOE_ACT_BF16 = 0, 1
MOE_RESIDENT, MOE_STREAMED = 0, 1
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL, MOE_PATH_FUSED = 0, 1, 2, 3

_STATUS = {1: "MOE_ERR_INVALID", 2: "MOE_ERR_NOMEM", 3: "MOE_ERR_HIP", 4: "MOE_ERR_IO", 5: "MOE_ERR_STATE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_P = C.c_void_p
_WEIGHTS = ["router_w", "router_scale", "router_bias",
            "gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b", "down_q", "down_s", "down_b",
            "sh_gate_q", "sh_gate_s", "sh_gate_b", "sh_up_q", "sh_up_s", "sh_up_b",
            "sh_down_q", "sh_down_s", "sh_down_b"]


class moe_layer_desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("d_model", "n_experts", "top_k", "d_ff", "d_ff_shared",
                                         "act_dtype", "max_tokens", "residency")] + [(n, _P) for n in _WEIGHTS]


class moe_fwd_opts(C.Structure):
    _fields_ = [("topk_ids", _P), ("topk_w", _P), ("forced_ids", _P), ("reuse_previous", C.c_int32),
                ("path", C.c_int32), ("residual", C.c_int32), ("residual_src", _P),
                ("sort_offsets", _P), ("sort_perm", _P)]


class moe_cache_stats(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("accesses", "hits", "misses", "evictions", "h2d_bytes", "h2d_ns",
                                          "prefetches", "prefetch_used", "ahead_slots")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


# name -> argtypes (all return moe_status except moe_last_error)
_SIGS = {
    "moe_layer_create": [C.POINTER(moe_layer_desc), C.POINTER(_P)],
    "moe_layer_destroy": [_P],
    "moe_layer_forward": [_P, _P, _P, C.c_int32, _P],
    "moe_layer_forward_ex": [_P, _P, _P, C.c_int32, C.POINTER(moe_fwd_opts), _P],
    "moe_layer_forward_noalloc": [_P, _P, _P, C.c_int32, _P],
    "moe_layer_route": [_P, _P, _P, _P, C.c_int32, _P],
    "moe_layer_sort": [_P, _P, C.c_int32, _P, _P, _P, _P, _P],
    "moe_layer_bytes": [_P, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)],
    "moe_layer_check_errors": [_P, C.POINTER(C.c_int32)],
    "moe_layer_set_default_path": [_P, C.c_int32],
    "moe_layer_profile": [_P, C.c_int32],
    "moe_layer_profile_read": [_P, _P, _P],
    "moe_cache_attach": [_P, C.c_int32, _P],
    "moe_cache_stats_get": [_P, C.POINTER(moe_cache_stats)],
    "moe_cache_reset": [_P, C.c_int32],
    "moe_cache_contents": [_P, _P, _P],
    "moe_cache_fail_expert": [_P, C.c_int32, C.c_int32],
    "moe_stack_create": [_P, C.c_int32, C.c_float, C.POINTER(_P)],
    "moe_stack_forward": [_P, _P, C.c_int32, _P, _P, _P],
    "moe_stack_destroy": [_P],
    "moe_lfu_create": [C.c_int32, C.POINTER(_P)],
    "moe_lfu_step": [_P, _P, C.c_int32, _P, _P],
    "moe_lfu_stats": [_P, C.POINTER(moe_cache_stats)],
    "moe_lfu_destroy": [_P],
    "moe_lfu_prefetch": [_P, _P, C.c_int32, _P],
    "moe_cache_prefetch": [_P, _P, C.c_int32, _P],
    "moe_stack_set_prefetch": [_P, C.c_int32],
    "moe_lru_create": [C.c_int32, C.POINTER(_P)],
    "moe_lru_step": [_P, C.c_int32, _P, C.c_int32, _P, _P],
    "moe_lru_stats": [_P, C.POINTER(moe_cache_stats)],
    "moe_lru_destroy": [_P],
    "moe_cache_pool_create": [C.c_uint64, C.c_uint64, _P, C.POINTER(_P)],
    "moe_cache_pool_destroy": [_P],
    "moe_cache_attach_pool": [_P, _P],
    "moe_cache_detach": [_P],
    "moe_cache_pool_stats": [_P, C.POINTER(moe_cache_stats)],
    "moe_cache_pool_contents": [_P, _P, _P],
    "moe_debug_dequant": [_P, C.c_int32, C.c_int32, _P],
    "moe_debug_host_wait": [_P, C.c_int64],
}

_lib = None


def load() -> C.CDLL:
    """Load libmoe.so (building it first only if no build exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoe.so is missing at {LIB_PATH}; the HIP library is required")
    # torch ships its own HIP runtime (same soname).  Loading torch first makes
    # the library bind to that copy, so the process holds one HIP runtime and
    # device pointers and streams from torch are valid here.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def exported_symbols() -> list:
    return list(_SIGS) + ["moe_last_error"]


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode(errors="replace"))


def _addr(t) -> int | None:
    """Device/host address of a torch tensor, numpy array or int (None stays None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def moe_last_error() -> str:
    return load().moe_last_error().decode(errors="replace")


# ----------------------------------------------------------------- layers
def make_desc(arrays: dict, d_model, n_experts, top_k, d_ff, d_ff_shared, act_dtype, max_tokens,
              residency=MOE_RESIDENT):
    """Descriptor over canonical HOST numpy arrays.  Returns (desc, keepalive)."""
    keep = {k: (None if v is None else np.ascontiguousarray(v)) for k, v in arrays.items()}
    desc = moe_layer_desc(d_model, n_experts, top_k, d_ff, d_ff_shared, act_dtype, max_tokens, residency)
    for n in _WEIGHTS:
        v = keep.get(n)
        setattr(desc, n, None if v is None else v.ctypes.data)
    return desc, keep


def moe_layer_create(desc: moe_layer_desc) -> int:
    out = _P()
    _check(load().moe_layer_create(C.byref(desc), C.byref(out)))
    return out.value


def moe_layer_destroy(layer: int):
    _check(load().moe_layer_destroy(layer))


def moe_layer_forward(x, layer: int, out, n_tokens: int, stream=None):
    _check(load().moe_layer_forward(_addr(x), layer, _addr(out), n_tokens, _stream(stream)))


def moe_layer_forward_ex(x, layer: int, out, n_tokens: int, opts: moe_fwd_opts | None = None, stream=None):
    _check(load().moe_layer_forward_ex(_addr(x), layer, _addr(out), n_tokens,
                                       None if opts is None else C.byref(opts), _stream(stream)))


def moe_layer_forward_noalloc(x, layer: int, out, n_tokens: int, stream=None):
    _check(load().moe_layer_forward_noalloc(_addr(x), layer, _addr(out), n_tokens, _stream(stream)))


def fwd_opts(topk_ids=None, topk_w=None, forced_ids=None, reuse_previous=0, path=MOE_PATH_AUTO,
             residual_src=None, sort_offsets=None, sort_perm=None) -> moe_fwd_opts:
    return moe_fwd_opts(_addr(topk_ids), _addr(topk_w), _addr(forced_ids), int(reuse_previous), int(path),
                        1 if residual_src is not None else 0, _addr(residual_src),
                        _addr(sort_offsets), _addr(sort_perm))


def moe_layer_route(x, layer: int, ids, w, n_tokens: int, stream=None):
    _check(load().moe_layer_route(_addr(x), layer, _addr(ids), _addr(w), n_tokens, _stream(stream)))


def moe_layer_sort(ids, layer: int, n_tokens: int, counts, offsets, perm, inv, stream=None):
    _check(load().moe_layer_sort(_addr(ids), layer, n_tokens, _addr(counts), _addr(offsets), _addr(perm),
                                 _addr(inv), _stream(stream)))


def moe_layer_bytes(layer: int):
    db, eb = C.c_uint64(), C.c_uint64()
    _check(load().moe_layer_bytes(layer, C.byref(db), C.byref(eb)))
    return db.value, eb.value


def moe_layer_set_default_path(layer: int, path: int):
    _check(load().moe_layer_set_default_path(layer, path))


def moe_layer_check_errors(layer: int) -> int:
    f = C.c_int32()
    _check(load().moe_layer_check_errors(layer, C.byref(f)))
    return f.value


MOE_KERNEL_NAMES = ["route_shared", "routed_gate_up", "down_combine", "sort", "prefill_gate_up",
                    "prefill_down", "prefill_combine", "prefill_route", "topk", "fused_layer"]


def moe_layer_profile(layer: int, enable: bool = True):
    _check(load().moe_layer_profile(layer, 1 if enable else 0))


def moe_layer_profile_read(layer: int) -> dict:
    n = len(MOE_KERNEL_NAMES)
    launches = np.zeros(n, np.int64)
    ms = np.zeros(n, np.float64)
    _check(load().moe_layer_profile_read(layer, launches.ctypes.data, ms.ctypes.data))
    return {MOE_KERNEL_NAMES[i]: (int(launches[i]), float(ms[i])) for i in range(n) if launches[i]}


# ----------------------------------------------------------------- cache
def moe_cache_attach(layer: int, n_slots: int, side_stream=None):
    _check(load().moe_cache_attach(layer, n_slots, _stream(side_stream)))


def moe_cache_stats_get(layer: int) -> dict:
    s = moe_cache_stats()
    _check(load().moe_cache_stats_get(layer, C.byref(s)))
    return s.as_dict()


def moe_cache_reset(layer: int, drop_contents: bool = False):
    _check(load().moe_cache_reset(layer, 1 if drop_contents else 0))


def moe_cache_contents(layer: int, n_slots: int):
    e = np.empty(n_slots, np.int32)
    c = np.empty(n_slots, np.uint32)
    _check(load().moe_cache_contents(layer, e.ctypes.data, c.ctypes.data))
    return e, c


def moe_cache_fail_expert(layer: int, expert: int, fail: bool = True):
    _check(load().moe_cache_fail_expert(layer, expert, 1 if fail else 0))


# ----------------------------------------------------------------- stack
def moe_stack_create(layers: list, rms_eps: float = 1e-6) -> int:
    arr = (_P * len(layers))(*layers)
    out = _P()
    _check(load().moe_stack_create(arr, len(layers), rms_eps, C.byref(out)))
    return out.value


def moe_stack_forward(h, stack: int, n_tokens: int, reuse_mask=None, ids_out=None, stream=None):
    m = None if reuse_mask is None else np.ascontiguousarray(reuse_mask, dtype=np.uint8)
    _check(load().moe_stack_forward(_addr(h), stack, n_tokens, None if m is None else m.ctypes.data,
                                    _addr(ids_out), _stream(stream)))


def moe_stack_destroy(stack: int):
    _check(load().moe_stack_destroy(stack))


# ----------------------------------------------------------------- host policy
def moe_lfu_create(n_slots: int) -> int:
    out = _P()
    _check(load().moe_lfu_create(n_slots, C.byref(out)))
    return out.value


def moe_lfu_step(lfu: int, chosen):
    c = np.ascontiguousarray(chosen, dtype=np.int32)
    slot = np.empty(len(c), np.int32)
    miss = np.empty(len(c), np.int32)
    _check(load().moe_lfu_step(lfu, c.ctypes.data, len(c), slot.ctypes.data, miss.ctypes.data))
    return slot, miss


def moe_lfu_stats(lfu: int) -> dict:
    s = moe_cache_stats()
    _check(load().moe_lfu_stats(lfu, C.byref(s)))
    return s.as_dict()


def moe_lfu_destroy(lfu: int):
    _check(load().moe_lfu_destroy(lfu))


def moe_lfu_prefetch(lfu: int, experts):
    e = np.ascontiguousarray(experts, dtype=np.int32)
    slot = np.empty(max(1, len(e)), np.int32)
    _check(load().moe_lfu_prefetch(lfu, e.ctypes.data, len(e), slot.ctypes.data))
    return slot[:len(e)]


def moe_cache_prefetch(layer: int, experts, stream=None):
    e = np.ascontiguousarray(experts, dtype=np.int32)
    _check(load().moe_cache_prefetch(layer, e.ctypes.data, len(e), _stream(stream)))


def moe_stack_set_prefetch(stack: int, depth: int):
    _check(load().moe_stack_set_prefetch(stack, depth))


def moe_lru_create(n_slots: int) -> int:
    out = _P()
    _check(load().moe_lru_create(n_slots, C.byref(out)))
    return out.value


def moe_lru_step(lru: int, layer: int, chosen):
    c = np.ascontiguousarray(chosen, dtype=np.int32)
    slot = np.empty(len(c), np.int32)
    miss = np.empty(len(c), np.int32)
    _check(load().moe_lru_step(lru, layer, c.ctypes.data, len(c), slot.ctypes.data, miss.ctypes.data))
    return slot, miss


def moe_lru_stats(lru: int) -> dict:
    s = moe_cache_stats()
    _check(load().moe_lru_stats(lru, C.byref(s)))
    return s.as_dict()


def moe_lru_destroy(lru: int):
    _check(load().moe_lru_destroy(lru))


# ------------------------------------------------------- shared cache pool
def moe_cache_pool_create(budget_bytes: int, expert_bytes: int, side_stream=None) -> int:
    out = _P()
    _check(load().moe_cache_pool_create(budget_bytes, expert_bytes, _stream(side_stream), C.byref(out)))
    return out.value


def moe_cache_pool_destroy(pool: int):
    _check(load().moe_cache_pool_destroy(pool))


def moe_cache_attach_pool(layer: int, pool: int):
    _check(load().moe_cache_attach_pool(layer, pool))


def moe_cache_detach(layer: int):
    _check(load().moe_cache_detach(layer))


def moe_cache_pool_stats(pool: int) -> dict:
    s = moe_cache_stats()
    _check(load().moe_cache_pool_stats(pool, C.byref(s)))
    return s.as_dict()


def moe_cache_pool_contents(pool: int, n_slots: int):
    lay = np.empty(n_slots, np.int32)
    exp = np.empty(n_slots, np.int32)
    _check(load().moe_cache_pool_contents(pool, lay.ctypes.data, exp.ctypes.data))
    return lay, exp


# ----------------------------------------------------------------- test hooks
def moe_debug_dequant(layer: int, which: int, expert: int, rows: int, cols: int) -> np.ndarray:
    """fp32 [rows][cols] of matrix `which` (0 gate, 1 up, 2 down) of `expert`
    (-1 = shared), dequantised on the GPU from the device layout."""
    out = np.empty((rows, cols), np.float32)
    _check(load().moe_debug_dequant(layer, which, expert, out.ctypes.data))
    return out


def moe_debug_host_wait(layer: int, microseconds: int):
    _check(load().moe_debug_host_wait(layer, int(microseconds)))
