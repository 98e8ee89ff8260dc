"""ctypes binding of libmoe_hip.so (argument marshalling only).

Every function has the name and argument order of the C ABI in
include/*.h and takes torch tensors (device memory) or raw device pointers.
All computation happens in the HIP library; if it cannot be loaded, import of
this module's functions raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_hip.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_EALIGN = -4
MOE_EDEVICE = -5

MOE_ACT_F32 = 0
MOE_ACT_BF16 = 1

MOE_MAX_DIM = 131072  # d, I and I_shared must be below this

# moe_forward's diagnostic counters
MOE_DIAG_H_FP16_NONFINITE = 0
MOE_DIAG_COUNT = 1

MOE_FLAG_BATCH_INVARIANT = 1

MOE_ROUTER_SIGMOID_BIAS = 0
MOE_ROUTER_SOFTMAX = 1
MOE_ROUTER_EXPERT_CHOICE = 2

MOE_PATH_AUTO = 0
MOE_PATH_GEMV = 1
MOE_PATH_GEMM = 2
MOE_AUTO_DECODE_MAX_T = 40  # MOE_PATH_AUTO: the decode kernels up to this T, the matrix-core path above

MOE_CACHE_WEIGHTED_LRU = 0
MOE_CACHE_LRU = 1

# names declared in include/*.h
EXPORTS = ("moe_workspace_size", "moe_route", "moe_permute", "moe_forward", "moe_forward_static", "moe_combine",
           "moe_last_error", "moe_abi_version", "dsa_index_workspace_size", "dsa_index_topk",
           "moe_cache_state_size", "moe_cache_init", "moe_cache_plan", "moe_cache_fetch", "moe_forward_cached",
           "moe_cache_stats", "moe_route_permute", "moe_layer")

MOE_STATIC_SCRATCH_BYTES = 64 << 20  # moe_forward_static's scratch


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class moe_shape(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32), ("I", C.c_int32),
                ("I_shared", C.c_int32), ("routed_scale", C.c_float), ("act_dtype", C.c_int32),
                ("wbits", C.c_int32), ("path", C.c_int32), ("flags", C.c_int32), ("router", C.c_int32),
                ("capacity_factor", C.c_float)]


class dsa_index_shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "S", "H", "D", "K", "pos0")]


class moe_cache_shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("E", "slots", "pinned", "policy")]


class moe_qffn(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down")]


_lib = None


def lib():
    """Load the HIP library (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m routed_expert_ffn_sigmoid_amd.build")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        S = C.POINTER(moe_shape)
        Q = C.POINTER(moe_qffn)
        L.moe_workspace_size.argtypes = [S]
        L.moe_workspace_size.restype = C.c_size_t
        L.moe_route.argtypes = [S, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_permute.argtypes = [S, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_forward.argtypes = [S, P, Q, Q, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_forward_static.argtypes = [S, P, Q, Q, P, P, P, P, P, P, P, P]
        L.moe_combine.argtypes = [S, P, P, P, P, P, P]
        for f in ("moe_route", "moe_permute", "moe_forward", "moe_forward_static", "moe_combine", "moe_abi_version"):
            getattr(L, f).restype = C.c_int
        L.moe_last_error.restype = C.c_char_p
        X = C.POINTER(dsa_index_shape)
        L.dsa_index_workspace_size.argtypes = [X]
        L.dsa_index_workspace_size.restype = C.c_size_t
        L.dsa_index_topk.argtypes = [X, P, P, P, P, P, P, P, C.c_size_t, P]
        L.dsa_index_topk.restype = C.c_int
        K = C.POINTER(moe_cache_shape)
        I32 = C.c_int32
        L.moe_cache_state_size.argtypes = [K]
        L.moe_cache_state_size.restype = C.c_size_t
        L.moe_cache_init.argtypes = [K, P, P, P, P, P]
        L.moe_cache_plan.argtypes = [K, I32, I32, P, P, P, P, P, P, P, P]
        L.moe_cache_fetch.argtypes = [S, K, Q, Q, P, P, P, P]
        L.moe_forward_cached.argtypes = [S, K, P, Q, P, Q, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_cache_stats.argtypes = [K, P, P, P, P]
        for f in ("moe_cache_init", "moe_cache_plan", "moe_cache_fetch", "moe_forward_cached", "moe_cache_stats"):
            getattr(L, f).restype = C.c_int
        L.moe_route_permute.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_route_permute.restype = C.c_int
        L.moe_layer.argtypes = [S, P, P, P, Q, Q, P, P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
        L.moe_layer.restype = C.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def make_shape(T, d, E, k, I, I_shared=0, routed_scale=1.0, act_dtype=MOE_ACT_BF16, wbits=4,
               path=MOE_PATH_AUTO, flags=0, router=0, capacity_factor=0.0) -> moe_shape:
    return moe_shape(T, d, E, k, I, I_shared, routed_scale, act_dtype, wbits, path, flags, router, capacity_factor)


def make_qffn(q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up, z_down) -> moe_qffn:
    return moe_qffn(*[_ptr(t) for t in (q_gate, q_up, q_down, s_gate, s_up, s_down, z_gate, z_up, z_down)])


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_workspace_size(shape: moe_shape) -> int:
    return int(lib().moe_workspace_size(C.byref(shape)))


def moe_route(shape, x, W_r, bias, topk_idx, topk_w, gap, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_route(C.byref(shape), _ptr(x), _ptr(W_r), _ptr(bias), _ptr(topk_idx), _ptr(topk_w),
                           _ptr(gap), _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(shape, topk_idx, counts, offsets, perm, inv, uniq, n_uniq, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_permute(C.byref(shape), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
                             _ptr(uniq), _ptr(n_uniq), _ptr(ws), ws_bytes, _stream(stream)))


def moe_forward(shape, x, routed: moe_qffn, shared: Optional[moe_qffn], offsets, perm, uniq, n_uniq, y_perm,
                y_shared, diag, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_forward(C.byref(shape), _ptr(x), C.byref(routed),
                             C.byref(shared) if shared is not None else None, _ptr(offsets), _ptr(perm),
                             _ptr(uniq), _ptr(n_uniq), _ptr(y_perm), _ptr(y_shared), _ptr(diag), _ptr(ws),
                             ws_bytes, _stream(stream)))


def moe_forward_static(shape, x, routed: moe_qffn, shared: Optional[moe_qffn], offsets, perm, uniq, n_uniq, y_perm,
                       y_shared, diag, stream=None) -> None:
    _check(lib().moe_forward_static(C.byref(shape), _ptr(x), C.byref(routed),
                                    C.byref(shared) if shared is not None else None, _ptr(offsets), _ptr(perm),
                                    _ptr(uniq), _ptr(n_uniq), _ptr(y_perm), _ptr(y_shared), _ptr(diag),
                                    _stream(stream)))


def moe_route_permute(shape, x, W_r, bias, topk_idx, topk_w, gap, counts, offsets, perm, inv, uniq, n_uniq, ws,
                      ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_route_permute(C.byref(shape), _ptr(x), _ptr(W_r), _ptr(bias), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(gap), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(uniq),
                                   _ptr(n_uniq), _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer(shape, x, W_r, bias, routed: moe_qffn, shared: Optional[moe_qffn], topk_idx, topk_w, gap, counts,
              offsets, perm, inv, uniq, n_uniq, y_perm, y_shared, y, diag, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_layer(C.byref(shape), _ptr(x), _ptr(W_r), _ptr(bias), C.byref(routed),
                           C.byref(shared) if shared is not None else None, _ptr(topk_idx), _ptr(topk_w), _ptr(gap),
                           _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(uniq), _ptr(n_uniq),
                           _ptr(y_perm), _ptr(y_shared), _ptr(y), _ptr(diag), _ptr(ws), ws_bytes, _stream(stream)))


def moe_combine(shape, y_perm, y_shared, inv, topk_w, y, stream=None) -> None:
    _check(lib().moe_combine(C.byref(shape), _ptr(y_perm), _ptr(y_shared), _ptr(inv), _ptr(topk_w), _ptr(y),
                             _stream(stream)))


def dsa_index_workspace_size(shape: dsa_index_shape) -> int:
    return int(lib().dsa_index_workspace_size(C.byref(shape)))


def dsa_index_topk(shape, q, w, k, kscale, top, gap, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().dsa_index_topk(C.byref(shape), _ptr(q), _ptr(w), _ptr(k), _ptr(kscale), _ptr(top), _ptr(gap),
                                _ptr(ws), ws_bytes, _stream(stream)))


def make_cache_shape(E, slots, pinned=0, policy=MOE_CACHE_WEIGHTED_LRU) -> moe_cache_shape:
    return moe_cache_shape(E, slots, pinned, policy)


def moe_cache_state_size(cache: moe_cache_shape) -> int:
    return int(lib().moe_cache_state_size(C.byref(cache)))


def moe_cache_init(cache, pinned_ids, state, miss, n_miss, stream=None) -> None:
    """pinned_ids: a sequence of ints (host), or None when cache.pinned == 0."""
    arr = None
    if pinned_ids is not None and len(pinned_ids):
        arr = (C.c_int32 * len(pinned_ids))(*[int(v) for v in pinned_ids])
    _check(lib().moe_cache_init(C.byref(cache), C.cast(arr, C.c_void_p) if arr is not None else None, _ptr(state),
                                _ptr(miss), _ptr(n_miss), _stream(stream)))


def moe_cache_plan(cache, T, k, uniq, n_uniq, state, hit, n_hit, miss, n_miss, stream=None) -> None:
    _check(lib().moe_cache_plan(C.byref(cache), int(T), int(k), _ptr(uniq), _ptr(n_uniq), _ptr(state), _ptr(hit),
                                _ptr(n_hit), _ptr(miss), _ptr(n_miss), _stream(stream)))


def moe_cache_fetch(shape, cache, host_tier: moe_qffn, slots: moe_qffn, state, miss, n_miss, stream=None) -> None:
    _check(lib().moe_cache_fetch(C.byref(shape), C.byref(cache), C.byref(host_tier), C.byref(slots), _ptr(state),
                                 _ptr(miss), _ptr(n_miss), _stream(stream)))


def moe_forward_cached(shape, cache, x, slots: moe_qffn, state, shared: Optional[moe_qffn], offsets, perm, lst,
                       n_list, y_perm, y_shared, diag, ws, ws_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().moe_forward_cached(C.byref(shape), C.byref(cache), _ptr(x), C.byref(slots), _ptr(state),
                                    C.byref(shared) if shared is not None else None, _ptr(offsets), _ptr(perm),
                                    _ptr(lst), _ptr(n_list), _ptr(y_perm), _ptr(y_shared), _ptr(diag), _ptr(ws),
                                    ws_bytes, _stream(stream)))


def moe_cache_stats(cache, state, want_slots: bool = False, stream=None):
    """(steps, hits, misses, evictions, unplaced) and, with want_slots, each slot's expert (a list)."""
    out = (C.c_int64 * 5)()
    se = (C.c_int32 * cache.slots)() if want_slots else None
    _check(lib().moe_cache_stats(C.byref(cache), _ptr(state), C.cast(out, C.c_void_p),
                                 C.cast(se, C.c_void_p) if se is not None else None, _stream(stream)))
    stats = tuple(int(v) for v in out)
    return (stats, list(se)) if want_slots else stats
