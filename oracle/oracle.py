"""ctypes wrapper of the C oracle (test infrastructure only).

Every function takes and returns numpy arrays; the arithmetic is all in
moe_oracle.c.  Only tests/, the smoke check and the benchmark's CPU-baseline
leg import this module.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

_lib = None

P = C.c_void_p


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(_build.ensure_built())
        _lib.oracle_set_threads.argtypes = [C.c_int]
        _lib.oracle_max_threads.restype = C.c_int
        _lib.oracle_decode_act.argtypes = [P, C.c_int, C.c_long, P]
        _lib.oracle_router_logits.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P]
        _lib.oracle_router_select.argtypes = [C.c_int, C.c_int, C.c_int, P, P, C.c_double, P, P, P, P, P]
        _lib.oracle_permute.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P, P, P]
        _lib.oracle_expert_apply.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int] + [P] * 9 + [P, P, P]
        _lib.oracle_combine.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P]
        _lib.oracle_moe_layer.argtypes = ([C.c_int] * 7 + [C.c_double, C.c_int] + [P] * 5 + [P] * 12)
        _lib.oracle_moe_tokens.argtypes = ([C.c_int, P] + [C.c_int] * 6 + [C.c_double, C.c_int] + [P] * 5 + [P] * 4)
        _lib.oracle_router_select_softmax.argtypes = [C.c_int, C.c_int, C.c_int, P, C.c_double, P, P, P]
        _lib.oracle_capacity.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P]
        _lib.oracle_expert_choice.argtypes = [C.c_int, C.c_int, C.c_int, P, C.c_double, P, P, P]
        _lib.oracle_index_topk.argtypes = [C.c_int] * 6 + [P] * 7
        _lib.oracle_cache_init.argtypes = [C.c_int] * 3 + [P] * 5
        _lib.oracle_cache_step.argtypes = [C.c_int] * 4 + [C.c_int64] + [P] * 4 + [C.c_int] + [P] * 6
        _lib.oracle_cache_step.restype = C.c_int
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


class _QFFN(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down")]


def _qffn(ws) -> Optional[_QFFN]:
    if ws is None:
        return None
    s = _QFFN()
    for n, _ in _QFFN._fields_:
        setattr(s, n, getattr(ws, n).ctypes.data)
    return s


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def decode_act(x: np.ndarray, act: int) -> np.ndarray:
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_decode_act(_p(x), int(act), x.size, _p(out))
    return out


def router_logits(xd: np.ndarray, W_r: np.ndarray) -> np.ndarray:
    xd = np.ascontiguousarray(xd, dtype=np.float64)
    W_r = np.ascontiguousarray(W_r, dtype=np.float32)
    T, d = xd.shape
    E = W_r.shape[1]
    z = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(T, d, E, _p(xd), _p(W_r), _p(z))
    return z


@dataclass
class Routing:
    idx: np.ndarray   # [T][k] int32
    w: np.ndarray     # [T][k] fp32
    gap: np.ndarray   # [T] fp64
    s: np.ndarray     # [T][E] fp64 sigmoid scores
    sel: np.ndarray   # [T][E] fp64 selection scores


def router_select(z: np.ndarray, bias: np.ndarray, k: int, lam: float) -> Routing:
    z = np.ascontiguousarray(z, dtype=np.float64)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    gap = np.empty(T, dtype=np.float64)
    s = np.empty((T, E), dtype=np.float64)
    sel = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_select(T, E, k, _p(z), _p(bias), float(lam), _p(idx), _p(w), _p(gap), _p(s), _p(sel))
    return Routing(idx, w, gap, s, sel)


@dataclass
class Permutation:
    counts: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray
    inv: np.ndarray
    uniq: np.ndarray
    n_uniq: int


def permute(idx: np.ndarray, E: int) -> Permutation:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    A = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(A, np.int32)
    inv = np.empty(A, np.int32)
    uniq = np.empty(E, np.int32)
    n = np.zeros(1, np.int32)
    lib().oracle_permute(T, k, E, _p(idx), _p(counts), _p(offsets), _p(perm), _p(inv), _p(uniq), _p(n))
    return Permutation(counts, offsets, perm, inv, uniq, int(n[0]))


def expert_apply(X: np.ndarray, d: int, I: int, wbits: int, ws, e: int, return_h: bool = False):
    """Apply expert e of a stacked expert set (synth.QExpertSet layout) to rows X [n][d] (fp64)."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    n = X.shape[0]
    Y = np.empty((n, d), dtype=np.float64)
    H = np.empty((n, I), dtype=np.float64) if return_h else None
    args = [np.ascontiguousarray(a[e]) for a in
            (ws.q_gate, ws.s_gate, ws.z_gate, ws.q_up, ws.s_up, ws.z_up, ws.q_down, ws.s_down, ws.z_down)]
    lib().oracle_expert_apply(n, d, I, wbits, *[_p(a) for a in args], _p(X), _p(Y), _p(H))
    return (Y, H) if return_h else Y


def combine(Y: np.ndarray, S: Optional[np.ndarray], inv: np.ndarray, w: np.ndarray) -> np.ndarray:
    T, k = w.shape
    d = Y.shape[1]
    y = np.empty((T, d), dtype=np.float64)
    lib().oracle_combine(T, k, d, _p(np.ascontiguousarray(Y, dtype=np.float64)),
                         _p(None if S is None else np.ascontiguousarray(S, dtype=np.float64)),
                         _p(np.ascontiguousarray(inv, dtype=np.int32)),
                         _p(np.ascontiguousarray(w, dtype=np.float32)), _p(y))
    return y


@dataclass
class LayerResult:
    idx: np.ndarray
    w: np.ndarray
    gap: np.ndarray
    perm: Permutation
    Yperm: np.ndarray
    S: Optional[np.ndarray]
    y: np.ndarray


def moe_layer(spec, x, W_r, bias, routed, shared) -> LayerResult:
    """Whole layer through the batch union (spec: synth.LayerSpec)."""
    T = x.shape[0]
    d, E, k, I, Is = spec.d, spec.E, spec.k, spec.I, spec.I_shared
    A = T * k
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    gap = np.empty(T, np.float64)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(A, np.int32)
    inv = np.empty(A, np.int32)
    uniq = np.empty(E, np.int32)
    n = np.zeros(1, np.int32)
    Yperm = np.empty((A, d), np.float64)
    S = np.empty((T, d), np.float64) if Is > 0 else None
    y = np.empty((T, d), np.float64)
    r = _qffn(routed)
    s = _qffn(shared)
    lib().oracle_moe_layer(T, d, E, k, I, Is, spec.wbits, float(spec.routed_scale), spec.act,
                           _p(np.ascontiguousarray(x)), _p(W_r), _p(bias), C.byref(r),
                           C.byref(s) if s is not None else None,
                           _p(idx), _p(w), _p(gap), _p(counts), _p(offsets), _p(perm), _p(inv), _p(uniq),
                           _p(n), _p(Yperm), _p(S), _p(y))
    return LayerResult(idx, w, gap, Permutation(counts, offsets, perm, inv, uniq, int(n[0])), Yperm, S, y)


@dataclass
class TokenResult:
    tokens: np.ndarray
    idx: np.ndarray
    w: np.ndarray
    gap: np.ndarray
    y: np.ndarray


def moe_tokens(spec, tokens, x, W_r, bias, routed, shared) -> TokenResult:
    """Per-token loop (no batch union) over the listed rows of x."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = tokens.size
    d, E, k = spec.d, spec.E, spec.k
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float32)
    gap = np.empty(n, np.float64)
    y = np.empty((n, d), np.float64)
    r = _qffn(routed)
    s = _qffn(shared)
    lib().oracle_moe_tokens(n, _p(tokens), d, E, k, spec.I, spec.I_shared, spec.wbits,
                            float(spec.routed_scale), spec.act, _p(np.ascontiguousarray(x)), _p(W_r), _p(bias),
                            C.byref(r), C.byref(s) if s is not None else None,
                            _p(idx), _p(w), _p(gap), _p(y))
    return TokenResult(tokens, idx, w, gap, y)


# ----------------------------------------------------------------------------
# router variants (softmax top-k, capacity, expert choice)
# ----------------------------------------------------------------------------

ROUTER_SIGMOID_BIAS = 0
ROUTER_SOFTMAX = 1
ROUTER_EXPERT_CHOICE = 2


def router_select_softmax(z: np.ndarray, k: int, lam: float) -> Routing:
    """Softmax top-k: the k largest logits (ties to the lower id), weights lambda * softmax renormalised over them;
    gap in logit units.  s and sel are not produced (None)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    gap = np.empty(T, dtype=np.float64)
    lib().oracle_router_select_softmax(T, E, k, _p(z), float(lam), _p(idx), _p(w), _p(gap))
    return Routing(idx, w, gap, None, None)


def capacity_of(T: int, k: int, E: int, cf: float) -> int:
    """C = ceil(cf * T * k / E) with cf as the fp32 value the ABI carries."""
    return int(np.ceil(float(np.float32(cf)) * T * k / E))


def capacity(idx: np.ndarray, E: int, C: int) -> np.ndarray:
    """A copy of idx [T][k] in which every expert keeps at most C assignments (choice-major, then token order)."""
    out = np.ascontiguousarray(idx, dtype=np.int32).copy()
    T, k = out.shape
    lib().oracle_capacity(T, k, E, int(C), _p(out))
    return out


def expert_choice_capacity(T: int, E: int, cf: float) -> int:
    """C = min(T, ceil(cf * T / E)) with cf as the fp32 value the ABI carries."""
    return min(T, int(np.ceil(float(np.float32(cf)) * T / E)))


def expert_choice(z: np.ndarray, C: int, lam: float):
    """Expert choice: per expert the C tokens of largest softmax probability.  Returns (idx [T][E], w [T][E],
    gap_e [E])."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, E = z.shape
    idx = np.empty((T, E), dtype=np.int32)
    w = np.empty((T, E), dtype=np.float32)
    gap = np.empty(E, dtype=np.float64)
    lib().oracle_expert_choice(T, E, int(C), _p(z), float(lam), _p(idx), _p(w), _p(gap))
    return idx, w, gap


def route_variant(spec, x, W_r, bias, router: int, capacity_factor: float = 0.0):
    """Routing of a layer under one of the router variants: (idx, w, gap).  gap is per token for the top-k routers
    and per expert for expert choice."""
    z = router_logits(decode_act(x, spec.act), W_r)
    T = z.shape[0]
    if router == ROUTER_EXPERT_CHOICE:
        return expert_choice(z, expert_choice_capacity(T, spec.E, capacity_factor), spec.routed_scale)
    if router == ROUTER_SOFTMAX:
        r = router_select_softmax(z, spec.k, spec.routed_scale)
    else:
        r = router_select(z, bias, spec.k, spec.routed_scale)
    idx = r.idx
    if capacity_factor > 0:
        idx = capacity(idx, spec.E, capacity_of(T, spec.k, spec.E, capacity_factor))
    return idx, r.w, r.gap


def moe_layer_routed(spec, x, idx, w, routed, shared, k=None):
    """The rest of the layer for a given routing idx/w [T][k] (empty slots -1): batch union, experts, shared expert,
    combine, each by the oracle functions above.  k defaults to spec.k (expert choice passes E)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T = idx.shape[0]
    k = idx.shape[1] if k is None else k
    xd = decode_act(x, spec.act)
    p = permute(idx, spec.E)
    Yperm = np.zeros((T * k, spec.d))
    for u in range(p.n_uniq):
        e = int(p.uniq[u])
        rows = p.perm[p.offsets[e]:p.offsets[e + 1]]
        Yperm[p.offsets[e]:p.offsets[e + 1]] = expert_apply(xd[rows // k], spec.d, spec.I, spec.wbits, routed, e)
    S = expert_apply(xd, spec.d, spec.I_shared, spec.wbits, shared, 0) if spec.I_shared else None
    y = combine(Yperm, S, p.inv, w)
    return p, Yperm, S, y


# ----------------------------------------------------------------------------
# sparse-attention indexer: scores and top-K causal keys
# ----------------------------------------------------------------------------


@dataclass
class IndexTopk:
    top: np.ndarray     # [T][K] int32, ascending positions, -1 padded
    gap: np.ndarray     # [T] fp64
    scores: Optional[np.ndarray]  # [T][S] fp64 (0 where not visible)


def index_topk(q: np.ndarray, w: np.ndarray, k: np.ndarray, kscale: np.ndarray, K: int, pos0: int,
               want_scores: bool = False) -> IndexTopk:
    """q [T][H][D] int8, w [T][H] fp32, k [S][D] int8, kscale [S] fp32; query t sees keys s <= pos0 + t."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.int8)
    kscale = np.ascontiguousarray(kscale, dtype=np.float32)
    T, H, D = q.shape
    S = k.shape[0]
    top = np.empty((T, K), np.int32)
    gap = np.empty(T, np.float64)
    sc = np.empty((T, S), np.float64) if want_scores else None
    lib().oracle_index_topk(T, S, H, D, K, pos0, _p(q), _p(w), _p(k), _p(kscale), _p(top), _p(gap), _p(sc))
    return IndexTopk(top, gap, sc)


# ----------------------------------------------------------------------------
# expert residency: weighted-LRU cache of HBM slots
# ----------------------------------------------------------------------------

CACHE_WEIGHTED_LRU = 0
CACHE_LRU = 1


@dataclass
class CacheStep:
    hits: np.ndarray     # experts of the step already resident, ascending
    misses: np.ndarray   # experts copied in this step, ascending
    evicted: np.ndarray  # per miss: the expert its slot held before (-1: the slot was empty)


class ExpertCache:
    """State of one layer's slots: slot_expert [S], expert_slot [E], last_used [S], hits [S], and the step count."""

    def __init__(self, E: int, S: int, pinned=(), policy: int = CACHE_WEIGHTED_LRU):
        pinned = np.ascontiguousarray(pinned, dtype=np.int32)
        if not 0 < S <= E or pinned.size > S or len(set(pinned.tolist())) != pinned.size:
            raise ValueError("bad cache shape")
        if pinned.size and (pinned.min() < 0 or pinned.max() >= E):
            raise ValueError("pinned expert out of range")
        self.E, self.S, self.P, self.policy = E, S, int(pinned.size), policy
        self.slot_expert = np.empty(S, np.int32)
        self.expert_slot = np.empty(E, np.int32)
        self.last_used = np.empty(S, np.int64)
        self.hits = np.empty(S, np.int64)
        self.now = 0
        self.n_hits = self.n_misses = self.n_evictions = 0
        lib().oracle_cache_init(E, S, self.P, _p(pinned), _p(self.slot_expert), _p(self.expert_slot),
                                _p(self.last_used), _p(self.hits))

    def step(self, uniq) -> CacheStep:
        """One layer call whose tokens chose the experts in uniq (the batch union, any order)."""
        u = np.unique(np.ascontiguousarray(uniq, dtype=np.int32))
        hit = np.empty(max(u.size, 1), np.int32)
        miss = np.empty(max(u.size, 1), np.int32)
        ev = np.empty(max(u.size, 1), np.int32)
        nh = np.zeros(1, np.int32)
        nm = np.zeros(1, np.int32)
        self.now += 1
        rc = lib().oracle_cache_step(self.E, self.S, self.P, self.policy, self.now, _p(self.slot_expert),
                                     _p(self.expert_slot), _p(self.last_used), _p(self.hits), int(u.size), _p(u),
                                     _p(hit), _p(nh), _p(miss), _p(nm), _p(ev))
        if rc != 0:
            raise RuntimeError("a step's misses exceed the evictable slots")
        r = CacheStep(hit[:nh[0]].copy(), miss[:nm[0]].copy(), ev[:nm[0]].copy())
        self.n_hits += r.hits.size
        self.n_misses += r.misses.size
        self.n_evictions += int((r.evicted >= 0).sum())
        return r
