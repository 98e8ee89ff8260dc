"""Seeded synthetic inputs for the MoE-layer forward.

This module produces raw input buffers only: activations, router weights,
selection biases and per-output-channel quantised SwiGLU expert weights.  It
holds none of the layer's arithmetic (no routing, no dequantisation, no
matmul), so the HIP path and the CPU oracle can both take their inputs from it
without sharing any computation.

Shapes and value distributions follow the workloads the pages describe: a
DeepSeek-V3-style sigmoid router choosing 8 of 256 experts per token
(pwwt.cn "Colibri" write-up, section 3.1), experts stored contiguously per
expert (discosf.com walk-through, section 2.3) and quantised per output
channel with a scale and a zero point (discosf.com walk-through, section 3.4).
The concrete sizes are the five workloads named in ``CONFIGS``.

Every buffer is drawn from ``numpy.random.PCG64`` seeded with
``SeedSequence([seed, family, layer, tensor, expert])``, so any single expert
of any layer can be regenerated alone, byte for byte.

Weight layout (canonical, row-major [out][in], quantised per output row):
  int8: q is int8 in [-127, 127], zero point int8, scale fp32;
  int4: q is an unsigned nibble 0..15, two per byte, the even input index in
        the low nibble; zero point fp32 (integer valued), scale fp32.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
import os
from typing import Dict, List, Optional

import numpy as np

# tensor ids inside a SeedSequence
_T_X, _T_WR, _T_BIAS, _T_GATE, _T_UP, _T_DOWN, _T_POP, _T_CAL = range(8)
_SHARED_EXPERT_ID = 1 << 20  # expert slot used for the always-on shared expert

ACT_F32 = 0
ACT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Architecture of one MoE layer (no token count)."""
    name: str
    family: int          # seed namespace shared by workloads that use the same layer weights
    d: int               # hidden size
    E: int               # routed experts
    k: int               # experts chosen per token
    I: int               # routed expert intermediate size
    I_shared: int        # shared expert intermediate size (0 = no shared expert)
    wbits: int           # 8 or 4
    routed_scale: float  # lambda, multiplies the normalised combine weights
    act: int             # ACT_F32 or ACT_BF16
    bias: str            # "uniform0.01" | "normal0.05" | "zero" | "zipf1.1"

    @property
    def row_bytes_in(self) -> int:
        return self.d * self.wbits // 8

    @property
    def row_bytes_hidden(self) -> int:
        return self.I * self.wbits // 8

    def expert_bytes(self, I: Optional[int] = None) -> int:
        """Weight + scale + zero-point bytes of one SwiGLU expert."""
        I = self.I if I is None else I
        w = 3 * I * self.d * self.wbits // 8
        zp_bytes = 1 if self.wbits == 8 else 4
        ch = 2 * I + self.d
        return w + ch * (4 + zp_bytes)


# The five workloads.  "family" groups the ones that share layer weights.
CONFIGS: Dict[str, LayerSpec] = {
    # d=256, 8 experts, top-2, I=512, int8, fp32 activations, T=16
    "tiny": LayerSpec("tiny", 0, 256, 8, 2, 512, 0, 8, 1.0, ACT_F32, "uniform0.01"),
    # d=4096, 8 experts, top-2, I=14336, int8, fp32 activations, T=1 and 4
    "mid": LayerSpec("mid", 1, 4096, 8, 2, 14336, 0, 8, 1.0, ACT_F32, "uniform0.01"),
    # d=7168, 256 experts, top-8, I=2048 + shared 2048, int4, bf16, T=1
    "large": LayerSpec("large", 2, 7168, 256, 8, 2048, 2048, 4, 2.5, ACT_BF16, "normal0.05"),
    # same layer weights, Zipf(1.1) popularity, T=4 and 512
    "large_zipf": LayerSpec("large_zipf", 2, 7168, 256, 8, 2048, 2048, 4, 2.5, ACT_BF16, "zipf1.1"),
    # same layer, T=8192, int4/int8 x uniform(bias 0)/Zipf
    "prefill_int4_uniform": LayerSpec("prefill_int4_uniform", 2, 7168, 256, 8, 2048, 2048, 4, 2.5, ACT_BF16, "zero"),
    "prefill_int4_zipf": LayerSpec("prefill_int4_zipf", 2, 7168, 256, 8, 2048, 2048, 4, 2.5, ACT_BF16, "zipf1.1"),
    "prefill_int8_uniform": LayerSpec("prefill_int8_uniform", 3, 7168, 256, 8, 2048, 2048, 8, 2.5, ACT_BF16, "zero"),
    "prefill_int8_zipf": LayerSpec("prefill_int8_zipf", 3, 7168, 256, 8, 2048, 2048, 8, 2.5, ACT_BF16, "zipf1.1"),
}

# token counts each workload is run at
WORKLOAD_T: Dict[str, List[int]] = {
    "tiny": [16],
    "mid": [1, 4],
    "large": [1],
    "large_zipf": [4, 512],
    "prefill_int4_uniform": [8192],
    "prefill_int4_zipf": [8192],
    "prefill_int8_uniform": [8192],
    "prefill_int8_zipf": [8192],
}

ZIPF_S = 1.1
# Router weights of the 256-expert layers: family 3 (int8 experts) reuses the
# router of family 2 so the two prefill variants route identically.
_ROUTER_FAMILY = {0: 0, 1: 1, 2: 2, 3: 2}


def _rng(seed: int, family: int, layer: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, family, layer, tensor, expert])))


def _uniform_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniformly distributed bytes from the raw 64-bit PCG64 stream (little endian)."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return np.ascontiguousarray(words.astype("<u8").view(np.uint8)[:n])


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# activations, router, bias
# ----------------------------------------------------------------------------

def gen_x(spec: LayerSpec, T: int, seed: int = 0, batch: int = 0) -> np.ndarray:
    """Layer input [T][d]: N(0,1) samples, fp32 or bf16 bits (uint16)."""
    rng = _rng(seed, spec.family, 0, _T_X, batch)
    x = rng.standard_normal((T, spec.d), dtype=np.float32)
    if spec.act == ACT_BF16:
        return round_to_bf16_bits(x).reshape(T, spec.d)
    return x


def gen_x_correlated(spec: LayerSpec, n: int, rho: float, seed: int = 0, batch: int = 0) -> np.ndarray:
    """n consecutive token activations [n][d] as a first-order autoregressive sequence, x_0 ~ N(0, 1) and
    x_t = rho x_{t-1} + sqrt(1 - rho^2) e_t with e_t ~ N(0, 1) (every x_t is N(0, 1)): neighbouring tokens
    with similar activations, hence similar experts.  fp32, or bf16 bits like gen_x."""
    rng = _rng(seed, spec.family, 0, _T_X, (1 << 16) + batch)
    e = rng.standard_normal((n, spec.d), dtype=np.float32)
    x = np.empty_like(e)
    c = np.float32(math.sqrt(1.0 - rho * rho))
    x[0] = e[0]
    for t in range(1, n):
        x[t] = np.float32(rho) * x[t - 1] + c * e[t]
    if spec.act == ACT_BF16:
        return round_to_bf16_bits(x).reshape(n, spec.d)
    return x


def gen_router(spec: LayerSpec, seed: int = 0, layer: int = 0) -> np.ndarray:
    """W_r [d][E] fp32, entries N(0, 0.02^2)."""
    rng = _rng(seed, _ROUTER_FAMILY.get(spec.family, spec.family), layer, _T_WR)
    return (rng.standard_normal((spec.d, spec.E), dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def popularity_order(spec: LayerSpec, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Seeded permutation: element r-1 is the expert id of popularity rank r."""
    rng = _rng(seed, _ROUTER_FAMILY.get(spec.family, spec.family), layer, _T_POP)
    return rng.permutation(spec.E).astype(np.int32)


def zipf_target(E: int, k: int, s: float = ZIPF_S) -> np.ndarray:
    """Per-token selection frequency by popularity rank r=1..E.

    f(r) = min(1, c * r^-s), with c chosen so that sum_r f(r) = k (each token
    picks k distinct experts, so no expert can exceed frequency 1).
    """
    r = np.arange(1, E + 1, dtype=np.float64)
    lo, hi = 0.0, float(E) ** s * k
    for _ in range(200):
        c = 0.5 * (lo + hi)
        tot = np.minimum(1.0, c * r ** (-s)).sum()
        if tot > k:
            hi = c
        else:
            lo = c
    return np.minimum(1.0, 0.5 * (lo + hi) * r ** (-s))


def calibration_x(spec: LayerSpec, n_tokens: int = 4096, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Separate seeded token batch used only to calibrate the Zipf bias (bf16 or fp32 like gen_x)."""
    rng = _rng(seed, _ROUTER_FAMILY.get(spec.family, spec.family), layer, _T_CAL)
    x = rng.standard_normal((n_tokens, spec.d), dtype=np.float32)
    if spec.act == ACT_BF16:
        return round_to_bf16_bits(x).reshape(n_tokens, spec.d)
    return x


_GOLDEN_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")


def zipf_bias_path(E: int, d: int, layer: int, seed: int = 0) -> str:
    return os.path.join(_GOLDEN_DIR, f"zipf_bias_E{E}_d{d}_s{seed}_l{layer}.txt")


def load_zipf_bias(spec: LayerSpec, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Calibrated Zipf(1.1) selection bias, stored as hex floats (written offline by a calibration script)."""
    path = zipf_bias_path(spec.E, spec.d, layer, seed)
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(float.fromhex(line))
    b = np.asarray(vals, dtype=np.float64).astype(np.float32)
    if b.shape != (spec.E,):
        raise ValueError(f"{path}: expected {spec.E} values, got {b.shape}")
    return b


def gen_bias(spec: LayerSpec, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Per-expert selection bias b [E] fp32."""
    if spec.bias == "zero":
        return np.zeros(spec.E, dtype=np.float32)
    if spec.bias == "zipf1.1":
        return load_zipf_bias(spec, seed, layer)
    rng = _rng(seed, _ROUTER_FAMILY.get(spec.family, spec.family), layer, _T_BIAS)
    if spec.bias == "uniform0.01":
        return rng.uniform(-0.01, 0.01, size=spec.E).astype(np.float32)
    if spec.bias == "normal0.05":
        return (rng.standard_normal(spec.E) * 0.05).astype(np.float32)
    raise ValueError(spec.bias)


# ----------------------------------------------------------------------------
# quantised experts
# ----------------------------------------------------------------------------

SIGMA_Q = {8: 73.6, 4: 4.61}  # standard deviation of U{-127..127} and U{0..15}


@dataclasses.dataclass
class QMatrix:
    """One quantised matrix [rows][cols] with per-row scale and zero point."""
    q: np.ndarray       # int8 [rows][cols] or uint8 [rows][cols/2] (packed nibbles)
    scale: np.ndarray   # fp32 [rows]
    zp: np.ndarray      # int8 [rows] (wbits 8) or fp32 [rows] (wbits 4)


def _gen_qmatrix(rng: np.random.Generator, rows: int, cols: int, wbits: int) -> QMatrix:
    if wbits == 8:
        q = _uniform_bytes(rng, rows * cols).view(np.int8).copy()
        bad = np.flatnonzero(q == -128)
        if bad.size:
            q[bad] = rng.integers(-127, 128, size=bad.size, dtype=np.int8)
        q = q.reshape(rows, cols)
        zp = rng.integers(-8, 9, size=rows, dtype=np.int8)
    elif wbits == 4:
        q = _uniform_bytes(rng, rows * cols // 2).reshape(rows, cols // 2)
        zp = rng.integers(0, 16, size=rows).astype(np.float32)
    else:
        raise ValueError(wbits)
    scale = (rng.uniform(0.5, 1.5, size=rows) / (SIGMA_Q[wbits] * math.sqrt(cols))).astype(np.float32)
    return QMatrix(q, scale, zp)


@dataclasses.dataclass
class QExpert:
    gate: QMatrix   # [I][d]
    up: QMatrix     # [I][d]
    down: QMatrix   # [d][I]


def gen_expert(spec: LayerSpec, expert: int, seed: int = 0, layer: int = 0) -> QExpert:
    """Routed expert ``expert`` (0..E-1) or the shared expert (expert = -1)."""
    if expert < 0:
        I, eid = spec.I_shared, _SHARED_EXPERT_ID
        if I == 0:
            raise ValueError("layer has no shared expert")
    else:
        I, eid = spec.I, expert
    f = spec.family
    g = _gen_qmatrix(_rng(seed, f, layer, _T_GATE, eid), I, spec.d, spec.wbits)
    u = _gen_qmatrix(_rng(seed, f, layer, _T_UP, eid), I, spec.d, spec.wbits)
    dn = _gen_qmatrix(_rng(seed, f, layer, _T_DOWN, eid), spec.d, I, spec.wbits)
    return QExpert(g, u, dn)


@dataclasses.dataclass
class QExpertSet:
    """n experts stacked: q_* [n][rows][row_bytes], s_* [n][rows], z_* [n][rows]."""
    q_gate: np.ndarray
    q_up: np.ndarray
    q_down: np.ndarray
    s_gate: np.ndarray
    s_up: np.ndarray
    s_down: np.ndarray
    z_gate: np.ndarray
    z_up: np.ndarray
    z_down: np.ndarray

    @property
    def n(self) -> int:
        return self.q_gate.shape[0]


def stack_experts(experts: List[QExpert]) -> QExpertSet:
    def st(get):
        return np.ascontiguousarray(np.stack([get(e) for e in experts]))
    return QExpertSet(
        st(lambda e: e.gate.q), st(lambda e: e.up.q), st(lambda e: e.down.q),
        st(lambda e: e.gate.scale), st(lambda e: e.up.scale), st(lambda e: e.down.scale),
        st(lambda e: e.gate.zp), st(lambda e: e.up.zp), st(lambda e: e.down.zp),
    )


def gen_routed_experts(spec: LayerSpec, seed: int = 0, layer: int = 0,
                       experts: Optional[List[int]] = None) -> QExpertSet:
    ids = range(spec.E) if experts is None else experts
    return stack_experts([gen_expert(spec, e, seed, layer) for e in ids])


def gen_shared_expert(spec: LayerSpec, seed: int = 0, layer: int = 0) -> Optional[QExpertSet]:
    if spec.I_shared == 0:
        return None
    return stack_experts([gen_expert(spec, -1, seed, layer)])


@dataclasses.dataclass
class LayerInputs:
    spec: LayerSpec
    T: int
    x: np.ndarray          # [T][d] fp32 or uint16 (bf16 bits)
    W_r: np.ndarray        # [d][E] fp32
    bias: np.ndarray       # [E] fp32
    routed: QExpertSet
    shared: Optional[QExpertSet]


def gen_layer(spec: LayerSpec, T: int, seed: int = 0, layer: int = 0, batch: int = 0) -> LayerInputs:
    return LayerInputs(spec, T, gen_x(spec, T, seed, batch), gen_router(spec, seed, layer),
                       gen_bias(spec, seed, layer), gen_routed_experts(spec, seed, layer),
                       gen_shared_expert(spec, seed, layer))


def small_spec(base: LayerSpec, **kw) -> LayerSpec:
    """A copy of a layer spec with some fields replaced (used for scaled-down test cases)."""
    return dataclasses.replace(base, **kw)


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ----------------------------------------------------------------------------
# sparse-attention indexer inputs
# ----------------------------------------------------------------------------

_T_IQ, _T_IW, _T_IK, _T_IKS = 20, 21, 22, 23
_INDEX_FAMILY = 50


@dataclasses.dataclass
class IndexInputs:
    q: np.ndarray       # [T][H][D] int8
    w: np.ndarray       # [T][H] fp32
    k: np.ndarray       # [S][D] int8
    kscale: np.ndarray  # [S] fp32


def gen_index(T: int, S: int, H: int, D: int, seed: int = 0, dup_keys: bool = False) -> IndexInputs:
    """Indexer queries and keys as int8 (N(0,1) samples times 40, rounded and clipped to [-127, 127]), head weights
    N(0, 1/H) and key scales U(0.5, 1.5) / 40.  dup_keys: the second half of the keys repeats the first with one
    common scale, so that exactly equal scores occur."""
    def rng(tid):
        return _rng(seed, _INDEX_FAMILY, 0, tid)
    q = np.clip(np.rint(rng(_T_IQ).standard_normal((T, H, D), dtype=np.float32) * 40), -127, 127).astype(np.int8)
    k = np.clip(np.rint(rng(_T_IK).standard_normal((S, D), dtype=np.float32) * 40), -127, 127).astype(np.int8)
    w = (rng(_T_IW).standard_normal((T, H)) / math.sqrt(H)).astype(np.float32)
    ks = (rng(_T_IKS).uniform(0.5, 1.5, S) / 40).astype(np.float32)
    if dup_keys:
        k[S // 2:] = k[:S - S // 2]
        ks[:] = np.float32(1 / 40)
    return IndexInputs(q, w, k, ks)
