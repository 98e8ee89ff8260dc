"""Device-resident MoE layer: uploads seeded synthetic inputs and runs the ABI calls (the four steps one by one,
or the whole layer in one moe_layer call).

torch provides device memory and the stream; every step of the layer runs in
libmoe_hip.so through the binding.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from . import synth


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceExperts:
    """n quantised SwiGLU experts stacked per matrix, resident in HBM."""

    def __init__(self, spec: synth.LayerSpec, n: int, I: int, device):
        rb_in = spec.d * spec.wbits // 8
        rb_hid = I * spec.wbits // 8
        zt = torch.int8 if spec.wbits == 8 else torch.float32
        qt = torch.int8 if spec.wbits == 8 else torch.uint8
        self.q_gate = torch.empty((n, I, rb_in), dtype=qt, device=device)
        self.q_up = torch.empty((n, I, rb_in), dtype=qt, device=device)
        self.q_down = torch.empty((n, spec.d, rb_hid), dtype=qt, device=device)
        self.s_gate = torch.empty((n, I), dtype=torch.float32, device=device)
        self.s_up = torch.empty((n, I), dtype=torch.float32, device=device)
        self.s_down = torch.empty((n, spec.d), dtype=torch.float32, device=device)
        self.z_gate = torch.empty((n, I), dtype=zt, device=device)
        self.z_up = torch.empty((n, I), dtype=zt, device=device)
        self.z_down = torch.empty((n, spec.d), dtype=zt, device=device)

    def set(self, i: int, ex: synth.QExpert) -> None:
        for name, m in (("gate", ex.gate), ("up", ex.up), ("down", ex.down)):
            getattr(self, "q_" + name)[i].copy_(torch.from_numpy(np.ascontiguousarray(m.q)))
            getattr(self, "s_" + name)[i].copy_(torch.from_numpy(m.scale))
            getattr(self, "z_" + name)[i].copy_(torch.from_numpy(np.ascontiguousarray(m.zp)))

    def qffn(self) -> B.moe_qffn:
        return B.make_qffn(self.q_gate, self.q_up, self.q_down, self.s_gate, self.s_up, self.s_down,
                           self.z_gate, self.z_up, self.z_down)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.q_gate, self.q_up, self.q_down, self.s_gate, self.s_up, self.s_down,
                    self.z_gate, self.z_up, self.z_down))

    @staticmethod
    def from_set(spec: synth.LayerSpec, ws: synth.QExpertSet, I: int, device) -> "DeviceExperts":
        d = DeviceExperts(spec, ws.n, I, device)
        for name in ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down"):
            getattr(d, name).copy_(torch.from_numpy(np.ascontiguousarray(getattr(ws, name))))
        return d


def upload_routed(spec: synth.LayerSpec, seed: int, layer: int, device) -> DeviceExperts:
    """Generate the E routed experts one at a time straight into device memory."""
    d = DeviceExperts(spec, spec.E, spec.I, device)
    for e in range(spec.E):
        d.set(e, synth.gen_expert(spec, e, seed, layer))
    return d


def upload_shared(spec: synth.LayerSpec, seed: int, layer: int, device) -> Optional[DeviceExperts]:
    if spec.I_shared == 0:
        return None
    d = DeviceExperts(spec, 1, spec.I_shared, device)
    d.set(0, synth.gen_expert(spec, -1, seed, layer))
    return d


class DeviceLayerWeights:
    """Router and expert weights of one layer in HBM (routed=False: router and shared expert only, the routed
    experts living in a host tier)."""

    def __init__(self, spec: synth.LayerSpec, seed: int = 0, layer: int = 0, device="cuda", routed: bool = True):
        self.spec = spec
        self.W_r = _dev(synth.gen_router(spec, seed, layer), device)
        self.bias = _dev(synth.gen_bias(spec, seed, layer), device)
        self.routed = upload_routed(spec, seed, layer, device) if routed else None
        self.shared = upload_shared(spec, seed, layer, device)
        self.routed_q = self.routed.qffn() if routed else None
        self.shared_q = self.shared.qffn() if self.shared is not None else None


class MoeRun:
    """Output and workspace buffers for one (spec, T) and the four calls that fill them."""

    def __init__(self, spec: synth.LayerSpec, T: int, device="cuda", path: int = B.MOE_PATH_AUTO, flags: int = 0,
                 router: int = B.MOE_ROUTER_SIGMOID_BIAS, capacity_factor: float = 0.0):
        self.spec, self.T = spec, T
        k, E, d = spec.k, spec.E, spec.d
        A = T * k
        self.shape = B.make_shape(T, d, E, k, spec.I, spec.I_shared, spec.routed_scale, spec.act, spec.wbits, path,
                                  flags, router, capacity_factor)
        i32 = dict(dtype=torch.int32, device=device)
        self.idx = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=device)
        # the selection margin per token, or per expert under expert choice
        self.gap = torch.empty(E if router == B.MOE_ROUTER_EXPERT_CHOICE else T, dtype=torch.float64, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(A, **i32)
        self.inv = torch.empty(A, **i32)
        self.uniq = torch.empty(E, **i32)
        self.n_uniq = torch.empty(1, **i32)
        self.y_perm = torch.empty((A, d), dtype=torch.float32, device=device)
        self.y_shared = torch.empty((T, d), dtype=torch.float32, device=device) if spec.I_shared > 0 else None
        self.y = torch.empty((T, d), dtype=torch.float32, device=device)
        self.ws = torch.empty(max(B.moe_workspace_size(self.shape), 256), dtype=torch.uint8, device=device)
        # moe_forward's diagnostic counters (uint32 in the ABI), added to by every forward call
        self.diag = torch.zeros(B.MOE_DIAG_COUNT, dtype=torch.int32, device=device)

    def route(self, x, W: DeviceLayerWeights, stream=None):
        B.moe_route(self.shape, x, W.W_r, W.bias, self.idx, self.w, self.gap, self.ws, stream=stream)

    def permute(self, stream=None):
        B.moe_permute(self.shape, self.idx, self.counts, self.offsets, self.perm, self.inv, self.uniq, self.n_uniq,
                      self.ws, stream=stream)

    def forward(self, x, W: DeviceLayerWeights, stream=None):
        B.moe_forward(self.shape, x, W.routed_q, W.shared_q, self.offsets, self.perm, self.uniq, self.n_uniq,
                      self.y_perm, self.y_shared, self.diag, self.ws, stream=stream)

    def combine(self, stream=None):
        B.moe_combine(self.shape, self.y_perm, self.y_shared, self.inv, self.w, self.y, stream=stream)

    def route_permute(self, x, W: DeviceLayerWeights, stream=None):
        B.moe_route_permute(self.shape, x, W.W_r, W.bias, self.idx, self.w, self.gap, self.counts, self.offsets,
                            self.perm, self.inv, self.uniq, self.n_uniq, self.ws, stream=stream)

    def layer(self, x, W: DeviceLayerWeights, stream=None):
        B.moe_layer(self.shape, x, W.W_r, W.bias, W.routed_q, W.shared_q, self.idx, self.w, self.gap, self.counts,
                    self.offsets, self.perm, self.inv, self.uniq, self.n_uniq, self.y_perm, self.y_shared, self.y,
                    self.diag, self.ws, stream=stream)

    def run(self, x, W: DeviceLayerWeights, stream=None):
        """The layer in one call (moe_layer); the same bits as run_calls."""
        self.layer(x, W, stream)
        return self.y

    def run_calls(self, x, W: DeviceLayerWeights, stream=None):
        """The layer as the three calls moe_route_permute, moe_forward, moe_combine."""
        self.route_permute(x, W, stream)
        self.forward(x, W, stream)
        self.combine(stream)
        return self.y


def upload_x(spec: synth.LayerSpec, x: np.ndarray, device="cuda") -> torch.Tensor:
    """Activations as a device tensor (bf16 inputs arrive as uint16 bit patterns)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if spec.act == synth.ACT_BF16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


class HostTier(DeviceExperts):
    """The E routed experts of a layer in pinned host memory, the tier that an expert cache's slots are filled
    from (read by the GPU over the host link)."""

    def __init__(self, spec: synth.LayerSpec, seed: int = 0, layer: int = 0):
        super().__init__(spec, spec.E, spec.I, "cpu")
        for name in ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down"):
            setattr(self, name, getattr(self, name).pin_memory())
        for e in range(spec.E):
            self.set(e, synth.gen_expert(spec, e, seed, layer))


class CachedMoeRun(MoeRun):
    """One layer's expert cache (slots in HBM over a HostTier) and its step: route, permute and plan on the
    current stream; the missed experts copied on a second stream while the resident ones and the shared expert
    compute; then the missed experts and the combine."""

    def __init__(self, spec: synth.LayerSpec, T: int, slots: int, pinned=(), policy: int = B.MOE_CACHE_WEIGHTED_LRU,
                 device="cuda", path: int = B.MOE_PATH_AUTO, copy_stream=None):
        super().__init__(spec, T, device, path)
        E = spec.E
        self.cache = B.make_cache_shape(E, slots, len(pinned), policy)
        self.pinned = [int(e) for e in pinned]
        self.state = torch.empty(B.moe_cache_state_size(self.cache), dtype=torch.uint8, device=device)
        self.slots = DeviceExperts(spec, slots, spec.I, device)
        self.slots_q = self.slots.qffn()
        i32 = dict(dtype=torch.int32, device=device)
        self.hit, self.n_hit = torch.empty(E, **i32), torch.empty(1, **i32)
        self.miss, self.n_miss = torch.empty(E, **i32), torch.empty(1, **i32)
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream(device=device)

    def init(self, tier: HostTier, stream=None):
        """Empties the cache and loads the pinned experts (waits for them)."""
        B.moe_cache_init(self.cache, self.pinned, self.state, self.miss, self.n_miss, stream=stream)
        B.moe_cache_fetch(self.shape, self.cache, tier.qffn(), self.slots_q, self.state, self.miss, self.n_miss,
                          stream=stream)
        torch.cuda.synchronize()

    def plan(self, stream=None):
        B.moe_cache_plan(self.cache, self.T, self.spec.k, self.uniq, self.n_uniq, self.state, self.hit, self.n_hit,
                         self.miss, self.n_miss, stream=stream)

    def step(self, x, W: DeviceLayerWeights, tier: HostTier, tier_q: Optional[B.moe_qffn] = None, fetch_events=None):
        """One layer call on the current stream (and the copy stream); returns y.  fetch_events: optional pair of
        timing events recorded on the copy stream around the copy."""
        cs = torch.cuda.current_stream()
        tier_q = tier.qffn() if tier_q is None else tier_q
        self.route(x, W, cs)
        self.permute(cs)
        self.plan(cs)
        planned = torch.cuda.Event()
        planned.record(cs)
        self.copy_stream.wait_event(planned)
        if fetch_events is not None:
            fetch_events[0].record(self.copy_stream)
        B.moe_cache_fetch(self.shape, self.cache, tier_q, self.slots_q, self.state, self.miss, self.n_miss,
                          stream=self.copy_stream)
        if fetch_events is not None:
            fetch_events[1].record(self.copy_stream)
        fetched = torch.cuda.Event()
        fetched.record(self.copy_stream)
        B.moe_forward_cached(self.shape, self.cache, x, self.slots_q, self.state, W.shared_q, self.offsets,
                             self.perm, self.hit, self.n_hit, self.y_perm, self.y_shared, self.diag, self.ws,
                             stream=cs)
        cs.wait_event(fetched)
        B.moe_forward_cached(self.shape, self.cache, x, self.slots_q, self.state, W.shared_q, self.offsets,
                             self.perm, self.miss, self.n_miss, self.y_perm, None, self.diag, self.ws, stream=cs)
        self.combine(cs)
        return self.y

    def stats(self, want_slots: bool = False):
        return B.moe_cache_stats(self.cache, self.state, want_slots)
