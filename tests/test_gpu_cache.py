"""Parity of the expert residency tier (include/moe_cache.h) with the oracle's cache and with the resident path.

- The device planner's hit and miss lists and slot contents equal the oracle cache's after every step of long
  request streams (both policies, pinned experts, empty steps, the n_uniq = -1 prefix form).
- A layer run through the cache (plan, copy of the missed experts from pinned host memory on a second stream,
  the cached forward over hits then misses, combine) gives the same bits as moe_forward over resident weights,
  and the oracle's output within the layer tolerance; the slots hold exact copies of the host tier's experts.
"""
import numpy as np
import pytest
import torch

from helpers import SampledOracle, assert_layer_close, say
from routed_expert_ffn_sigmoid_amd import binding as B
from routed_expert_ffn_sigmoid_amd import layer as L
from routed_expert_ffn_sigmoid_amd import synth

pytestmark = pytest.mark.gpu

NAMES = ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def zipf_union(rng, E, k, T, pop):
    if T == 0:
        return np.zeros(0, np.int32)
    return np.unique(np.concatenate([rng.choice(E, size=k, replace=False, p=pop) for _ in range(T)])).astype(np.int32)


@pytest.mark.parametrize("policy", [B.MOE_CACHE_WEIGHTED_LRU, B.MOE_CACHE_LRU])
def test_plan_equals_oracle_cache(orc, dev, policy):
    E, k, S = 256, 8, 40
    pinned = [3, 77, 128, 255]
    say(f"[cache plan] policy={policy} E={E} S={S} pinned={pinned}")
    c = B.make_cache_shape(E, S, len(pinned), policy)
    i32 = dict(dtype=torch.int32, device=dev)
    state = torch.empty(B.moe_cache_state_size(c), dtype=torch.uint8, device=dev)
    hit, n_hit, miss, n_miss = (torch.empty(E, **i32), torch.empty(1, **i32), torch.empty(E, **i32),
                                torch.empty(1, **i32))
    uniq, n_uniq = torch.empty(E, **i32), torch.empty(1, **i32)
    B.moe_cache_init(c, pinned, state, miss, n_miss)
    assert n_miss.item() == len(pinned) and miss[:len(pinned)].tolist() == pinned
    assert (miss[len(pinned):] == -1).all()
    ref = orc.ExpertCache(E, S, pinned, policy)
    rng = np.random.default_rng(5 + policy)
    pop = 1.0 / np.arange(1, E + 1) ** 1.1
    pop = pop[rng.permutation(E)]
    pop /= pop.sum()
    for step in range(400):
        T = int(rng.integers(0, 5))
        U = zipf_union(rng, E, k, T, pop)
        host = np.full(E, -1, np.int32)
        host[:U.size] = rng.permutation(U) if step % 3 == 0 else U  # the planner takes any order
        uniq.copy_(torch.from_numpy(host))
        n_uniq.fill_(-1 if step % 7 == 0 else U.size)  # -1: the non-negative prefix
        B.moe_cache_plan(c, T, k, uniq, n_uniq, state, hit, n_hit, miss, n_miss)
        r = ref.step(U)
        nh, nm = n_hit.item(), n_miss.item()
        assert (nh, nm) == (r.hits.size, r.misses.size), f"step {step}"
        h, m = hit.cpu().numpy(), miss.cpu().numpy()
        np.testing.assert_array_equal(h[:nh], r.hits)
        np.testing.assert_array_equal(m[:nm], r.misses)
        assert (h[nh:] == -1).all() and (m[nm:] == -1).all()
        stats, slots = B.moe_cache_stats(c, state, want_slots=True)
        assert slots == ref.slot_expert.tolist(), f"step {step}"
    assert stats == (400, ref.n_hits, ref.n_misses, ref.n_evictions, 0)
    say(f"[cache plan] hits {ref.n_hits} misses {ref.n_misses} evictions {ref.n_evictions}")


_TIERS = {}


def _tier_and_weights(spec, dev):
    """The host tier of a layer and its device weights (router, shared, and a resident copy of the routed experts
    for the reference path), made once per layer."""
    if spec.name not in _TIERS:
        tier = L.HostTier(spec)
        W = L.DeviceLayerWeights(spec, device=dev, routed=False)
        W.routed = L.DeviceExperts(spec, spec.E, spec.I, dev)
        for n in NAMES:
            getattr(W.routed, n).copy_(getattr(tier, n))
        W.routed_q = W.routed.qffn()
        _TIERS.clear()  # one layer held at a time
        _TIERS[spec.name] = (tier, W)
    return _TIERS[spec.name]


def _layer_runs(spec, T, slots, pinned, dev, path=B.MOE_PATH_AUTO):
    tier, W = _tier_and_weights(spec, dev)
    cached = L.CachedMoeRun(spec, T, slots, pinned, device=dev, path=path)
    cached.init(tier)
    plain = L.MoeRun(spec, T, dev, path)
    return tier, W, cached, plain


def _check_slots_hold_tier(cached, tier):
    _, slot_expert = cached.stats(want_slots=True)
    for s, e in enumerate(slot_expert):
        if e < 0:
            continue
        for n in NAMES:
            a = getattr(cached.slots, n)[s].cpu()
            b = getattr(tier, n)[e]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"slot {s} expert {e} {n}"


def _run_steps(orc, spec, T, steps, cached, plain, W, tier, dev, oracle_steps=(0,), repeat_first=True):
    so = SampledOracle(orc, spec)
    requested = 0
    for i in range(steps):
        batch = 0 if (repeat_first and i == 1) else i  # step 1 repeats step 0: every expert a hit
        xh = synth.gen_x(spec, T, 0, batch)
        x = L.upload_x(spec, xh, dev)
        y_ref = plain.run(x, W).clone()
        y = cached.step(x, W, tier).clone()
        torch.cuda.synchronize()
        nu = plain.n_uniq.item()
        requested += nu
        if repeat_first and i == 1:
            assert cached.n_miss.item() == 0 and cached.n_hit.item() == nu
        assert torch.equal(y, y_ref), f"step {i}: cached output differs from the resident path"
        if i in oracle_steps:
            r, _, _, yo = so.run(xh, W.W_r.cpu().numpy(), W.bias.cpu().numpy(), np.arange(T))
            np.testing.assert_array_equal(plain.idx.cpu().numpy(), r.idx)
            assert_layer_close(y.cpu().numpy(), yo, f"cached step {i}")
    stats = cached.stats()
    assert stats[0] == steps and stats[1] + stats[2] == requested and stats[4] == 0
    return stats


@pytest.mark.parametrize("wbits,act", [(4, synth.ACT_BF16), (8, synth.ACT_F32)])
def test_cached_layer_small_equals_resident_and_oracle(orc, dev, wbits, act):
    spec = synth.LayerSpec(f"cache_small{wbits}", 210, 512, 16, 2, 352, 256, wbits, 2.5, act, "normal0.05")
    T, slots, pinned = 4, 10, [5, 9]
    say(f"[cache layer] wbits={wbits} T={T} slots={slots}")
    tier, W, cached, plain = _layer_runs(spec, T, slots, pinned, dev)
    stats = _run_steps(orc, spec, T, 12, cached, plain, W, tier, dev, oracle_steps=(0, 5))
    say(f"[cache layer] stats {stats}")
    assert stats[3] > 0  # evictions happened
    _check_slots_hold_tier(cached, tier)


def test_cached_layer_matrix_core_path(orc, dev):
    spec = synth.LayerSpec("cache_gemm", 211, 512, 16, 2, 384, 256, 4, 2.5, synth.ACT_BF16, "normal0.05")
    T = 24  # T*k = 48 >= E: every expert may be missing at once, so the slots hold them all
    say(f"[cache layer gemm] T={T}")
    tier, W, cached, plain = _layer_runs(spec, T, 16, [], dev, path=B.MOE_PATH_GEMM)
    _run_steps(orc, spec, T, 4, cached, plain, W, tier, dev, oracle_steps=(0,))
    _check_slots_hold_tier(cached, tier)


@pytest.mark.parametrize("T,slots", [(1, 32), (4, 36)])
def test_cached_layer_full_size(orc, dev, T, slots):
    """The 256-expert top-8 int4 layer with the Zipf-calibrated bias: the four most popular experts pinned."""
    spec = synth.CONFIGS["large_zipf"]
    pinned = synth.popularity_order(spec)[:4].tolist()
    say(f"[cache layer full] T={T} slots={slots} pinned={pinned}")
    tier, W, cached, plain = _layer_runs(spec, T, slots, pinned, dev)
    stats = _run_steps(orc, spec, T, 16, cached, plain, W, tier, dev, oracle_steps=(3,))
    say(f"[cache layer full] stats {stats}")
    _check_slots_hold_tier(cached, tier)
