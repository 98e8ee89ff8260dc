"""Pins of the oracle's expert cache (HBM slots over the host tier).

Each test checks the oracle's cache against something other than itself: steps worked by hand
(tests/golden/expert_cache_steps.txt), a textbook LRU built on an ordered dictionary, Belady's optimal
replacement as a lower bound on the misses, the closed form of a cache large enough for every expert, and the
invariants of the batch union and of pinning.
"""
import collections
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "expert_cache_steps.txt")


def _ids(s):
    return [] if s == "-" else [int(v) for v in s.split(",")]


def load_golden():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                parts = line.split()
                kv = dict(p.split("=", 1) for p in parts[2:])
                cur = dict(name=parts[1], E=int(kv["E"]), S=int(kv["S"]),
                           policy=0 if kv["policy"] == "weighted" else 1, pinned=_ids(kv["pinned"]), steps=[])
                cases.append(cur)
            else:
                assert line.startswith("step ")
                fields = [p.strip() for p in line[5:].split("|")]
                U = _ids(fields[0])
                kv = dict(p.split("=", 1) for p in fields[1:])
                cur["steps"].append((U, _ids(kv["hits"]), _ids(kv["misses"]), _ids(kv["evicted"])))
    return cases


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_cache_steps_worked_by_hand(orc, case):
    c = orc.ExpertCache(case["E"], case["S"], case["pinned"], case["policy"])
    for U, hits, misses, evicted in case["steps"]:
        r = c.step(U)
        assert r.hits.tolist() == hits
        assert r.misses.tolist() == misses
        assert r.evicted.tolist() == evicted


def textbook_lru_misses(stream, S):
    """Demand paging with least-recently-used replacement, one request at a time."""
    od = collections.OrderedDict()
    misses = []
    for e in stream:
        if e in od:
            od.move_to_end(e)
            misses.append(False)
        else:
            if len(od) == S:
                od.popitem(last=False)
            od[e] = True
            misses.append(True)
    return misses


def belady_misses(stream, S):
    """Optimal offline replacement (evict the resident page whose next use is farthest), one request a step."""
    res, n = set(), 0
    for i, e in enumerate(stream):
        if e in res:
            continue
        n += 1
        if len(res) == S:
            def next_use(p):
                for j in range(i + 1, len(stream)):
                    if stream[j] == p:
                        return j
                return len(stream) + p  # never used again: any of them (farthest)
            res.remove(max(res, key=next_use))
        res.add(e)
    return n


def zipf_stream(rng, E, n, s=1.1):
    p = 1.0 / np.arange(1, E + 1) ** s
    return rng.choice(E, size=n, p=p / p.sum()).tolist()


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,S", [(16, 4), (32, 7), (12, 11)])
def test_lru_policy_is_textbook_lru_one_request_per_step(orc, seed, E, S):
    rng = np.random.default_rng(seed)
    stream = zipf_stream(rng, E, 400)
    c = orc.ExpertCache(E, S, policy=orc.CACHE_LRU)
    got = [c.step([e]).misses.size == 1 for e in stream]
    assert got == textbook_lru_misses(stream, S)


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("seed", range(4))
def test_misses_not_below_belady_optimum(orc, policy, seed):
    rng = np.random.default_rng(100 + seed)
    E, S = 12, 4
    stream = zipf_stream(rng, E, 150, s=0.8)
    c = orc.ExpertCache(E, S, policy=policy)
    for e in stream:
        c.step([e])
    assert c.n_misses >= belady_misses(stream, S)


@pytest.mark.parametrize("policy", [0, 1])
def test_cache_holding_every_expert_misses_each_once(orc, policy):
    rng = np.random.default_rng(7)
    E = 20
    c = orc.ExpertCache(E, E, policy=policy)
    seen = set()
    for _ in range(200):
        U = rng.choice(E, size=rng.integers(1, 6), replace=False)
        r = c.step(U)
        assert set(r.misses.tolist()) == set(U.tolist()) - seen
        seen |= set(U.tolist())
        assert (r.evicted == -1).all()
    assert c.n_evictions == 0 and c.n_misses == len(seen)


@pytest.mark.parametrize("policy", [0, 1])
def test_batch_union_and_pinning_invariants(orc, policy):
    rng = np.random.default_rng(11)
    E, S, k = 64, 24, 4
    pinned = [5, 17, 40, 63]
    c = orc.ExpertCache(E, S, pinned, policy)
    pop = 1.0 / np.arange(1, E + 1) ** 1.1
    pop /= pop.sum()
    requested = 0
    for step in range(300):
        T = int(rng.integers(1, 6))
        # the batch union of T tokens choosing k distinct experts each
        U = np.unique(np.concatenate([rng.choice(E, size=k, replace=False, p=pop) for _ in range(T)]))
        before = c.expert_slot.copy()
        r = c.step(U)
        requested += U.size
        resident_before = set(np.flatnonzero(before >= 0).tolist())
        assert r.hits.tolist() == sorted(set(U.tolist()) & resident_before)
        assert r.misses.tolist() == sorted(set(U.tolist()) - resident_before)
        assert not set(r.misses.tolist()) & set(pinned)
        # every requested expert is resident afterwards; slot and expert maps are inverse
        assert (c.expert_slot[U] >= 0).all()
        occ = np.flatnonzero(c.slot_expert >= 0)
        assert (c.expert_slot[c.slot_expert[occ]] == occ).all()
        assert np.count_nonzero(c.expert_slot >= 0) == occ.size
        assert c.slot_expert[:4].tolist() == pinned
        # an evicted expert was resident and not requested
        for ev in r.evicted[r.evicted >= 0].tolist():
            assert ev in resident_before and ev not in U and ev not in pinned
    assert c.n_hits + c.n_misses == requested


def test_too_many_misses_for_the_slots_is_refused(orc):
    c = orc.ExpertCache(16, 3, [0])
    with pytest.raises(RuntimeError):
        c.step([1, 2, 3])


def test_weighted_keeps_hot_experts_better_than_lru_on_a_skewed_stream(orc):
    """On independent draws from a skewed popularity (the pages' claim of a higher hit rate for the weighted
    rule, measured on long generations) frequency counts keep the popular experts that LRU loses to one-off
    requests."""
    rng = np.random.default_rng(3)
    E, S, k = 128, 16, 4
    pop = 1.0 / np.arange(1, E + 1) ** 1.1
    pop /= pop.sum()
    steps = [rng.choice(E, size=k, replace=False, p=pop) for _ in range(3000)]
    rate = {}
    for policy in (0, 1):
        c = orc.ExpertCache(E, S, policy=policy)
        for U in steps:
            c.step(U)
        rate[policy] = c.n_hits / (c.n_hits + c.n_misses)
    assert rate[0] > rate[1] + 0.05
