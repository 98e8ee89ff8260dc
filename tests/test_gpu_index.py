"""Parity of the sparse-attention indexer's top-K causal keys (through the C ABI) with the oracle.

The positions are integer results and must match bit for bit.  The scores behind them are built so that both
sides compute the same bits (exact int8 dot products, an fp64 fused multiply-add chain over heads in head order),
so the test also compares the GPU's fp64 scores, read from the workspace where the kernels leave them (the first
T*S doubles), with the oracle's, bit for bit.
"""
import numpy as np
import pytest
import torch

from helpers import say
from routed_expert_ffn_sigmoid_amd import binding as B
from routed_expert_ffn_sigmoid_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _all_zero_queries(inp):
    inp.q[:] = 0  # every score 0: no spread between the smallest and the largest score


def _big_tie_block(inp):
    # 6000 copies of one key under one scale: the K-th largest falls in a bucket of more than 4096 equal scores
    inp.k[1000:7000] = inp.k[0]
    inp.kscale[1000:7000] = inp.kscale[0]


TWEAKS = {"all_scores_equal": _all_zero_queries, "tie_block_beyond_lds": _big_tie_block}

# (T, S, H, D, K, pos0, duplicated keys)
CASES = {
    "all_scores_equal": (2, 5000, 16, 64, 2048, 4998, False),
    "tie_block_beyond_lds": (2, 9000, 16, 64, 2048, 8998, False),
    "decode_32k_context": (1, 32768, 64, 128, 2048, 32767, False),
    "prefill_chunk_64_of_8192": (64, 8192, 64, 128, 2048, 8192 - 64, False),
    "short_context_padding": (8, 1000, 64, 128, 2048, 0, False),
    "crossing_k": (40, 3000, 32, 64, 2048, 2030, False),
    "exact_ties": (16, 6000, 16, 64, 1000, 5984, True),
    "h48_d192": (5, 4000, 48, 192, 512, 3995, False),
    "h16_d256_k1": (3, 700, 16, 256, 1, 697, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_index_topk_parity(orc, dev, case):
    T, S, H, D, K, pos0, dup = CASES[case]
    say(f"[index] {case} T={T} S={S} H={H} D={D} K={K} pos0={pos0}")
    inp = synth.gen_index(T, S, H, D, seed=len(case), dup_keys=dup)
    if case in TWEAKS:
        TWEAKS[case](inp)
    shape = B.dsa_index_shape(T, S, H, D, K, pos0)
    ws = torch.empty(B.dsa_index_workspace_size(shape), dtype=torch.uint8, device=dev)
    top = torch.full((T, K), -7, dtype=torch.int32, device=dev)
    gap = torch.empty(T, dtype=torch.float64, device=dev)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    B.dsa_index_topk(shape, up(inp.q), up(inp.w), up(inp.k), up(inp.kscale), top, gap, ws)
    torch.cuda.synchronize()
    ref = orc.index_topk(inp.q, inp.w, inp.k, inp.kscale, K, pos0, want_scores=True)
    np.testing.assert_array_equal(top.cpu().numpy(), ref.top, err_msg="top positions")
    np.testing.assert_array_equal(gap.cpu().numpy(), ref.gap, err_msg="gap")
    sc = ws[:T * S * 8].view(torch.float64).view(T, S).cpu().numpy()
    for t in range(T):
        n = min(S, pos0 + t + 1)
        np.testing.assert_array_equal(sc[t, :n], ref.scores[t, :n], err_msg=f"scores of query {t}")
    ties = int(np.sum(ref.gap == 0))
    say(f"   positions and scores bit-exact; {ties} queries with a tie at the K-th place")
    if dup or case in TWEAKS:
        assert ties > 0
