"""moe_route_permute against moe_route followed by moe_permute: the same bits for every output.

For a single token the permutation runs inside the selection's launch (the selecting workgroup then sorts);
elsewhere the combined call runs the two calls' kernels.  The cases cover both forms, both top-k routers,
the batch-invariant mode, calls in a row on one workspace, and a moe_route call between them.
"""
import numpy as np
import pytest
import torch

from helpers import say
from routed_expert_ffn_sigmoid_amd import binding as B
from routed_expert_ffn_sigmoid_amd import layer as L
from routed_expert_ffn_sigmoid_amd import synth

pytestmark = pytest.mark.gpu

OUTS = ("idx", "w", "gap", "counts", "offsets", "perm", "inv", "uniq", "n_uniq")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _spec(**kw):
    d = dict(name="rf", family=230, d=1024, E=64, k=6, I=64, I_shared=0, wbits=4, routed_scale=2.5,
             act=synth.ACT_BF16, bias="normal0.05")
    d.update(kw)
    return synth.LayerSpec(**d)


CASES = {
    "E64_T1": (dict(), 1, 0, 0),
    "E64_T3": (dict(), 3, 0, 0),
    "E256_k8_T4": (dict(d=7168, E=256, k=8), 4, 0, 0),
    "E8_k2_f32_T1": (dict(d=4096, E=8, k=2, wbits=8, act=synth.ACT_F32, bias="uniform0.01"), 1, 0, 0),
    "E4_k4_T2": (dict(d=256, E=4, k=4), 2, 0, 0),
    "softmax_E64_T2": (dict(), 2, B.MOE_ROUTER_SOFTMAX, 0),
    "invariant_E256_T1": (dict(d=7168, E=256, k=8), 1, 0, B.MOE_FLAG_BATCH_INVARIANT),
    "unfused_T5": (dict(), 5, 0, 0),
    "unfused_E12": (dict(E=12, k=3), 2, 0, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_route_permute_equals_route_then_permute(dev, case):
    kw, T, router, flags = CASES[case]
    spec = _spec(**kw)
    say(f"[route+permute] {case} T={T} d={spec.d} E={spec.E} k={spec.k} router={router} flags={flags}")
    W = L.DeviceLayerWeights.__new__(L.DeviceLayerWeights)
    W.W_r = torch.from_numpy(synth.gen_router(spec)).to(dev)
    W.bias = torch.from_numpy(synth.gen_bias(spec)).to(dev)
    a = L.MoeRun(spec, T, dev, flags=flags, router=router)
    b = L.MoeRun(spec, T, dev, flags=flags, router=router)
    for step in range(4):
        x = L.upload_x(spec, synth.gen_x(spec, T, 0, step), dev)
        for r in (a, b):
            for n in OUTS:
                getattr(r, n).fill_(-7)
        a.route(x, W)
        a.permute()
        if step == 2:
            b.route(x, W)  # a route call on the workspace between combined calls
        b.route_permute(x, W)
        torch.cuda.synchronize()
        for n in OUTS:
            ga, gb = getattr(a, n).cpu(), getattr(b, n).cpu()
            assert torch.equal(ga.view(torch.uint8) if ga.dtype == torch.float64 else ga,
                               gb.view(torch.uint8) if gb.dtype == torch.float64 else gb), f"step {step}: {n}"
