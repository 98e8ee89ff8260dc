"""moe_layer and moe_forward captured in a HIP graph and replayed, as bench.py times them: every replay gives
the bits of the eager calls.

Each case captures a rotation of steps (several layers and activation batches, each step its own buffers) in one
graph, replays it several times with eager work and synchronisations between the replays, and compares every
output of every step after every replay with the eager run.  The library enqueues no memset, so the graphs hold
kernel nodes only.
"""
import pytest
import torch

from helpers import say
from routed_expert_ffn_sigmoid_amd import binding as B
from routed_expert_ffn_sigmoid_amd import layer as L
from routed_expert_ffn_sigmoid_amd import synth

pytestmark = pytest.mark.gpu

OUTS = ("idx", "w", "gap", "counts", "offsets", "perm", "inv", "uniq", "n_uniq", "y_perm", "y_shared", "y")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _spec(**kw):
    d = dict(name="gr", family=250, d=1024, E=64, k=6, I=256, I_shared=256, wbits=4, routed_scale=2.5,
             act=synth.ACT_BF16, bias="normal0.05")
    d.update(kw)
    return synth.LayerSpec(**d)


CASES = {
    # one token, routing inside the gate/up launch
    "E256_k8_T1": (dict(d=7168, E=256, k=8, I=128, I_shared=128), 1),
    # one token, the combine inside the down launch too
    "combine_E8_k2_T1": (dict(d=8192, E=8, k=2, I=4096, I_shared=0), 1),
    # decode batch on the three calls' kernels
    "E64_T4": (dict(), 4),
    # the matrix-core path
    "gemm_T48": (dict(d=1024, E=16, k=4, I=256, I_shared=256), 48),
}


def _bits(t):
    return t.view(torch.uint8) if t.dtype in (torch.float64, torch.float32) else t


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_equal_eager(dev, case):
    kw, T = CASES[case]
    spec = _spec(**kw)
    say(f"[graph] {case} T={T} d={spec.d} E={spec.E} k={spec.k} I={spec.I} Is={spec.I_shared}")
    layers = [L.DeviceLayerWeights(spec, 0, l, dev) for l in range(2)]
    xs = [L.upload_x(spec, synth.gen_x(spec, T, 0, b), dev) for b in range(3)]
    steps = [(xs[i % 3], layers[i % 2]) for i in range(6)]
    runs = [L.MoeRun(spec, T, dev) for _ in steps]
    eager = []
    for r, (x, W) in zip(runs, steps):
        r.run(x, W)
        r.forward(x, W)  # moe_forward alone rewrites y_perm / y_shared with the same bits
    torch.cuda.synchronize()
    for r in runs:
        eager.append({n: getattr(r, n).clone() for n in OUTS if getattr(r, n) is not None})
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for r, (x, W) in zip(runs, steps):
            r.run(x, W)
            r.forward(x, W)
    torch.cuda.synchronize()
    for rep in range(4):
        for r in runs:
            for n in OUTS:
                t = getattr(r, n)
                if t is not None:
                    t.fill_(-3)
        # eager work between the replays: another layer call on the first step's buffers
        if rep % 2 == 1:
            x, W = steps[1]
            runs[0].run(x, W)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, r in enumerate(runs):
            for n, ref in eager[i].items():
                assert torch.equal(_bits(getattr(r, n)), _bits(ref)), f"replay {rep} step {i}: {n}"
