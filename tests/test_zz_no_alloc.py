"""moe_forward_static: moe_forward with no workspace argument, its scratch a static device array.

The outputs must equal moe_forward's (same kernels, same inputs) bit for bit, on two calls in a row whose second
has fewer tokens than the first (the scratch keeps the first call's contents), on both forward paths.
"""
import numpy as np
import pytest
import torch

from routed_expert_ffn_sigmoid_amd import binding as B
from routed_expert_ffn_sigmoid_amd import layer as L
from routed_expert_ffn_sigmoid_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def _weights(spec, inp, dev):
    W = L.DeviceLayerWeights.__new__(L.DeviceLayerWeights)
    W.spec = spec
    W.W_r = torch.from_numpy(inp.W_r).to(dev)
    W.bias = torch.from_numpy(inp.bias).to(dev)
    W.routed = L.DeviceExperts.from_set(spec, inp.routed, spec.I, dev)
    W.shared = L.DeviceExperts.from_set(spec, inp.shared, spec.I_shared, dev)
    W.routed_q, W.shared_q = W.routed.qffn(), W.shared.qffn()
    return W


# (layer, tokens of the first call, tokens of the second): the matrix-core path then the decode kernels, and the
# decode kernels twice
CASES = [(dict(d=512, E=16, k=4, I=384, I_shared=192, routed_scale=2.5), 70, 5),
         (dict(d=1024, E=8, k=2, I=1536, I_shared=512, wbits=8, act=synth.ACT_F32, bias="uniform0.01"), 9, 3)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_static_forward_equals_forward(dev, case):
    kw, T1, T2 = CASES[case]
    base = dict(name="static", family=300, wbits=4, routed_scale=1.0, act=synth.ACT_BF16, bias="normal0.05")
    base.update(kw)
    spec = synth.LayerSpec(**base)
    inp = synth.gen_layer(spec, T1)
    W = _weights(spec, inp, dev)
    for T in (T1, T2):
        print(f"[static] case {case} T={T}", flush=True)
        x = L.upload_x(spec, inp.x[:T], dev)
        run = L.MoeRun(spec, T, dev)
        run.run(x, W)  # moe_forward with a workspace
        torch.cuda.synchronize()
        ref_p, ref_s, ref_y = run.y_perm.clone(), run.y_shared.clone(), run.y.clone()
        run.y_perm.fill_(float("nan"))
        run.y_shared.fill_(float("nan"))
        run.diag.zero_()
        B.moe_forward_static(run.shape, x, W.routed_q, W.shared_q, run.offsets, run.perm, run.uniq, run.n_uniq,
                             run.y_perm, run.y_shared, run.diag)
        run.combine()
        torch.cuda.synchronize()
        assert torch.equal(run.y_perm, ref_p), "y_perm differs from moe_forward's"
        assert torch.equal(run.y_shared, ref_s), "y_shared differs from moe_forward's"
        assert torch.equal(run.y, ref_y), "y differs from moe_forward's"
        assert int(run.diag.cpu().numpy()[0]) == 0
        assert bool(torch.isfinite(run.y).all())


def test_static_forward_refuses_what_does_not_fit(dev):
    """The 256-expert top-8 layer at T = 8192 needs about 0.9 GB of scratch: refused, nothing enqueued."""
    s = B.make_shape(8192, 7168, 256, 8, 2048, 2048, 2.5, B.MOE_ACT_BF16, 4)
    q = B.make_qffn(*([0x10000] * 9))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(s, 0x10000, q, q, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None)
    assert ei.value.code == B.MOE_EWORKSPACE and "static" in str(ei.value)
