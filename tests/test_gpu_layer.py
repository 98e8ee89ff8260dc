"""moe_layer against moe_route_permute, moe_forward and moe_combine called in turn: the same bits for every output.

For one token on the decode path with a top-k router and no capacity, moe_layer selects and sorts inside the
forward's first launch (every workgroup for itself from the logits kernel's partial sums, the first writing the
routing outputs), and where the token's slots fit and balance, the combine inside the down launch; elsewhere it
runs the three calls' kernels.  The cases cover both forms: sigmoid and softmax
routers, E from 4 to 256 (every block shape of the single-token logits kernel) and a non-power-of-two E (the
matrix-core logits kernel), int4 and int8 weights, bf16 and fp32 activations, with and without a shared
expert, the batch-invariant mode, k = E (soft routing), capacity, and the empty batch and T > 1.
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
    d = dict(name="ly", family=240, d=1024, E=64, k=6, I=256, I_shared=256, wbits=4, routed_scale=2.5,
             act=synth.ACT_BF16, bias="normal0.05")
    d.update(kw)
    return synth.LayerSpec(**d)


# (spec fields, T, router, flags, capacity factor)
CASES = {
    "E256_k8_shared_T1": (dict(d=7168, E=256, k=8, I=128, I_shared=128), 1, 0, 0, 0.0),
    "E8_k2_int8_f32_T1": (dict(d=4096, E=8, k=2, I=512, I_shared=0, wbits=8, act=synth.ACT_F32, routed_scale=1.0,
                                bias="uniform0.01"), 1, 0, 0, 0.0),
    "E64_T1": (dict(), 1, 0, 0, 0.0),
    # down launches that also combine: two slots per token over 256 tiles of 32 rows
    "combine_E8_k2_T1": (dict(d=8192, E=8, k=2, I=4096, I_shared=0), 1, 0, 0, 0.0),
    "combine_E8_k1_shared_T1": (dict(d=8192, E=8, k=1, I=4096, I_shared=4096), 1, 0, 0, 0.0),
    "combine_softmax_E8_k2_T1": (dict(d=8192, E=8, k=2, I=4096, I_shared=0), 1, B.MOE_ROUTER_SOFTMAX, 0, 0.0),
    "tiny_E8_k2_int8_f32_T1": (dict(d=256, E=8, k=2, I=512, I_shared=0, wbits=8, act=synth.ACT_F32,
                                    routed_scale=1.0, bias="uniform0.01"), 1, 0, 0, 0.0),
    "E4_k2_T1": (dict(d=512, E=4, k=2), 1, 0, 0, 0.0),
    "E32_k4_f32_T1": (dict(d=2048, E=32, k=4, act=synth.ACT_F32), 1, 0, 0, 0.0),
    "E64_noshared_T1": (dict(I_shared=0), 1, 0, 0, 0.0),
    "softmax_E64_T1": (dict(), 1, B.MOE_ROUTER_SOFTMAX, 0, 0.0),
    "E12_k3_T1": (dict(E=12, k=3), 1, 0, 0, 0.0),
    "soft_k_eq_E_T1": (dict(E=16, k=16, I=128), 1, B.MOE_ROUTER_SOFTMAX, 0, 0.0),
    "E64_k24_T1": (dict(E=64, k=24, I=128), 1, 0, 0, 0.0),
    "E512_k8_T1": (dict(d=1024, E=512, k=8, I=64), 1, 0, 0, 0.0),  # beyond the in-launch selection: three calls
    "invariant_E256_T1": (dict(d=7168, E=256, k=8, I=128, I_shared=128), 1, 0, B.MOE_FLAG_BATCH_INVARIANT, 0.0),
    "capacity_T1": (dict(), 1, 0, 0, 1.25),
    "unfused_T3": (dict(), 3, 0, 0, 0.0),
    "E256_k8_shared_T4": (dict(d=7168, E=256, k=8, I=128, I_shared=128), 4, 0, 0, 0.0),
    "E12_k3_T6": (dict(E=12, k=3), 6, 0, 0, 0.0),
    "unfused_gemm_T48": (dict(d=1024, E=16, k=4, I=256, I_shared=256), 48, 0, 0, 0.0),
    "empty_T0": (dict(), 0, 0, 0, 0.0),
}


def _weights(spec, dev):
    W = L.DeviceLayerWeights.__new__(L.DeviceLayerWeights)
    W.spec = spec
    W.W_r = torch.from_numpy(synth.gen_router(spec)).to(dev)
    W.bias = torch.from_numpy(synth.gen_bias(spec)).to(dev)
    W.routed = L.upload_routed(spec, 0, 0, dev)
    W.shared = L.upload_shared(spec, 0, 0, dev)
    W.routed_q = W.routed.qffn()
    W.shared_q = W.shared.qffn() if W.shared is not None else None
    return W


def _bits(t):
    return t.view(torch.uint8) if t.dtype in (torch.float64, torch.float32) else t


@pytest.mark.parametrize("case", list(CASES))
def test_layer_equals_three_calls(dev, case):
    kw, T, router, flags, cf = CASES[case]
    spec = _spec(**kw)
    say(f"[layer] {case} T={T} d={spec.d} E={spec.E} k={spec.k} I={spec.I} Is={spec.I_shared} w{spec.wbits} "
        f"act={spec.act} router={router} flags={flags} cf={cf}")
    W = _weights(spec, dev)
    a = L.MoeRun(spec, T, dev, flags=flags, router=router, capacity_factor=cf)
    b = L.MoeRun(spec, T, dev, flags=flags, router=router, capacity_factor=cf)
    for step in range(3):
        x = L.upload_x(spec, synth.gen_x(spec, max(T, 1), 0, step)[:T], dev)
        for r in (a, b):
            for n in OUTS:
                t = getattr(r, n)
                if t is not None:
                    t.fill_(-7)
        a.run_calls(x, W)
        b.run(x, W)
        torch.cuda.synchronize()
        for n in OUTS:
            ta, tb = getattr(a, n), getattr(b, n)
            if ta is None:
                continue
            assert torch.equal(_bits(ta.cpu()), _bits(tb.cpu())), f"step {step}: {n}"
