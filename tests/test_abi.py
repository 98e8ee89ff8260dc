"""Host-side checks of the C ABI: the library loads, exports what include/moe.h declares, and
rejects bad arguments before enqueuing anything (no GPU needed: every call here fails validation)."""
import ctypes
import os
import re

import pytest

from routed_expert_ffn_sigmoid_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 0x10000  # a 256-byte aligned, never dereferenced address


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_no_oracle_symbols_in_product_library():
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    assert "oracle" not in out


def shape(**kw):
    base = dict(T=4, d=256, E=8, k=2, I=512, I_shared=0, routed_scale=1.0, act_dtype=B.MOE_ACT_F32, wbits=8)
    base.update(kw)
    return B.make_shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(k=9), B.MOE_EINVAL),           # k > E
    (dict(k=0), B.MOE_EINVAL),
    (dict(T=-1), B.MOE_EINVAL),
    (dict(E=2048, k=2), B.MOE_EINVAL),   # E > 1024
    (dict(E=64, k=33), B.MOE_EINVAL),    # k > 32
    (dict(wbits=4, d=48), B.MOE_EINVAL),  # int4 needs multiples of 32
    (dict(wbits=8, I=40), B.MOE_EINVAL),  # int8 needs multiples of 16
    (dict(wbits=2), B.MOE_EUNSUPPORTED),
    (dict(act_dtype=7), B.MOE_EUNSUPPORTED),
    (dict(path=9), B.MOE_EINVAL),
])
def test_bad_shapes_rejected(kw, code):
    s = shape(**kw)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == code
    assert B.moe_workspace_size(s) == 0


def test_null_and_misaligned_pointers():
    s = shape()
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "x is NULL" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE + 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EALIGN
    with pytest.raises(B.MoeError) as ei:
        B.moe_permute(s, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "inv" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_combine(s, FAKE, None, FAKE, FAKE, None, stream=0)
    assert ei.value.code == B.MOE_EINVAL
    q = B.make_qffn(*([FAKE] * 9))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(s, FAKE, q, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 2, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EALIGN and "diag" in str(ei.value)


def test_workspace_checks():
    s = shape()
    need = B.moe_workspace_size(s)
    assert need > 0 and need % 256 == 0
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, stream=0)
    assert ei.value.code == B.MOE_EWORKSPACE
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, need, stream=0)
    assert ei.value.code == B.MOE_EWORKSPACE
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, need, stream=0)
    assert ei.value.code == B.MOE_EALIGN


def test_forward_requires_shared_weights_when_configured():
    s = shape(I_shared=256)
    q = B.make_qffn(*([FAKE] * 9))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(s, FAKE, q, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "shared" in str(ei.value)
    bad = B.make_qffn(*([FAKE] * 8 + [None]))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward(s, FAKE, bad, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "z_down" in str(ei.value)


def test_empty_batch_is_a_no_op():
    """T = 0: the shape is valid, T-sized pointers may be NULL, and route, forward and combine return OK
    without enqueueing anything (so this runs without a GPU).  Non-power-of-two E takes the router's
    matrix-core sizing, which must not divide by the empty token count."""
    for E in (16, 12):
        s = shape(T=0, E=E)
        need = B.moe_workspace_size(s)
        assert need > 0
        B.moe_route(s, None, FAKE, FAKE, None, None, None, FAKE, need, stream=0)
        q = B.make_qffn(*([FAKE] * 9))
        B.moe_forward(s, None, q, None, FAKE, None, FAKE, FAKE, None, None, None, FAKE, need, stream=0)
        B.moe_combine(s, None, None, None, None, None, stream=0)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(shape(T=0), None, None, FAKE, None, None, None, FAKE, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "W_r" in str(ei.value)


def test_workspace_size_covers_every_call():
    # large prefill shape: the router split, the GEMV buffers and the GEMM buffers all fit
    s = shape(T=8192, d=7168, E=256, k=8, I=2048, I_shared=2048, wbits=4, act_dtype=B.MOE_ACT_BF16,
              routed_scale=2.5)
    assert B.moe_workspace_size(s) >= 8192 * 8 * 2048 * 4
