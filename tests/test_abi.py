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
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"MOE_API\s+[\w\s\*]+?\b((?:moe|dsa)_\w+)\s*\(", text))
    return sorted(names)


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


HUGE_WS = 1 << 62  # any workspace size passes; these calls fail on the shape before the workspace is used


def test_dimension_limit_rejected():
    """d, I, I_shared at or above MOE_MAX_DIM: the decode path's int32 sums of a K part could overflow."""
    for kw in (dict(d=B.MOE_MAX_DIM), dict(I=B.MOE_MAX_DIM), dict(I_shared=B.MOE_MAX_DIM)):
        s = shape(**kw)
        with pytest.raises(B.MoeError) as ei:
            B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
        assert ei.value.code == B.MOE_EUNSUPPORTED and f"below {B.MOE_MAX_DIM}" in str(ei.value)
        assert B.moe_workspace_size(s) == 0
    B.moe_workspace_size(shape(d=B.MOE_MAX_DIM - 16))  # just below: accepted


def test_router_buffers_beyond_32_bit_offsets_rejected():
    """x of T*d*4 bytes >= 2^31 (fp32): the router's descriptors would wrap; rejected, not computed."""
    s = shape(T=65536, d=8192, E=8, k=2)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
    assert ei.value.code == B.MOE_EUNSUPPORTED and "x exceeds" in str(ei.value)
    s = shape(T=65536, d=8192, E=8, k=2, act_dtype=B.MOE_ACT_BF16)  # half the bytes: below the limit
    assert B.moe_workspace_size(s) > 0


def _forward(s):
    q = B.make_qffn(*([FAKE] * 9))
    sh = q if s.I_shared > 0 else None
    B.moe_forward(s, FAKE, q, sh, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE if s.I_shared > 0 else None, None, FAKE,
                  HUGE_WS, stream=0)


def test_decode_h_beyond_32_bit_offsets_rejected():
    """The mid layer with fp32 activations at T = 40000 goes to the decode kernels (no matrix-core path for fp32),
    whose h of T*k*I*4 = 4.6 GB would wrap a 32-bit descriptor: rejected before anything is enqueued."""
    s = shape(T=40000, d=4096, E=8, k=2, I=14336, wbits=8, act_dtype=B.MOE_ACT_F32)
    with pytest.raises(B.MoeError) as ei:
        _forward(s)
    assert ei.value.code == B.MOE_EUNSUPPORTED and "h of the routed rows" in str(ei.value)
    s = shape(T=40000, d=4096, E=8, k=2, I=14336, wbits=8, act_dtype=B.MOE_ACT_F32, path=B.MOE_PATH_GEMV)
    with pytest.raises(B.MoeError) as ei:
        _forward(s)
    assert ei.value.code == B.MOE_EUNSUPPORTED


def test_decode_expert_matrix_beyond_32_bit_offsets_rejected():
    """One int8 expert matrix of I*d bytes >= 2^31 (d = 65536, I = 32768)."""
    s = shape(T=2, d=65536, E=8, k=2, I=32768, wbits=8, act_dtype=B.MOE_ACT_F32)
    with pytest.raises(B.MoeError) as ei:
        _forward(s)
    assert ei.value.code == B.MOE_EUNSUPPORTED and "weight matrix" in str(ei.value)


def test_matrix_core_path_refuses_what_it_cannot_take():
    """MOE_PATH_GEMM with sizes that are not multiples of 64 (bf16 or fp32 activations) is refused with a
    message; MOE_PATH_AUTO sends such shapes to the decode kernels instead."""
    for kw in (dict(act_dtype=B.MOE_ACT_F32, d=272, wbits=8), dict(act_dtype=B.MOE_ACT_BF16, d=272, wbits=8),
               dict(act_dtype=B.MOE_ACT_F32, I=528)):
        s = shape(T=64, path=B.MOE_PATH_GEMM, **kw)
        with pytest.raises(B.MoeError) as ei:
            _forward(s)
        assert ei.value.code == B.MOE_EUNSUPPORTED and "matrix-core path" in str(ei.value)


def test_static_forward_checks_before_anything_runs():
    """moe_forward_static validates like moe_forward and refuses a shape whose scratch need passes its static
    array (no GPU needed: the call fails before looking the array up)."""
    s = shape(T=8192, d=7168, E=256, k=8, I=2048, I_shared=2048, wbits=4, act_dtype=B.MOE_ACT_BF16,
              routed_scale=2.5)
    q = B.make_qffn(*([FAKE] * 9))
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(s, FAKE, q, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.code == B.MOE_EWORKSPACE and "static" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(shape(), FAKE, q, None, FAKE, FAKE, FAKE, None, FAKE, None, None, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "n_uniq" in str(ei.value)
    # an empty batch is a no-op here too
    B.moe_forward_static(shape(T=0), None, q, None, FAKE, None, FAKE, FAKE, None, None, None, stream=0)


def test_flags_checked():
    """Unknown flag bits are refused; the batch-invariant flag is accepted and sizes the router's fixed split."""
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(shape(flags=2), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
    assert ei.value.code == B.MOE_EINVAL and "flags" in str(ei.value)
    big = dict(T=4096, d=7168, E=256, k=8, I=2048, I_shared=2048, wbits=4, act_dtype=B.MOE_ACT_BF16)
    assert B.moe_workspace_size(shape(flags=B.MOE_FLAG_BATCH_INVARIANT, **big)) > 0
    assert B.moe_workspace_size(shape(flags=B.MOE_FLAG_BATCH_INVARIANT)) > 0


def test_router_fields_checked():
    """Unknown routers and capacity factors out of range are refused; expert choice needs k = E and a factor;
    the softmax and expert-choice routers take no bias (NULL accepted), the sigmoid router needs it."""
    for kw, msg in ((dict(router=3), "router"), (dict(capacity_factor=-1.0), "capacity"),
                    (dict(capacity_factor=float("nan")), "capacity"),
                    (dict(router=B.MOE_ROUTER_EXPERT_CHOICE, capacity_factor=2.0), "expert choice"),
                    (dict(router=B.MOE_ROUTER_EXPERT_CHOICE, k=8, capacity_factor=0.0), "expert choice")):
        with pytest.raises(B.MoeError) as ei:
            B.moe_route(shape(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
        assert ei.value.code == B.MOE_EINVAL and msg in str(ei.value), str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(shape(), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
    assert "bias" in str(ei.value)
    # T = 0 returns before anything runs: no bias needed for the softmax and expert-choice routers
    B.moe_route(shape(T=0, router=B.MOE_ROUTER_SOFTMAX), None, FAKE, None, None, None, None, FAKE, HUGE_WS, stream=0)
    B.moe_route(shape(T=0, k=8, router=B.MOE_ROUTER_EXPERT_CHOICE, capacity_factor=2.0), None, FAKE, None, None, None,
                None, FAKE, HUGE_WS, stream=0)
    # the capacity step needs workspace beyond the partial sums
    base = B.moe_workspace_size(shape(T=5000))
    assert B.moe_workspace_size(shape(T=5000, capacity_factor=1.2)) >= base



def test_index_shape_checked():
    """The indexer's shape checks: heads and head dimension the kernels take, non-negative sizes, K >= 1."""
    for kw, code in ((dict(H=8), B.MOE_EUNSUPPORTED), (dict(D=96), B.MOE_EUNSUPPORTED), (dict(K=0), B.MOE_EINVAL),
                     (dict(T=-1), B.MOE_EINVAL), (dict(pos0=-1), B.MOE_EINVAL)):
        d = dict(T=2, S=100, H=64, D=128, K=16, pos0=98)
        d.update(kw)
        s = B.dsa_index_shape(**d)
        assert B.dsa_index_workspace_size(s) == 0
        with pytest.raises(B.MoeError) as ei:
            B.dsa_index_topk(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
        assert ei.value.code == code
    s = B.dsa_index_shape(T=2, S=100, H=64, D=128, K=16, pos0=98)
    assert B.dsa_index_workspace_size(s) == 2 * 100 * 8 + 256 - (2 * 100 * 8) % 256
    with pytest.raises(B.MoeError) as ei:
        B.dsa_index_topk(s, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, HUGE_WS, stream=0)
    assert "k is NULL" in str(ei.value)
    B.dsa_index_topk(B.dsa_index_shape(T=0, S=100, H=64, D=128, K=16, pos0=0), None, None, FAKE, FAKE, None, None,
                     FAKE, HUGE_WS, stream=0)


def test_cache_shape_checked():
    assert B.moe_cache_state_size(B.make_cache_shape(256, 32, 4)) >= 64 + 4 * (3 * 32 + 256)
    for bad in (B.make_cache_shape(0, 1), B.make_cache_shape(2048, 32), B.make_cache_shape(8, 9),
                B.make_cache_shape(8, 0), B.make_cache_shape(8, 4, 4), B.make_cache_shape(8, 4, -1),
                B.make_cache_shape(8, 4, 0, 2)):
        assert B.moe_cache_state_size(bad) == 0
        with pytest.raises(B.MoeError) as ei:
            B.moe_cache_plan(bad, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
        assert ei.value.code == B.MOE_EINVAL


def test_cache_plan_needs_slots_for_a_step():
    c = B.make_cache_shape(256, 36, 4)  # 32 unpinned slots
    args = [FAKE] * 7
    B.lib()  # a step of T*k <= 32 experts would be accepted (not run here: it would enqueue)
    with pytest.raises(B.MoeError) as ei:
        B.moe_cache_plan(c, 5, 8, *args, stream=0)  # up to 40 missing experts
    assert ei.value.code == B.MOE_EINVAL and "unpinned slots" in str(ei.value)
    with pytest.raises(B.MoeError) as ei:
        B.moe_cache_plan(c, 4, 8, FAKE, None, *args[2:], stream=0)  # n_uniq NULL
    assert ei.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as ei:
        B.moe_cache_plan(c, 4, 8, FAKE + 4, *args[1:], stream=0)  # misaligned
    assert ei.value.code == B.MOE_EALIGN


def test_cache_init_checks_pinned_ids_on_the_host():
    c = B.make_cache_shape(16, 8, 3)
    for ids in ([1, 2, 2], [1, 2, 16], [-1, 2, 3]):
        with pytest.raises(B.MoeError) as ei:
            B.moe_cache_init(c, ids, FAKE, FAKE, FAKE, stream=0)
        assert ei.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as ei:
        B.moe_cache_init(c, None, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.code == B.MOE_EINVAL


def test_cached_forward_and_fetch_check_shapes():
    s = shape(E=8, k=2)
    q = B.moe_qffn(*([FAKE] * 9))
    with pytest.raises(B.MoeError) as ei:  # cache E differs from the layer's
        B.moe_cache_fetch(s, B.make_cache_shape(16, 4), q, q, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_cached(s, B.make_cache_shape(16, 4), FAKE, q, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as ei:  # state NULL
        B.moe_forward_cached(s, B.make_cache_shape(8, 4), FAKE, q, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL
    sh = shape(E=8, k=2, I_shared=256)
    with pytest.raises(B.MoeError) as ei:  # the shared weights stay required with y_shared = NULL
        B.moe_forward_cached(sh, B.make_cache_shape(8, 4), FAKE, q, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             None, None, FAKE, 1 << 30, stream=0)
    assert ei.value.code == B.MOE_EINVAL


def test_route_permute_checks():
    s = shape(T=2)
    need = B.moe_workspace_size(s)
    args = dict(x=FAKE, W_r=FAKE, bias=FAKE, topk_idx=FAKE, topk_w=FAKE, gap=None, counts=FAKE, offsets=FAKE,
                perm=FAKE, inv=FAKE, uniq=FAKE, n_uniq=FAKE, ws=FAKE)
    for miss in ("counts", "offsets", "perm", "inv", "uniq", "n_uniq", "W_r", "topk_idx"):
        a = dict(args)
        a[miss] = None
        with pytest.raises(B.MoeError) as ei:
            B.moe_route_permute(s, **a, ws_bytes=need, stream=0)
        assert ei.value.code == B.MOE_EINVAL, miss
    with pytest.raises(B.MoeError) as ei:
        B.moe_route_permute(s, **args, ws_bytes=need - 1, stream=0)
    assert ei.value.code == B.MOE_EWORKSPACE


@pytest.mark.parametrize("T", [1, 3])
def test_layer_checks(T):
    """moe_layer refuses what any of its three calls refuses, before anything is enqueued (the fake pointers are
    never dereferenced), and needs the workspace moe_workspace_size gives: at T = 1 that covers the router's
    partial sums beside the forward's area."""
    s = shape(T=T, I_shared=256)
    need = B.moe_workspace_size(s)
    q = B.make_qffn(*([FAKE] * 9))
    args = dict(x=FAKE, W_r=FAKE, bias=FAKE, routed=q, shared=q, topk_idx=FAKE, topk_w=FAKE, gap=None, counts=FAKE,
                offsets=FAKE, perm=FAKE, inv=FAKE, uniq=FAKE, n_uniq=FAKE, y_perm=FAKE, y_shared=FAKE, y=FAKE,
                diag=None, ws=FAKE)
    for miss in ("x", "W_r", "bias", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "uniq", "n_uniq",
                 "y_perm", "y_shared", "y", "ws"):
        a = dict(args)
        a[miss] = None
        with pytest.raises(B.MoeError) as ei:
            B.moe_layer(s, **a, ws_bytes=need, stream=0)
        assert ei.value.code == (B.MOE_EWORKSPACE if miss == "ws" else B.MOE_EINVAL), miss
    a = dict(args)
    a["shared"] = B.make_qffn(*([FAKE] * 8 + [None]))
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer(s, **a, ws_bytes=need, stream=0)
    assert ei.value.code == B.MOE_EINVAL
    a = dict(args)
    a["y"] = FAKE + 4
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer(s, **a, ws_bytes=need, stream=0)
    assert ei.value.code == B.MOE_EALIGN
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer(s, **args, ws_bytes=need - 1, stream=0)
    assert ei.value.code == B.MOE_EWORKSPACE


def test_abi_version():
    assert B.moe_abi_version() == 4
