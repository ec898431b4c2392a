"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.
No GPU is touched: every call here fails validation (or is a size query)."""
import ctypes
import os
import re

import pytest

from sparse_moe_ffn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_moe_ffn_amd import build
        build.build()
    return B.load()


def header_symbols():
    src = open(os.path.join(ROOT, "include", "mobmoe.h")).read()
    return set(re.findall(r"^(?:mm_status|const char\*|size_t|int64_t|int32_t)\s+(mm_\w+)\(", src, re.M))


def test_header_and_binding_agree():
    assert header_symbols() == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_symbols():
        assert hasattr(lib, name), name
    assert "gfx950" in B.version()


def test_status_strings(lib):
    assert lib.mm_status_string(0) == b"MM_OK"
    assert lib.mm_status_string(5) == b"MM_ERR_WORKSPACE"


FAKE = 1 << 20           # aligned, never dereferenced (validation fails first)
MISALIGNED = FAKE + 4


def S():
    return B.desc(768, 60, 384, 1536, 4, "int4g32")


def rc_of(fn, *args):
    return fn(*args)


def test_desc_validation(lib):
    bad = [B.desc(100, 60, 384, 1536, 4), B.desc(768, 65, 384, 1536, 4), B.desc(768, 60, 96, 1536, 4),
           B.desc(768, 60, 384, 100, 4), B.desc(768, 4, 384, 0, 5), B.desc(768, 60, 384, 0, 9)]
    for ds in bad:
        assert lib.mm_router_topk(ctypes.byref(ds), 4, FAKE, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_SHAPE
        assert B.workspace_bytes(ds, 4) == 0
    for ds in (B.desc(768, 60, 384, 0, 4, wfmt=7), B.desc(768, 60, 384, 0, 4, gating=4),
               B.desc(768, 60, 384, 0, 4, gating=-1),
               B.desc(768, 60, 384, 0, 4, out_dtype=2)):
        assert lib.mm_router_topk(ctypes.byref(ds), 4, FAKE, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_FORMAT
    assert lib.mm_router_topk(None, 4, FAKE, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_NULL
    assert b"desc" in lib.mm_last_error_string()


def test_null_and_alignment(lib):
    ds = S()
    assert lib.mm_router_topk(ctypes.byref(ds), 4, None, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_NULL
    assert b"x is NULL" in lib.mm_last_error_string()
    assert lib.mm_router_topk(ctypes.byref(ds), 4, MISALIGNED, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_ALIGN
    assert lib.mm_router_topk(ctypes.byref(ds), 4, FAKE, FAKE, MISALIGNED, FAKE, FAKE, None) == B.MM_ERR_ALIGN
    assert lib.mm_combine(ctypes.byref(ds), 4, FAKE, FAKE, FAKE, None, None, None) == B.MM_ERR_NULL
    assert lib.mm_act_quant_i8(3, 768, FAKE, None, FAKE, None) == B.MM_ERR_NULL
    w = B.Weight(FAKE, None)
    assert lib.mm_expert_down(ctypes.byref(ds), 4, FAKE, FAKE, FAKE, w, FAKE, None, 0, None) == B.MM_ERR_NULL
    assert b"w_down.scales" in lib.mm_last_error_string()


def test_zero_tokens_is_a_noop(lib):
    ds = S()
    assert lib.mm_router_topk(ctypes.byref(ds), 0, None, None, None, None, None, None) == B.MM_OK
    assert lib.mm_route_permute(ctypes.byref(ds), 0, None, None, None, None, None, 0, None) == B.MM_OK
    assert lib.mm_act_quant_i8(0, 768, None, None, None, None) == B.MM_OK
    assert lib.mm_combine(ctypes.byref(ds), 0, None, None, None, None, None, None) == B.MM_OK
    w = B.Weight(None, None)
    assert lib.mm_expert_gateup_swiglu(ctypes.byref(ds), 0, None, None, None, None, w, None, None,
                                       None, 0, None) == B.MM_OK


def test_shape_limits(lib):
    ds = S()
    assert lib.mm_router_topk(ctypes.byref(ds), -1, FAKE, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert lib.mm_router_topk(ctypes.byref(ds), (1 << 22) + 1, FAKE, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    noshared = B.desc(768, 60, 384, 0, 4)
    w = B.Weight(FAKE, FAKE)
    assert lib.mm_shared_expert(ctypes.byref(noshared), 4, FAKE, FAKE, w, w, FAKE, FAKE, 1 << 20,
                                None) == B.MM_ERR_SHAPE
    assert lib.mm_quantize_int4g32(4, 40, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert lib.mm_prepack_int4g32(1, 48, 64, FAKE, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE


def test_format_rules(lib):
    f32 = B.desc(256, 60, 64, 256, 4, "f32")
    w_with_scales = B.Weight(FAKE, FAKE)
    assert lib.mm_expert_down(ctypes.byref(f32), 4, FAKE, None, FAKE, w_with_scales, FAKE, None, 0,
                              None) == B.MM_ERR_FORMAT
    w = B.Weight(FAKE, None)
    assert lib.mm_expert_down_dbg(ctypes.byref(f32), 4, FAKE, None, FAKE, w, FAKE, None, 0, FAKE,
                                  None) == B.MM_ERR_FORMAT


def test_workspace_checks(lib):
    ds = S()
    need = B.workspace_bytes(ds, 2048, B.MM_WS_ROUTE)
    assert need == ((2048 * 4 + 255) // 256) * 60 * 4
    assert lib.mm_route_permute(ctypes.byref(ds), 2048, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                None) == B.MM_ERR_WORKSPACE
    gu = B.workspace_bytes(ds, 2048, B.MM_WS_GATEUP)
    assert gu >= 2048 * 4 * 384 * 4
    w = B.Weight(FAKE, FAKE)
    assert lib.mm_expert_gateup_swiglu(ctypes.byref(ds), 2048, FAKE, FAKE, FAKE, FAKE, w, FAKE, FAKE,
                                       FAKE, gu - 1, None) == B.MM_ERR_WORKSPACE
    sh = B.workspace_bytes(ds, 2048, B.MM_WS_SHARED)
    assert lib.mm_shared_expert(ctypes.byref(ds), 2048, FAKE, FAKE, w, w, FAKE, FAKE, sh - 1,
                                None) == B.MM_ERR_WORKSPACE
    assert B.workspace_bytes(ds, 2048, B.MM_WS_MAX) == max(
        B.workspace_bytes(ds, 2048, i) for i in range(4))


def test_prepacked_sizes(lib):
    assert B.prepacked_bytes(768, 768) == 768 * 384
    assert B.prepacked_scale_bytes(768, 768) == 768 * 24 * 4
    assert B.prepacked_bytes(48, 64) == 0


def test_forward_checks(lib):
    """mm_moe_forward validates everything before any launch."""
    ds = S()
    w = B.Weight(FAKE, FAKE)
    need = B.workspace_bytes(ds, 2048, B.MM_WS_FORWARD)
    # at least the routing tables, the quantised rows and the expert outputs
    assert need >= 2048 * 4 * (768 * 4 + 384 * 5) + 2048 * (768 * 5 + 1536 * 5)
    args = lambda ws_bytes: (ctypes.byref(ds), 2048, FAKE, FAKE, None, w, w, w, w, FAKE, FAKE, FAKE,
                             None, 0.0, FAKE, ws_bytes, None)
    assert lib.mm_moe_forward(*args(need - 1)) == B.MM_ERR_WORKSPACE
    assert b"forward workspace" in lib.mm_last_error_string()
    assert lib.mm_moe_forward(ctypes.byref(ds), 0, None, None, None, w, w, w, w, None, None, None,
                              None, 0.0, None, 0, None) == B.MM_OK
    assert lib.mm_moe_forward(ctypes.byref(ds), 4, None, FAKE, None, w, w, w, w, FAKE, FAKE, FAKE,
                              None, 0.0, FAKE, need, None) == B.MM_ERR_NULL
    no_scales = B.Weight(FAKE, None)
    assert lib.mm_moe_forward(ctypes.byref(ds), 4, FAKE, FAKE, None, w, w, no_scales, w, FAKE, FAKE,
                              FAKE, None, 0.0, FAKE, need, None) == B.MM_ERR_NULL
    assert b"ws_gateup.scales" in lib.mm_last_error_string()
    # the RMSNorm output needs FP32 y and a positive eps
    assert lib.mm_moe_forward(ctypes.byref(ds), 4, FAKE, FAKE, None, w, w, w, w, FAKE, FAKE, FAKE,
                              FAKE, 0.0, FAKE, need, None) == B.MM_ERR_SHAPE
    bf = B.desc(768, 60, 384, 1536, 4, "bf16", out_dtype=B.MM_OUT_BF16)
    wb = B.Weight(FAKE, None)
    assert lib.mm_moe_forward(ctypes.byref(bf), 4, FAKE, FAKE, None, wb, wb, wb, wb, FAKE, FAKE, FAKE,
                              FAKE, 1e-5, FAKE, 1 << 30, None) == B.MM_ERR_FORMAT
    # without a shared expert its weights are not looked at
    noshared = B.desc(768, 60, 384, 0, 4)
    zero = B.Weight(None, None)
    assert B.workspace_bytes(noshared, 2048, B.MM_WS_FORWARD) < need


def test_decode_checks(lib):
    """mm_moe_decode: the one-launch form's limits and every argument check
    happen on the host before the launch."""
    ds = S()
    w = B.Weight(FAKE, FAKE)
    for T in (1, 2, 3, 4):
        assert B.moe_decode_supported(ds, T)
    assert not B.moe_decode_supported(ds, 5) and not B.moe_decode_supported(ds, 0)
    need = B.workspace_bytes(ds, 1, B.MM_WS_DECODE)
    # one size for every T <= 4: state + routed rows/outputs for 4 tokens
    assert need == B.workspace_bytes(ds, 4, B.MM_WS_DECODE)
    assert need >= 4 * 4 * (384 + 768) * 4 + 4 * (1536 + 768) * 4
    assert B.workspace_bytes(ds, 5, B.MM_WS_DECODE) == 0
    args = lambda T, ws_bytes, y_norm=None, eps=0.0, d=ds, wt=w: (
        ctypes.byref(d), T, FAKE, FAKE, None, wt, wt, wt, wt, FAKE, FAKE, FAKE, y_norm, eps, FAKE,
        ws_bytes, None)
    assert lib.mm_moe_decode(*args(1, need - 1)) == B.MM_ERR_WORKSPACE
    assert lib.mm_moe_decode(*args(5, need)) == B.MM_ERR_SHAPE
    assert lib.mm_moe_decode(*args(-1, need)) == B.MM_ERR_SHAPE
    assert lib.mm_moe_decode(*args(0, need)) == B.MM_OK
    assert lib.mm_moe_decode(*args(2, need, FAKE, 0.0)) == B.MM_ERR_SHAPE  # eps must be positive
    bf = B.desc(768, 60, 384, 1536, 4, "bf16")
    assert lib.mm_moe_decode(*args(2, need, d=bf, wt=B.Weight(FAKE, None))) == B.MM_ERR_FORMAT
    assert not B.moe_decode_supported(bf, 1)
    wide = B.desc(1536, 60, 768, 3072, 4)  # d beyond the one-launch router's 1280
    assert not B.moe_decode_supported(wide, 1)
    odd = B.desc(704, 60, 320, 640, 4)     # d % 128 != 0
    assert not B.moe_decode_supported(odd, 1)
    assert lib.mm_moe_decode(*args(1, need, d=odd)) == B.MM_ERR_SHAPE
    unaligned = FAKE + 4
    assert lib.mm_moe_decode(ctypes.byref(ds), 1, unaligned, FAKE, None, w, w, w, w, FAKE, FAKE,
                             FAKE, None, 0.0, FAKE, need, None) == B.MM_ERR_ALIGN


def test_decode_noalloc_checks(lib):
    """The no-allocation decode form: the checks of mm_moe_decode, and a layer
    whose state and rows exceed the fixed 512 KiB device scratch is refused on
    the host (before the scratch is looked up)."""
    w = B.Weight(FAKE, FAKE)
    args = lambda d, T: (ctypes.byref(d), T, FAKE, FAKE, None, w, w, w, w, FAKE, FAKE, FAKE, None,
                         0.0, None)
    big = B.desc(1280, 64, 2560, 2560, 8)  # 32 slots of 2560 + 1280 floats: over 512 KiB
    assert B.moe_decode_supported(big, 4)
    assert B.workspace_bytes(big, 4, B.MM_WS_DECODE) > 512 * 1024
    assert lib.mm_moe_decode_noalloc(*args(big, 4)) == B.MM_ERR_WORKSPACE
    assert b"512" in lib.mm_last_error_string() or b"524288" in lib.mm_last_error_string()
    ds = S()
    assert B.workspace_bytes(ds, 4, B.MM_WS_DECODE) <= 512 * 1024
    assert lib.mm_moe_decode_noalloc(*args(ds, 5)) == B.MM_ERR_SHAPE
    assert lib.mm_moe_decode_noalloc(*args(ds, 0)) == B.MM_OK
    assert lib.mm_moe_decode_noalloc(ctypes.byref(ds), 1, None, FAKE, None, w, w, w, w, FAKE, FAKE,
                                     FAKE, None, 0.0, None) == B.MM_ERR_NULL


def test_layout_and_pair_checks(lib):
    """mm_act_quant_i8_layout and the merged product entries validate before
    any launch."""
    I32 = ctypes.c_int32
    assert lib.mm_act_quant_i8_layout(4, 768, FAKE, FAKE, FAKE, I32(3), None) == B.MM_ERR_FORMAT
    assert lib.mm_act_quant_i8_layout(4, 768, FAKE, FAKE, FAKE, I32(-1), None) == B.MM_ERR_FORMAT
    for lay in (B.MM_ACT_GROUP_MAJOR, B.MM_ACT_F16_PAIRED):
        assert lib.mm_act_quant_i8_layout(4, 704, FAKE, FAKE, FAKE, I32(lay), None) == B.MM_ERR_SHAPE
        assert lib.mm_act_quant_i8_layout(4, 768, None, FAKE, FAKE, I32(lay), None) == B.MM_ERR_NULL
    assert lib.mm_act_quant_i8_layout(0, 768, None, None, None, I32(B.MM_ACT_ROW_MAJOR),
                                      None) == B.MM_OK
    ds = S()
    w = B.Weight(FAKE, FAKE)
    args = lambda d, T, x, wu: (ctypes.byref(d), T, x, FAKE, FAKE, FAKE, wu, wu, FAKE, FAKE, None)
    assert lib.mm_expert_gateup_pair_f32(*args(ds, 0, None, w)) == B.MM_OK
    assert lib.mm_expert_gateup_pair_f32(*args(ds, 4, None, w)) == B.MM_ERR_NULL
    assert lib.mm_expert_gateup_pair_f32(*args(ds, 4, FAKE, B.Weight(FAKE, None))) == B.MM_ERR_NULL
    assert lib.mm_expert_gateup_pair_f32(*args(ds, 4, FAKE + 8, w)) == B.MM_ERR_ALIGN
    bf = B.desc(768, 60, 384, 1536, 4, "bf16")
    assert lib.mm_expert_gateup_pair_f32(*args(bf, 4, FAKE, B.Weight(FAKE, None))) == B.MM_ERR_FORMAT
    noshared = B.desc(768, 60, 384, 0, 4)
    assert lib.mm_expert_gateup_pair_f32(*args(noshared, 4, FAKE, w)) == B.MM_ERR_SHAPE
    for odd in (B.desc(704, 60, 320, 640, 4), B.desc(768, 60, 352, 1536, 4),
                B.desc(768, 60, 384, 1504, 4)):
        assert lib.mm_expert_gateup_pair_f32(*args(odd, 4, FAKE, w)) == B.MM_ERR_SHAPE
    # the group-sum twin needs its two extra outputs
    assert lib.mm_expert_gateup_pair_f32_dbg(ctypes.byref(ds), 4, FAKE, FAKE, FAKE, FAKE, w, w, FAKE,
                                             FAKE, None, FAKE, None) == B.MM_ERR_NULL
    # the merged down products
    dargs = lambda d, T, hr, wu, f: (ctypes.byref(d), T, hr, FAKE, FAKE, FAKE, FAKE, wu, wu, f,
                                     FAKE, None)
    assert lib.mm_expert_down_pair_f32(*dargs(ds, 0, None, w, None)) == B.MM_OK
    assert lib.mm_expert_down_pair_f32(*dargs(ds, 4, None, w, FAKE)) == B.MM_ERR_NULL
    assert lib.mm_expert_down_pair_f32(*dargs(ds, 4, FAKE, w, None)) == B.MM_ERR_NULL
    assert lib.mm_expert_down_pair_f32(*dargs(ds, 4, FAKE, B.Weight(FAKE, None), FAKE)) == \
        B.MM_ERR_NULL
    assert lib.mm_expert_down_pair_f32(*dargs(bf, 4, FAKE, B.Weight(FAKE, None), FAKE)) == \
        B.MM_ERR_FORMAT
    assert lib.mm_expert_down_pair_f32(*dargs(noshared, 4, FAKE, w, FAKE)) == B.MM_ERR_SHAPE
    assert lib.mm_expert_down_pair_f32_dbg(ctypes.byref(ds), 4, FAKE, FAKE, FAKE, FAKE, FAKE, w, w,
                                           FAKE, FAKE, FAKE, None, None) == B.MM_ERR_NULL


def test_linear_w4a8_checks(lib):
    """The dense W4A8 linear: shape, NULL and alignment checks on the host
    (nothing reaches a device); zero rows is a no-op without pointers."""
    W = B.weight(None, None)
    Wf = B.Weight(FAKE, FAKE)
    f = lib.mm_linear_w4a8
    assert f(0, 768, 256, None, None, W, None, None) == B.MM_OK
    for rows, K, N in [(-1, 768, 256), (4, 100, 256), (4, 768, 96), (4, 0, 64), (1 << 22, 1024, 64)]:
        assert f(rows, K, N, FAKE, FAKE, Wf, FAKE, None) == B.MM_ERR_SHAPE
    assert f(4, 768, 256, None, FAKE, Wf, FAKE, None) == B.MM_ERR_NULL
    assert f(4, 768, 256, FAKE, FAKE, W, FAKE, None) == B.MM_ERR_NULL
    assert f(4, 768, 256, FAKE, FAKE, Wf, MISALIGNED, None) == B.MM_ERR_ALIGN


def test_attention_checks(lib):
    """KV append and decode attention: shape, workspace, NULL checks on the host."""
    a, d = lib.mm_kv_append_i8, lib.mm_attn_decode_i8
    assert a(0, 4, 64, 16, None, None, None, None, None, None, None, None) == B.MM_OK
    for nkv, dh, maxT in [(0, 64, 16), (4, 32, 16), (4, 64, 0)]:
        assert a(2, nkv, dh, maxT, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert a(2, 4, 64, 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.MM_ERR_NULL
    ws = lib.mm_attn_workspace_bytes(2, 4, 16)
    assert ws > 0 and lib.mm_attn_workspace_bytes(2, 0, 16) == 0
    args = (FAKE,) * 7
    for nh, nkv, ml in [(12, 5, 16), (40, 4, 16), (12, 4, 0), (12, 4, 17)]:
        assert d(2, nh, nkv, 64, 16, ml, *args, FAKE, ws, None) == B.MM_ERR_SHAPE
    assert d(2, 12, 4, 64, 16, 16, *args, FAKE, ws - 4, None) == B.MM_ERR_WORKSPACE
    assert d(2, 12, 4, 64, 16, 16, None, *args[1:], FAKE, ws, None) == B.MM_ERR_NULL


def test_training_side_checks(lib):
    """Bias update, drop-and-pad and fake quantisation: host-side checks,
    and the exact capacity arithmetic."""
    from fractions import Fraction
    import math
    assert lib.mm_bias_update(0, 60, 4, None, 1e-3, None, None, None) == B.MM_OK
    for E, k in [(0, 4), (4097, 4), (60, 0)]:
        assert lib.mm_bias_update(8, E, k, FAKE, 1e-3, FAKE, None, None) == B.MM_ERR_SHAPE
    assert lib.mm_bias_update(8, 60, 4, None, 1e-3, FAKE, None, None) == B.MM_ERR_NULL
    for T, k, E in [(2048, 4, 60), (8192, 4, 60), (1, 4, 60), (7, 2, 3), (0, 4, 60)]:
        assert lib.mm_drop_pad_capacity(T, k, E, 3, 2) == math.ceil(Fraction(3, 2) * T * k / E)
    assert lib.mm_drop_pad_capacity(8, 4, 0, 3, 2) == -1
    args = (FAKE,) * 8
    assert lib.mm_drop_pad(8, 60, 4, -1, *args, None) == B.MM_ERR_SHAPE
    assert lib.mm_drop_pad(8, 0, 4, 10, *args, None) == B.MM_ERR_SHAPE
    assert lib.mm_drop_pad(8, 60, 4, 10, None, *args[1:], None) == B.MM_ERR_NULL
    assert lib.mm_drop_pad(8, 60, 4, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == B.MM_ERR_NULL
    fq = lib.mm_fake_quant
    assert fq(4, 64, 5, 32, FAKE, FAKE, None, None, None) == B.MM_ERR_SHAPE
    assert fq(4, 48, 4, 32, FAKE, FAKE, None, None, None) == B.MM_ERR_SHAPE
    assert fq(4, 64, 4, 16, FAKE, FAKE, None, None, None) == B.MM_ERR_SHAPE
    assert fq(4, 66, 8, 66, FAKE, FAKE, None, None, None) == B.MM_ERR_SHAPE
    assert fq(4, 64, 4, 32, FAKE, FAKE, FAKE, None, None) == B.MM_ERR_NULL
    assert fq(4, 64, 4, 32, None, FAKE, None, None, None) == B.MM_ERR_NULL
    assert fq(0, 64, 4, 32, None, None, None, None, None) == B.MM_OK


def test_expert_training_checks(lib):
    f, b = lib.mm_expert_train_forward_f32, lib.mm_expert_backward_f32
    for E, d, h in [(0, 64, 32), (3, 60, 32), (3, 64, 24), (5000, 64, 32)]:
        assert f(E, d, h, 10, *(FAKE,) * 7, None) == B.MM_ERR_SHAPE
    assert f(3, 64, 32, 0, *(None,) * 7, None) == B.MM_OK
    assert f(3, 64, 32, 10, None, *(FAKE,) * 6, None) == B.MM_ERR_NULL
    ws = lib.mm_expert_backward_workspace_bytes(10, 32)
    assert ws == 10 * 3 * 32 * 4
    assert b(3, 64, 32, 10, *(FAKE,) * 11, ws - 4, None) == B.MM_ERR_WORKSPACE
    assert b(3, 64, 32, 10, *(FAKE,) * 10, None, ws, None) == B.MM_ERR_NULL
    assert lib.mm_gather_rows(4, 6, 2, FAKE, None, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert lib.mm_gather_rows(4, 8, 2, None, None, FAKE, FAKE, None) == B.MM_ERR_NULL


def test_router_backward_checks(lib):
    rb = lib.mm_router_backward_f32
    for E, d in [(62, 768), (68, 768), (60, 760)]:
        ds = B.desc(d, E, 384, 0, 4)
        assert rb(ctypes.byref(ds), 8, *(FAKE,) * 7, 1e-4, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    ds = B.desc(768, 60, 384, 0, 4)
    assert rb(ctypes.byref(ds), 0, *(FAKE,) * 7, 1e-4, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert rb(ctypes.byref(ds), 8, *(FAKE,) * 7, 1e-4, FAKE, None, FAKE, None) == B.MM_ERR_NULL


def test_profile_events_checks(lib):
    assert lib.mm_set_profile_events(FAKE, None) == B.MM_ERR_NULL
    assert lib.mm_set_profile_events(None, FAKE) == B.MM_ERR_NULL
    assert lib.mm_set_profile_events(None, None) == B.MM_OK


def test_add_rmsnorm_checks(lib):
    """Residual add + RMSNorm: shape, eps, NULL and aliasing checks on the host."""
    f = lib.mm_add_rmsnorm_f32
    assert f(0, 768, 1e-5, None, None, None, None, None) == B.MM_OK
    assert f(2, 0, 1e-5, FAKE, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert f(-1, 768, 1e-5, FAKE, FAKE, FAKE, FAKE, None) == B.MM_ERR_SHAPE
    assert f(2, 768, 0.0, FAKE, FAKE, FAKE + 4096, FAKE + 8192, None) == B.MM_ERR_SHAPE
    assert f(2, 768, 1e-5, None, FAKE, FAKE + 4096, None, None) == B.MM_ERR_NULL
    assert f(2, 768, 1e-5, FAKE, None, FAKE + 4096, None, None) == B.MM_ERR_NULL
    assert f(2, 768, 1e-5, FAKE, FAKE + 4096, None, None, None) == B.MM_ERR_NULL
    assert f(2, 768, 1e-5, FAKE, FAKE + 4096, FAKE, None, None) == B.MM_ERR_SHAPE        # sum == x
    assert f(2, 768, 1e-5, FAKE, FAKE + 4096, FAKE + 8192, FAKE + 8192, None) == B.MM_ERR_SHAPE


def test_kv_cache_bytes_match_eq5():
    """The library's INT8 KV cache for MobileMoE-S/M/L (20/26/32 layers, 4 KV
    heads of 64) at the 8K mid-training context: its code bytes for K and V
    over all layers equal eq. (5)'s KV-cache term with b_kv = 8, and its
    per-vector FP32 scales add one sixteenth of that.  With the printed total
    parameter counts in INT4 (eq. (5)'s weight term) each model's memory
    function stays under the page's DRAM budget of about 5 GB."""
    import json
    g = {e["key"]: e["value"] for e in
         json.load(open(os.path.join(ROOT, "tests", "golden", "mobilemoe_printed_shapes.json")))["entries"]}
    T, n_kv, d_h, b_kv, b_w = (g["mid_training_context"], g["kv_heads"], g["head_dim"], g["kv_bits"],
                               g["weight_bits"])
    for key, n_l in (("S", 20), ("M", 26), ("L", 32)):
        term = b_kv * 2 * T * n_l * n_kv * d_h // 8                 # eq. (5), bytes
        codes = B.kv_cache_bytes(1, n_kv, d_h, T, B.MM_KV_CODES)    # one layer, one of K / V
        scales = B.kv_cache_bytes(1, n_kv, d_h, T, B.MM_KV_SCALES)
        assert 2 * n_l * codes == term
        assert 2 * n_l * scales * 16 == term
        assert B.kv_cache_bytes(8, n_kv, d_h, T, B.MM_KV_CODES) == 8 * codes
        mem = b_w / 8 * g[f"total_params_{key}"] + term
        assert mem < g["dram_budget_bytes"], (key, mem)
    assert B.kv_cache_bytes(1, 0, 64, T, B.MM_KV_CODES) == 0
    assert B.kv_cache_bytes(1, 4, 64, T, 7) == 0
