"""Thin ctypes binding of libmobmoe (include/mobmoe.h).

Every function here only marshals arguments: torch device tensors become raw
device pointers, the current torch stream becomes the HIP stream, and a
non-OK status becomes an MMError carrying the library's message.  All
computation happens in the library's HIP kernels.  If libmobmoe.so is missing
the import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# MOBMOE_LIB names another build of the same sources (the host-sanitizer build
# of the argument checks, tests/test_sanitizers.py).
LIB_PATH = os.environ.get("MOBMOE_LIB") or os.path.join(HERE, "libmobmoe.so")

MM_OK, MM_ERR_NULL, MM_ERR_SHAPE, MM_ERR_ALIGN, MM_ERR_FORMAT, MM_ERR_WORKSPACE, MM_ERR_HIP = range(7)
MM_W_F32, MM_W_INT4G32, MM_W_BF16 = range(3)
MM_GATE_SOFTMAX, MM_GATE_SIGMOID_NORM, MM_GATE_BIAS_SELECT_ONLY = 0, 1, 2
MM_OUT_F32, MM_OUT_BF16 = range(2)
MM_WS_ROUTE, MM_WS_GATEUP, MM_WS_DOWN, MM_WS_SHARED, MM_WS_MAX, MM_WS_FORWARD, MM_WS_DECODE = range(7)
MM_ACT_ROW_MAJOR, MM_ACT_GROUP_MAJOR, MM_ACT_F16_PAIRED = range(3)

WFMT = {"f32": MM_W_F32, "int4g32": MM_W_INT4G32, "bf16": MM_W_BF16}

# Every symbol include/mobmoe.h declares.
EXPORTS = (
    "mm_version", "mm_status_string", "mm_last_error_string", "mm_workspace_bytes",
    "mm_quantize_int4g32", "mm_prepacked_bytes", "mm_prepacked_scale_bytes", "mm_prepack_int4g32",
    "mm_convert_bf16", "mm_router_topk", "mm_route_permute", "mm_act_quant_i8",
    "mm_expert_gateup_swiglu", "mm_expert_down", "mm_shared_expert", "mm_combine",
    "mm_rmsnorm_f32", "mm_expert_gateup_swiglu_dbg", "mm_expert_down_dbg", "mm_moe_forward",
    "mm_act_quant_i8_layout", "mm_expert_gateup_pair_f32", "mm_linear_w4a8",
    "mm_attn_workspace_bytes", "mm_kv_append_i8", "mm_attn_decode_i8",
    "mm_bias_update", "mm_drop_pad_capacity", "mm_drop_pad", "mm_fake_quant",
    "mm_gather_rows", "mm_expert_train_forward_f32", "mm_expert_backward_workspace_bytes",
    "mm_expert_backward_f32", "mm_router_backward_f32", "mm_set_profile_events",
    "mm_moe_decode", "mm_moe_decode_supported", "mm_moe_decode_noalloc",
    "mm_expert_gateup_pair_f32_dbg", "mm_expert_down_pair_f32", "mm_expert_down_pair_f32_dbg",
    "mm_add_rmsnorm_f32", "mm_kv_cache_bytes",
)


class MMError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


STATUS_NAMES = {0: "MM_OK", 1: "MM_ERR_NULL", 2: "MM_ERR_SHAPE", 3: "MM_ERR_ALIGN",
                4: "MM_ERR_FORMAT", 5: "MM_ERR_WORKSPACE", 6: "MM_ERR_HIP"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("shared_hidden", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("gating", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class Weight(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_VP, _I64, _I32, _SZ, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_DESC = ctypes.POINTER(LayerDesc)

_SIGS = {
    "mm_version": ([], ctypes.c_char_p),
    "mm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "mm_last_error_string": ([], ctypes.c_char_p),
    "mm_workspace_bytes": ([_DESC, _I64, _I32], _SZ),
    "mm_quantize_int4g32": ([_I64, _I64, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_prepacked_bytes": ([_I64, _I64], _SZ),
    "mm_prepacked_scale_bytes": ([_I64, _I64], _SZ),
    "mm_prepack_int4g32": ([_I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_convert_bf16": ([_I64, _VP, _VP, _VP], ctypes.c_int),
    "mm_router_topk": ([_DESC, _I64, _VP, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_route_permute": ([_DESC, _I64, _VP, _VP, _VP, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "mm_act_quant_i8": ([_I64, _I64, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_act_quant_i8_layout": ([_I64, _I64, _VP, _VP, _VP, _I32, _VP], ctypes.c_int),
    "mm_expert_gateup_pair_f32": ([_DESC, _I64, _VP, _VP, _VP, _VP, Weight, Weight, _VP, _VP, _VP],
                                  ctypes.c_int),
    "mm_expert_gateup_pair_f32_dbg": ([_DESC, _I64, _VP, _VP, _VP, _VP, Weight, Weight, _VP, _VP,
                                       _VP, _VP, _VP], ctypes.c_int),
    "mm_expert_down_pair_f32": ([_DESC, _I64, _VP, _VP, _VP, _VP, _VP, Weight, Weight, _VP, _VP,
                                 _VP], ctypes.c_int),
    "mm_expert_down_pair_f32_dbg": ([_DESC, _I64, _VP, _VP, _VP, _VP, _VP, Weight, Weight, _VP,
                                     _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_expert_gateup_swiglu": ([_DESC, _I64, _VP, _VP, _VP, _VP, Weight, _VP, _VP, _VP, _SZ, _VP],
                                ctypes.c_int),
    "mm_expert_gateup_swiglu_dbg": ([_DESC, _I64, _VP, _VP, _VP, _VP, Weight, _VP, _VP, _VP, _SZ,
                                     _VP, _VP], ctypes.c_int),
    "mm_expert_down": ([_DESC, _I64, _VP, _VP, _VP, Weight, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "mm_expert_down_dbg": ([_DESC, _I64, _VP, _VP, _VP, Weight, _VP, _VP, _SZ, _VP, _VP],
                           ctypes.c_int),
    "mm_shared_expert": ([_DESC, _I64, _VP, _VP, Weight, Weight, _VP, _VP, _SZ, _VP], ctypes.c_int),
    "mm_combine": ([_DESC, _I64, _VP, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_rmsnorm_f32": ([_I64, _I64, _F, _VP, _VP, _VP], ctypes.c_int),
    "mm_add_rmsnorm_f32": ([_I64, _I64, _F, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_kv_cache_bytes": ([_I64, _I32, _I32, _I64, _I32], _SZ),
    "mm_linear_w4a8": ([_I64, _I64, _I64, _VP, _VP, Weight, _VP, _VP], ctypes.c_int),
    "mm_attn_workspace_bytes": ([_I64, _I32, _I64], _SZ),
    "mm_kv_append_i8": ([_I64, _I32, _I32, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
                        ctypes.c_int),
    "mm_attn_decode_i8": ([_I64, _I32, _I32, _I32, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                           _VP, _SZ, _VP], ctypes.c_int),
    "mm_bias_update": ([_I64, _I32, _I32, _VP, _F, _VP, _VP, _VP], ctypes.c_int),
    "mm_drop_pad_capacity": ([_I64, _I32, _I32, _I32, _I32], _I64),
    "mm_drop_pad": ([_I64, _I32, _I32, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
                    ctypes.c_int),
    "mm_fake_quant": ([_I64, _I64, _I32, _I64, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_gather_rows": ([_I64, _I64, _I32, _VP, _VP, _VP, _VP, _VP], ctypes.c_int),
    "mm_expert_train_forward_f32": ([_I32, _I32, _I32, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
                                    ctypes.c_int),
    "mm_expert_backward_workspace_bytes": ([_I64, _I32], _SZ),
    "mm_expert_backward_f32": ([_I32, _I32, _I32, _I64] + [_VP] * 11 + [_SZ, _VP], ctypes.c_int),
    "mm_router_backward_f32": ([_DESC, _I64] + [_VP] * 7 + [_F] + [_VP] * 4, ctypes.c_int),
    "mm_set_profile_events": ([_VP, _VP], ctypes.c_int),
    "mm_moe_forward": ([_DESC, _I64, _VP, _VP, _VP, Weight, Weight, Weight, Weight, _VP, _VP, _VP,
                        _VP, _F, _VP, _SZ, _VP], ctypes.c_int),
    "mm_moe_decode": ([_DESC, _I64, _VP, _VP, _VP, Weight, Weight, Weight, Weight, _VP, _VP, _VP,
                       _VP, _F, _VP, _SZ, _VP], ctypes.c_int),
    "mm_moe_decode_supported": ([_DESC, _I64], _I32),
    "mm_moe_decode_noalloc": ([_DESC, _I64, _VP, _VP, _VP, Weight, Weight, Weight, Weight, _VP, _VP,
                               _VP, _VP, _F, _VP], ctypes.c_int),
}

_lib = None


def load() -> ctypes.CDLL:
    """Loads libmobmoe.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_moe_ffn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, name: str):
    if rc != MM_OK:
        raise MMError(rc, name, load().mm_last_error_string().decode())


def desc(d: int, E: int, h: int, hs: int, k: int, wfmt="int4g32", gating: int = 0,
         out_dtype: int = MM_OUT_F32) -> LayerDesc:
    return LayerDesc(d, E, h, hs, k, WFMT[wfmt] if isinstance(wfmt, str) else wfmt, gating, out_dtype)


def weight(data, scales=None) -> Weight:
    return Weight(_ptr(data), _ptr(scales))


def version() -> str:
    return load().mm_version().decode()


def workspace_bytes(ds: LayerDesc, T: int, which: int = MM_WS_MAX) -> int:
    return load().mm_workspace_bytes(ctypes.byref(ds), T, which)


def prepacked_bytes(rows: int, cols: int) -> int:
    return load().mm_prepacked_bytes(rows, cols)


def prepacked_scale_bytes(rows: int, cols: int) -> int:
    return load().mm_prepacked_scale_bytes(rows, cols)


def quantize_int4g32(rows, cols, w, q, scales, stream=None):
    _check(load().mm_quantize_int4g32(rows, cols, _ptr(w), _ptr(q), _ptr(scales), _stream(stream)),
           "mm_quantize_int4g32")


def prepack_int4g32(n_mat, rows, cols, q_canon, s_canon, q_out, s_out, stream=None):
    _check(load().mm_prepack_int4g32(n_mat, rows, cols, _ptr(q_canon), _ptr(s_canon), _ptr(q_out),
                                     _ptr(s_out), _stream(stream)), "mm_prepack_int4g32")


def convert_bf16(n, x, y, stream=None):
    _check(load().mm_convert_bf16(n, _ptr(x), _ptr(y), _stream(stream)), "mm_convert_bf16")


def router_topk(ds, T, x, w_router, bias, topk_idx, topk_w, stream=None):
    _check(load().mm_router_topk(ctypes.byref(ds), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                 _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "mm_router_topk")


def route_permute(ds, T, topk_idx, offsets, perm, inv_perm, ws, ws_bytes, stream=None):
    _check(load().mm_route_permute(ctypes.byref(ds), T, _ptr(topk_idx), _ptr(offsets), _ptr(perm),
                                   _ptr(inv_perm), _ptr(ws), ws_bytes, _stream(stream)),
           "mm_route_permute")


def act_quant_i8(rows, cols, x, q, scale, stream=None):
    _check(load().mm_act_quant_i8(rows, cols, _ptr(x), _ptr(q), _ptr(scale), _stream(stream)),
           "mm_act_quant_i8")


def act_quant_i8_layout(rows, cols, x, q, scale, layout, stream=None):
    _check(load().mm_act_quant_i8_layout(rows, cols, _ptr(x), _ptr(q), _ptr(scale), layout,
                                         _stream(stream)), "mm_act_quant_i8_layout")


def expert_gateup_pair_f32(ds, T, xq, sx, perm, offsets, w_gu, ws_gu, h_r, h_s, stream=None,
                           isum_r=None, isum_s=None):
    lib = load()
    if isum_r is None:
        _check(lib.mm_expert_gateup_pair_f32(ctypes.byref(ds), T, _ptr(xq), _ptr(sx), _ptr(perm),
                                             _ptr(offsets), w_gu, ws_gu, _ptr(h_r), _ptr(h_s),
                                             _stream(stream)), "mm_expert_gateup_pair_f32")
    else:
        _check(lib.mm_expert_gateup_pair_f32_dbg(ctypes.byref(ds), T, _ptr(xq), _ptr(sx),
                                                 _ptr(perm), _ptr(offsets), w_gu, ws_gu, _ptr(h_r),
                                                 _ptr(h_s), _ptr(isum_r), _ptr(isum_s),
                                                 _stream(stream)), "mm_expert_gateup_pair_f32_dbg")


def expert_down_pair_f32(ds, T, hq_r, hs_r, hq_s, hs_s, offsets, w_d, ws_d, f, ys, stream=None,
                         isum_r=None, isum_s=None):
    lib = load()
    if isum_r is None:
        _check(lib.mm_expert_down_pair_f32(ctypes.byref(ds), T, _ptr(hq_r), _ptr(hs_r), _ptr(hq_s),
                                           _ptr(hs_s), _ptr(offsets), w_d, ws_d, _ptr(f), _ptr(ys),
                                           _stream(stream)), "mm_expert_down_pair_f32")
    else:
        _check(lib.mm_expert_down_pair_f32_dbg(ctypes.byref(ds), T, _ptr(hq_r), _ptr(hs_r),
                                               _ptr(hq_s), _ptr(hs_s), _ptr(offsets), w_d, ws_d,
                                               _ptr(f), _ptr(ys), _ptr(isum_r), _ptr(isum_s),
                                               _stream(stream)), "mm_expert_down_pair_f32_dbg")


def expert_gateup_swiglu(ds, T, act, act_scale, perm, offsets, w, h, h_scale, ws, ws_bytes,
                         stream=None, isum=None):
    lib = load()
    if isum is None:
        rc = lib.mm_expert_gateup_swiglu(ctypes.byref(ds), T, _ptr(act), _ptr(act_scale), _ptr(perm),
                                         _ptr(offsets), w, _ptr(h), _ptr(h_scale), _ptr(ws), ws_bytes,
                                         _stream(stream))
        _check(rc, "mm_expert_gateup_swiglu")
    else:
        rc = lib.mm_expert_gateup_swiglu_dbg(ctypes.byref(ds), T, _ptr(act), _ptr(act_scale),
                                             _ptr(perm), _ptr(offsets), w, _ptr(h), _ptr(h_scale),
                                             _ptr(ws), ws_bytes, _ptr(isum), _stream(stream))
        _check(rc, "mm_expert_gateup_swiglu_dbg")


def expert_down(ds, T, h, h_scale, offsets, w, f, ws, ws_bytes, stream=None, isum=None):
    lib = load()
    if isum is None:
        _check(lib.mm_expert_down(ctypes.byref(ds), T, _ptr(h), _ptr(h_scale), _ptr(offsets), w,
                                  _ptr(f), _ptr(ws), ws_bytes, _stream(stream)), "mm_expert_down")
    else:
        _check(lib.mm_expert_down_dbg(ctypes.byref(ds), T, _ptr(h), _ptr(h_scale), _ptr(offsets), w,
                                      _ptr(f), _ptr(ws), ws_bytes, _ptr(isum), _stream(stream)),
               "mm_expert_down_dbg")


def shared_expert(ds, T, act, act_scale, w_gateup, w_down, ys, ws, ws_bytes, stream=None):
    _check(load().mm_shared_expert(ctypes.byref(ds), T, _ptr(act), _ptr(act_scale), w_gateup, w_down,
                                   _ptr(ys), _ptr(ws), ws_bytes, _stream(stream)), "mm_shared_expert")


def combine(ds, T, f, inv_perm, topk_w, ys, y, stream=None):
    _check(load().mm_combine(ctypes.byref(ds), T, _ptr(f), _ptr(inv_perm), _ptr(topk_w), _ptr(ys),
                             _ptr(y), _stream(stream)), "mm_combine")


def moe_forward(ds, T, x, w_router, bias, w_gu, w_d, ws_gu, ws_d, topk_idx, topk_w, y, ws,
                ws_bytes, stream=None, y_norm=None, norm_eps=0.0):
    """The whole layer in one call (routed + shared experts, combine); with
    y_norm also RMSNorm(y) for the next layer of a stack."""
    _check(load().mm_moe_forward(ctypes.byref(ds), T, _ptr(x), _ptr(w_router), _ptr(bias), w_gu,
                                 w_d, ws_gu, ws_d, _ptr(topk_idx), _ptr(topk_w), _ptr(y),
                                 _ptr(y_norm), norm_eps, _ptr(ws), ws_bytes, _stream(stream)),
           "mm_moe_forward")


def moe_decode(ds, T, x, w_router, bias, w_gu, w_d, ws_gu, ws_d, topk_idx, topk_w, y, ws,
               ws_bytes, stream=None, y_norm=None, norm_eps=0.0):
    """moe_forward for 1..4 tokens as one kernel launch.  ws
    (workspace_bytes(ds, T, MM_WS_DECODE)) holds state between calls: zero it
    once before the first call; calls sharing it must not overlap."""
    _check(load().mm_moe_decode(ctypes.byref(ds), T, _ptr(x), _ptr(w_router), _ptr(bias), w_gu,
                                w_d, ws_gu, ws_d, _ptr(topk_idx), _ptr(topk_w), _ptr(y),
                                _ptr(y_norm), norm_eps, _ptr(ws), ws_bytes, _stream(stream)),
           "mm_moe_decode")


def moe_decode_noalloc(ds, T, x, w_router, bias, w_gu, w_d, ws_gu, ws_d, topk_idx, topk_w, y,
                       stream=None, y_norm=None, norm_eps=0.0):
    """moe_decode without a workspace: the library's fixed device scratch
    (one per GPU, shared by every call on it; calls must not overlap)."""
    _check(load().mm_moe_decode_noalloc(ctypes.byref(ds), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                        w_gu, w_d, ws_gu, ws_d, _ptr(topk_idx), _ptr(topk_w),
                                        _ptr(y), _ptr(y_norm), norm_eps, _stream(stream)),
           "mm_moe_decode_noalloc")


def moe_decode_supported(ds, T) -> bool:
    return bool(load().mm_moe_decode_supported(ctypes.byref(ds), T))


def set_profile_events(start=None, stop=None):
    """Events (torch.cuda.Event, created with enable_timing=True, or None)
    that mm_moe_forward records around its gate/up product stage; None, None
    switches the hook off."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:  # torch creates the event on its first record
            ev.record()
        return ev.cuda_event
    _check(load().mm_set_profile_events(handle(start), handle(stop)), "mm_set_profile_events")


def linear_w4a8(rows, in_features, out_features, xq, sx, w, y, stream=None):
    """y [rows, out] FP32 = W4A8 product of x_q [rows, in] (scales sx) and the
    prepacked INT4 weight w (a Weight) [out, in]."""
    _check(load().mm_linear_w4a8(rows, in_features, out_features, _ptr(xq), _ptr(sx), w, _ptr(y),
                                 _stream(stream)), "mm_linear_w4a8")


def attn_workspace_bytes(B, n_kv, max_len) -> int:
    return int(load().mm_attn_workspace_bytes(B, n_kv, max_len))


def kv_append_i8(B, n_kv, d_h, max_T, pos, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                 stream=None):
    _check(load().mm_kv_append_i8(B, n_kv, d_h, max_T, _ptr(pos), _ptr(k_new), _ptr(v_new),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                  _stream(stream)), "mm_kv_append_i8")


def attn_decode_i8(B, n_h, n_kv, d_h, max_T, max_len, lens, q, k_cache, v_cache, k_scale, v_scale,
                   out, ws, ws_bytes, stream=None):
    _check(load().mm_attn_decode_i8(B, n_h, n_kv, d_h, max_T, max_len, _ptr(lens), _ptr(q),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "mm_attn_decode_i8")


def bias_update(T, E, k, topk_idx, lam, bias, load_out=None, stream=None):
    _check(load().mm_bias_update(T, E, k, _ptr(topk_idx), lam, _ptr(bias), _ptr(load_out),
                                     _stream(stream)), "mm_bias_update")


def drop_pad_capacity(T, k, E, num=3, den=2) -> int:
    return int(load().mm_drop_pad_capacity(T, k, E, num, den))


def drop_pad(T, E, k, capacity, topk_idx, offsets, perm, inv_perm, buf, offsets_c, perm_c, inv_c,
             stream=None):
    _check(load().mm_drop_pad(T, E, k, capacity, _ptr(topk_idx), _ptr(offsets), _ptr(perm),
                                  _ptr(inv_perm), _ptr(buf), _ptr(offsets_c), _ptr(perm_c),
                                  _ptr(inv_c), _stream(stream)), "mm_drop_pad")


def fake_quant(rows, cols, bits, group, x, x_bar=None, grad_out=None, grad_in=None, stream=None):
    _check(load().mm_fake_quant(rows, cols, bits, group, _ptr(x), _ptr(x_bar), _ptr(grad_out),
                                    _ptr(grad_in), _stream(stream)), "mm_fake_quant")


def gather_rows(R, d, k, perm, scale, src, dst, stream=None):
    _check(load().mm_gather_rows(R, d, k, _ptr(perm), _ptr(scale), _ptr(src), _ptr(dst),
                                 _stream(stream)), "mm_gather_rows")


def expert_train_forward_f32(E, d, h, R, offsets, xs, w_gu, w_d, gu, a_bar, f, stream=None):
    _check(load().mm_expert_train_forward_f32(E, d, h, R, _ptr(offsets), _ptr(xs), _ptr(w_gu),
                                              _ptr(w_d), _ptr(gu), _ptr(a_bar), _ptr(f),
                                              _stream(stream)), "mm_expert_train_forward_f32")


def expert_backward_workspace_bytes(R, h) -> int:
    return int(load().mm_expert_backward_workspace_bytes(R, h))


def expert_backward_f32(E, d, h, R, offsets, xs, w_gu, w_d, gu, a_bar, df, dxs, dw_gu, dw_d, ws,
                        ws_bytes, stream=None):
    _check(load().mm_expert_backward_f32(E, d, h, R, _ptr(offsets), _ptr(xs), _ptr(w_gu), _ptr(w_d),
                                         _ptr(gu), _ptr(a_bar), _ptr(df), _ptr(dxs), _ptr(dw_gu),
                                         _ptr(dw_d), _ptr(ws), ws_bytes, _stream(stream)),
           "mm_expert_backward_f32")


def router_backward_f32(ds, T, x, w_router, bias, topk_idx, f, inv, dy, lambda_z, dz, dw_router, dx,
                        stream=None):
    _check(load().mm_router_backward_f32(ctypes.byref(ds), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                         _ptr(topk_idx), _ptr(f), _ptr(inv), _ptr(dy), lambda_z,
                                         _ptr(dz), _ptr(dw_router), _ptr(dx), _stream(stream)),
           "mm_router_backward_f32")


def rmsnorm_f32(rows, cols, eps, x, y, stream=None):
    _check(load().mm_rmsnorm_f32(rows, cols, eps, _ptr(x), _ptr(y), _stream(stream)),
           "mm_rmsnorm_f32")


def add_rmsnorm_f32(rows, cols, eps, x, r, out_sum, out_norm=None, stream=None):
    _check(load().mm_add_rmsnorm_f32(rows, cols, eps, _ptr(x), _ptr(r), _ptr(out_sum),
                                     _ptr(out_norm), _stream(stream)), "mm_add_rmsnorm_f32")


MM_KV_CODES, MM_KV_SCALES = 0, 1


def kv_cache_bytes(B, n_kv, d_h, max_T, which) -> int:
    return int(load().mm_kv_cache_bytes(B, n_kv, d_h, max_T, which))
