"""CPU oracle for the MobileMoE MoE-FFN layer (eq. (*) of the MobileMoE close
reading, paper-archivist.com).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports this
package and this package never imports the HIP library; they share no code.

The arithmetic lives in ``mobmoe_oracle.cpp`` (plain C++, no fast-math, FMAs
written out); this module builds it with g++ and wraps it with ctypes/numpy.
Every wrapper names the oracle function it calls; the passage each follows is
cited in the C++ source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mobmoe_oracle.cpp")
_LIB = os.path.join(_HERE, "libmobmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library with g++ (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    """Loads the oracle library (MOBMOE_ORACLE_LIB names another build of the
    same source, e.g. the sanitizer build of tests/test_sanitizers.py)."""
    global _lib
    if _lib is None:
        other = os.environ.get("MOBMOE_ORACLE_LIB")
        if other:
            _lib = ctypes.CDLL(other)
            _lib.ora_version.restype = ctypes.c_char_p
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _lib.ora_version.restype = ctypes.c_char_p
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i8(a):
    return np.ascontiguousarray(a, dtype=np.int8)


def _i64(v):
    return ctypes.c_int64(int(v))


def version() -> str:
    return _load().ora_version().decode()


def quant_w4g32(w: np.ndarray):
    """eq. (6), b=4, group 32 -> (q int8 [rows, cols], s float32 [rows, cols/32])."""
    w = _f32(w)
    rows, cols = w.reshape(-1, w.shape[-1]).shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, cols // 32), np.float32)
    rc = _load().ora_quant_w4g32(_i64(rows), _i64(cols), _p(w), _p(q), _p(s))
    if rc:
        raise ValueError("ora_quant_w4g32: cols must be a multiple of 32")
    return q.reshape(w.shape), s.reshape(w.shape[:-1] + (cols // 32,))


def quant_act_i8(x: np.ndarray):
    """Per-row INT8 (eq. (6) with b=8, one group per row) -> (q int8, s float32 [rows])."""
    x = _f32(x)
    rows, cols = x.reshape(-1, x.shape[-1]).shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.float32)
    _load().ora_quant_act_i8(_i64(rows), _i64(cols), _p(x), _p(q), _p(s))
    return q.reshape(x.shape), s.reshape(x.shape[:-1])


def router(x, wr, bias, k: int, gating: int = 0):
    """FP32 router -> (idx int32 [T,k], w float64 [T,k], logits float32 [T,E]).
    gating: 0 softmax, 1 sigmoid renormalised over the k; plus 2: the bias
    takes part in the selection only (logits then holds logit + bias)."""
    x, wr = _f32(x), _f32(wr)
    T, d = x.shape
    E = wr.shape[0]
    b = None if bias is None else _f32(bias)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib = _load()
    sel_only = (gating >> 1) & 1
    if gating & 1 == 0:
        logits = np.empty((T, E), np.float32)
        rc = lib.ora_router(_i64(T), d, E, k, _p(x), _p(wr), _p(b), _p(logits), _p(idx), _p(w),
                            sel_only)
    else:
        logits = None
        rc = lib.ora_router_sigmoid(_i64(T), d, E, k, _p(x), _p(wr), _p(b), _p(idx), _p(w),
                                    sel_only)
    if rc:
        raise ValueError("ora_router: bad shapes")
    return idx, w, logits


def route(idx: np.ndarray, E: int):
    """Stable count sort -> (offsets [E+1], perm [T*k], inv_perm [T*k]) int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    rc = _load().ora_route(_i64(T), E, k, _p(idx), _p(offsets), _p(perm), _p(inv))
    if rc:
        raise ValueError("ora_route: expert id out of range")
    return offsets, perm, inv


def linear_w4a8(aq, sa, wq, ws, want_isum: bool = False):
    """out[r,o] = sa[r] * (fma chain over g of ws[o,g] * isum[r,o,g]) in FP32; isum optional."""
    aq, wq = _i8(aq), _i8(wq)
    sa, ws = _f32(sa), _f32(ws)
    rows, K = aq.shape
    N = wq.shape[0]
    out = np.empty((rows, N), np.float32)
    isum = np.empty((rows, N, K // 32), np.int32) if want_isum else None
    _load().ora_linear_w4a8(_i64(rows), N, K, _p(aq), _p(sa), _p(wq), _p(ws), _p(out), _p(isum))
    return (out, isum) if want_isum else out


def ffn_w4a8(xq, sx, wgu_q, wgu_s, wd_q, wd_s, want_isum: bool = False, want_a: bool = False):
    """SwiGLU expert on INT8 rows -> (hq, hs, f[, isum_gu, isum_d][, a]); a is
    the FP32 hidden row SiLU(g) * u before its re-quantisation."""
    xq, wgu_q, wd_q = _i8(xq), _i8(wgu_q), _i8(wd_q)
    sx, wgu_s, wd_s = _f32(sx), _f32(wgu_s), _f32(wd_s)
    rows, d = xq.shape
    h = wd_q.shape[1]
    hq = np.empty((rows, h), np.int8)
    hs = np.empty((rows,), np.float32)
    f = np.empty((rows, d), np.float32)
    igu = np.empty((rows, 2 * h, d // 32), np.int32) if want_isum else None
    idn = np.empty((rows, d, h // 32), np.int32) if want_isum else None
    a = np.empty((rows, h), np.float32) if want_a else None
    _load().ora_ffn_w4a8(_i64(rows), d, h, _p(xq), _p(sx), _p(wgu_q), _p(wgu_s), _p(wd_q),
                         _p(wd_s), _p(hq), _p(hs), _p(f), _p(igu), _p(idn), _p(a))
    out = (hq, hs, f) + ((igu, idn) if want_isum else ())
    return out + (a,) if want_a else out


def ffn_float(x, wgu, wd, bf16: bool = False):
    x, wgu, wd = _f32(x), _f32(wgu), _f32(wd)
    rows, d = x.shape
    h = wd.shape[1]
    f = np.empty((rows, d), np.float64)
    _load().ora_ffn_float(_i64(rows), d, h, _p(x), _p(wgu), _p(wd), 1 if bf16 else 0, _p(f))
    return f


def combine(f, w, ys):
    """f [T,k,d], w [T,k], ys [T,d] or None (all float64) -> y [T,d] float64."""
    f = np.ascontiguousarray(f, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    ys = None if ys is None else np.ascontiguousarray(ys, dtype=np.float64)
    T, k, d = f.shape
    y = np.empty((T, d), np.float64)
    _load().ora_combine(_i64(T), k, d, _p(f), _p(w), _p(ys), _p(y))
    return y


def combine_f32(f, w, ys):
    """FP32 combine of the INT4 path: fma chain over slots, then + ys."""
    f = _f32(f)
    w = _f32(w)
    ys = None if ys is None else _f32(ys)
    T, k, d = f.shape
    y = np.empty((T, d), np.float32)
    _load().ora_combine_f32(_i64(T), k, d, _p(f), _p(w), _p(ys), _p(y))
    return y


def attn_decode(q, kq, vq, ks, vs, T: int):
    """GQA attention of one token per sequence over an INT8 KV cache, double.
    q [B, n_h, d_h]; kq / vq int8 [B, n_kv, max_T, d_h]; ks / vs [B, n_kv, max_T];
    positions 0..T-1 of the cache are used.  Returns out [B, n_h, d_h] float64."""
    q, ks, vs = _f32(q), _f32(ks), _f32(vs)
    kq, vq = _i8(kq), _i8(vq)
    B, nh, dh = q.shape
    nkv, maxT = kq.shape[1], kq.shape[2]
    out = np.empty((B, nh, dh), np.float64)
    rc = _load().ora_attn_decode(_i64(B), nh, nkv, dh, _i64(T), _i64(maxT), _p(q), _p(kq), _p(vq),
                                 _p(ks), _p(vs), _p(out))
    if rc:
        raise ValueError("ora_attn_decode: bad shapes")
    return out


def exp_ref(x):
    """The FP32 exponential the INT4 path uses (Cody-Waite + Taylor)."""
    x = _f32(x)
    y = np.empty_like(x)
    _load().ora_exp_ref(_i64(x.size), _p(x), _p(y))
    return y


def rmsnorm(x, eps: float = 1e-5):
    x = _f32(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float64)
    _load().ora_rmsnorm(_i64(rows), cols, ctypes.c_double(eps), _p(x), _p(y))
    return y


def round_bf16(x):
    x = _f32(x)
    y = np.empty_like(x)
    _load().ora_round_bf16(_i64(x.size), _p(x), _p(y))
    return y


class _Out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("y", "idx", "w", "logits", "xq", "sx", "hq", "hs", "f", "ys", "hq_s", "hs_s")]


@dataclass
class LayerResult:
    y: np.ndarray
    idx: np.ndarray
    w: np.ndarray
    logits: Optional[np.ndarray]
    f: np.ndarray
    ys: Optional[np.ndarray]
    xq: Optional[np.ndarray] = None
    sx: Optional[np.ndarray] = None
    hq: Optional[np.ndarray] = None
    hs: Optional[np.ndarray] = None
    hq_s: Optional[np.ndarray] = None
    hs_s: Optional[np.ndarray] = None


WFMT = {"f32": 0, "int4g32": 1, "bf16": 2}


def forward(x, wr, bias, w_gu, w_d, ws_gu, ws_d, *, k: int, wfmt: str = "int4g32",
            gating: int = 0, nthreads: int = 1) -> LayerResult:
    """Whole layer, eq. (*), with every intermediate returned.

    x [T,d]; wr [E,d]; bias [E] or None; w_gu [E,2h,d]; w_d [E,d,h];
    ws_gu [2hs,d] / ws_d [d,hs] or None for no shared expert.
    """
    x, wr, w_gu, w_d = _f32(x), _f32(wr), _f32(w_gu), _f32(w_d)
    b = None if bias is None else _f32(bias)
    T, d = x.shape
    E, h2, _ = w_gu.shape
    h = h2 // 2
    hs = 0 if ws_gu is None else ws_gu.shape[0] // 2
    ws_gu = None if ws_gu is None else _f32(ws_gu)
    ws_d = None if ws_d is None else _f32(ws_d)
    fm = WFMT[wfmt]
    r = LayerResult(
        y=np.empty((T, d), np.float64), idx=np.empty((T, k), np.int32),
        w=np.empty((T, k), np.float64),
        logits=np.empty((T, E), np.float32) if gating & 1 == 0 else None,
        f=np.empty((T, k, d), np.float64), ys=np.empty((T, d), np.float64) if hs else None)
    if fm == 1:
        r.xq, r.sx = np.empty((T, d), np.int8), np.empty((T,), np.float32)
        r.hq, r.hs = np.empty((T, k, h), np.int8), np.empty((T, k), np.float32)
        if hs:
            r.hq_s, r.hs_s = np.empty((T, hs), np.int8), np.empty((T,), np.float32)
    o = _Out(*[None if a is None else a.ctypes.data for a in
               (r.y, r.idx, r.w, r.logits, r.xq, r.sx, r.hq, r.hs, r.f, r.ys, r.hq_s, r.hs_s)])
    rc = _load().ora_forward(d, E, h, hs, k, fm, gating, _i64(T), _p(x), _p(wr), _p(b),
                             _p(w_gu), _p(w_d), _p(ws_gu), _p(ws_d), int(nthreads),
                             ctypes.byref(o))
    if rc:
        raise ValueError("ora_forward: bad shapes or formats")
    return r


def bias_update(idx, bias, E: int, lam: float = 1e-3):
    """Aux-loss-free balancing step -> (new bias float32 [E], load int32 [E])."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    b = np.array(bias, np.float32, copy=True)
    load = np.empty((E,), np.int32)
    rc = _load().ora_bias_update(_i64(T), E, k, _p(idx), ctypes.c_float(lam), _p(b), _p(load))
    if rc:
        raise ValueError("ora_bias_update: expert id out of range")
    return b, load


def capacity(T: int, k: int, E: int, num: int = 3, den: int = 2) -> int:
    """Per-expert buffer rows of drop-and-pad: ceil((num/den) * T*k / E), exact."""
    return -(-(T * k * num) // (E * den))


def drop_pad(idx, E: int, C: int):
    """Drop-and-pad dispatch -> (buf [E, C], offsets_c [E+1], perm_c [T*k], inv_c [T*k]) int32."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    buf = np.empty((E, C), np.int32)
    offs = np.empty((E + 1,), np.int32)
    perm = np.empty((T * k,), np.int32)
    inv = np.empty((T * k,), np.int32)
    rc = _load().ora_drop_pad(_i64(T), E, k, _i64(C), _p(idx), _p(buf), _p(offs), _p(perm), _p(inv))
    if rc:
        raise ValueError("ora_drop_pad: bad ids or capacity")
    return buf, offs, perm, inv


def fake_quant(x, bits: int, group: int, gout=None):
    """QAT fake quantisation (eq. (6)) -> xbar, or (xbar, gin) when gout is given."""
    x = _f32(x)
    rows, cols = x.reshape(-1, x.shape[-1]).shape
    xbar = np.empty_like(x)
    g = None if gout is None else _f32(gout)
    gin = None if gout is None else np.empty_like(x)
    rc = _load().ora_fake_quant(_i64(rows), _i64(cols), bits, _i64(group), _p(x), _p(xbar), _p(g),
                                _p(gin))
    if rc:
        raise ValueError("ora_fake_quant: bad bits or group")
    return xbar if gout is None else (xbar, gin)


def expert_train_forward(offsets, xs, wgu, wd):
    """QAT forward of the routed experts over expert-ordered rows ->
    (gu [R, 2h], abar [R, h], f [R, d]) float32."""
    offsets = np.ascontiguousarray(offsets, np.int32)
    xs, wgu, wd = _f32(xs), _f32(wgu), _f32(wd)
    E, h2, d = wgu.shape
    h = h2 // 2
    R = xs.shape[0]
    gu = np.empty((R, 2 * h), np.float32)
    abar = np.empty((R, h), np.float32)
    f = np.empty((R, d), np.float32)
    _load().ora_expert_train_forward(E, d, h, _p(offsets), _p(xs), _p(wgu), _p(wd), _p(gu), _p(abar),
                                     _p(f))
    return gu, abar, f


def expert_backward(offsets, xs, wgu, wd, gu, df):
    """Backward of expert_train_forward -> (dxs [R, d], dwgu [E, 2h, d], dwd [E, d, h]) float64."""
    offsets = np.ascontiguousarray(offsets, np.int32)
    xs, wgu, wd, gu, df = _f32(xs), _f32(wgu), _f32(wd), _f32(gu), _f32(df)
    E, h2, d = wgu.shape
    h = h2 // 2
    R = xs.shape[0]
    dxs = np.empty((R, d), np.float64)
    dwgu = np.empty((E, 2 * h, d), np.float64)
    dwd = np.empty((E, d, h), np.float64)
    _load().ora_expert_backward(E, d, h, _p(offsets), _p(xs), _p(wgu), _p(wd), _p(gu), _p(df),
                                _p(dxs), _p(dwgu), _p(dwd))
    return dxs, dwgu, dwd


def router_backward(x, wr, bias, idx, f, inv, dy, gating: int = 0, lambda_z: float = 1e-4, dx=None):
    """Router backward of the training step -> (dz [T, E], dwr [E, d], dx [T, d]) float64;
    dx accumulates onto the given array (zeros if None)."""
    x, wr, f, dy = _f32(x), _f32(wr), _f32(f), _f32(dy)
    b = None if bias is None else _f32(bias)
    idx = np.ascontiguousarray(idx, np.int32)
    inv = np.ascontiguousarray(inv, np.int32)
    T, d = x.shape
    E = wr.shape[0]
    k = idx.shape[1]
    dz = np.empty((T, E), np.float64)
    dwr = np.empty((E, d), np.float64)
    dxo = np.zeros((T, d), np.float64) if dx is None else np.array(dx, np.float64, copy=True)
    _load().ora_router_backward(_i64(T), d, E, k, gating, _p(x), _p(wr), _p(b), _p(idx), _p(f), _p(inv),
                                _p(dy), ctypes.c_double(lambda_z), _p(dz), _p(dwr), _p(dxo))
    return dz, dwr, dxo
