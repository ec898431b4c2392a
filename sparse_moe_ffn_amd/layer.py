"""A MoE-FFN layer object on top of the C ABI: owns the device weights and the
per-call buffers, and issues the seven calls on the current stream (the
shared expert, which depends only on the quantised input, on a second stream
joined before the combine).

Weight preparation runs on the device through the library (eq. (6)
quantisation with mm_quantize_int4g32, then mm_prepack_int4g32; or BF16
conversion).  torch is used only to allocate device memory and to provide the
stream.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _empty(shape, dtype, device) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=device)


@dataclass
class DevWeight:
    data: torch.Tensor
    scales: Optional[torch.Tensor]
    canon: Optional[torch.Tensor] = None        # INT4 canonical nibbles (kept for tests)
    canon_scales: Optional[torch.Tensor] = None

    def c(self) -> B.Weight:
        return B.weight(self.data, self.scales)


def prepare_weight(w: np.ndarray, wfmt: str, device, keep_canonical: bool = False) -> DevWeight:
    """w: FP32 [n_mat, rows, cols] (or [rows, cols]) -> device weight in `wfmt`."""
    a = w if w.ndim == 3 else w[None]
    n, rows, cols = a.shape
    src = _dev(a.astype(np.float32, copy=False), device)
    if wfmt == "f32":
        return DevWeight(src, None)
    if wfmt == "bf16":
        out = _empty((n, rows, cols), torch.int16, device)
        B.convert_bf16(src.numel(), src, out)
        return DevWeight(out, None)
    qc = _empty((n * rows, cols // 2), torch.uint8, device)
    sc = _empty((n * rows, cols // 32), torch.float32, device)
    B.quantize_int4g32(n * rows, cols, src, qc, sc)
    qp = _empty((n * B.prepacked_bytes(rows, cols),), torch.uint8, device)
    sp = _empty((n * B.prepacked_scale_bytes(rows, cols) // 4,), torch.float32, device)
    B.prepack_int4g32(n, rows, cols, qc, sc, qp, sp)
    del src
    if keep_canonical:
        return DevWeight(qp, sp, qc, sc)
    return DevWeight(qp, sp)


class MoELayer:
    """One MoE-FFN layer (eq. (*)) with device-resident weights."""

    def __init__(self, d, E, h, hs, k, wr, bias, w_gu, w_d, ws_gu=None, ws_d=None, *,
                 wfmt="int4g32", gating=0, out_dtype=B.MM_OUT_F32, device="cuda",
                 keep_canonical=False, overlap_shared=True):
        self.d, self.E, self.h, self.hs, self.k = d, E, h, hs, k
        self.wfmt = wfmt
        self.device = torch.device(device)
        self.desc = B.desc(d, E, h, hs, k, wfmt, gating, out_dtype)
        self.wr = _dev(wr.astype(np.float32), self.device)
        self.bias = None if bias is None else _dev(bias.astype(np.float32), self.device)
        self.w_gu = prepare_weight(w_gu, wfmt, self.device, keep_canonical)
        self.w_d = prepare_weight(w_d, wfmt, self.device, keep_canonical)
        self.ws_gu = prepare_weight(ws_gu, wfmt, self.device, keep_canonical) if hs else None
        self.ws_d = prepare_weight(ws_d, wfmt, self.device, keep_canonical) if hs else None
        self._T = -1
        # The shared expert depends only on the (quantised) input, so it can run
        # on a second stream (default priority) beside the routed experts.
        self.overlap_shared = overlap_shared and bool(hs)
        self.side = torch.cuda.Stream(device=self.device) if self.overlap_shared else None
        self._xq_ready = torch.cuda.Event() if self.overlap_shared else None

    @classmethod
    def from_workload(cls, w, lw, device="cuda", **kw):
        return cls(w.d, w.E, w.h, w.hs, w.k, lw.wr, lw.bias, lw.w_gu, lw.w_d, lw.ws_gu, lw.ws_d,
                   wfmt=w.wfmt, device=device,
                   out_dtype=B.MM_OUT_BF16 if w.wfmt == "bf16" else B.MM_OUT_F32, **kw)

    def buffers(self, T: int):
        """(Re)allocates the per-call buffers for T tokens."""
        if T == self._T:
            return
        dv, k, d, h = self.device, self.k, self.d, self.h
        self.idx = _empty((T, k), torch.int32, dv)
        self.topw = _empty((T, k), torch.float32, dv)
        self.offsets = _empty((self.E + 1,), torch.int32, dv)
        self.perm = _empty((T * k,), torch.int32, dv)
        self.inv = _empty((T * k,), torch.int32, dv)
        if self.wfmt == "int4g32":
            self.xq = _empty((T, d), torch.int8, dv)
            self.sx = _empty((T,), torch.float32, dv)
            self.hbuf = _empty((T * k, h), torch.int8, dv)
            self.hscale = _empty((T * k,), torch.float32, dv)
        else:
            self.xq, self.sx, self.hscale = None, None, None
            self.hbuf = _empty((T * k, h), torch.float32 if self.wfmt == "f32" else torch.int16, dv)
        self.f = _empty((T * k, d), torch.float32, dv)
        self.ys = _empty((T, d), torch.float32, dv) if self.hs else None
        self.y = _empty((T, d), torch.float32 if self.desc.out_dtype == B.MM_OUT_F32 else torch.int16, dv)
        # One workspace per call that needs one (the shared expert runs
        # concurrently with the routed calls on a second stream).
        self.wk_route_bytes = max(B.workspace_bytes(self.desc, T, B.MM_WS_ROUTE), 256)
        self.wk_route = _empty((self.wk_route_bytes,), torch.uint8, dv)
        self.wk_gu_bytes = max(B.workspace_bytes(self.desc, T, B.MM_WS_GATEUP), 256)
        self.wk_gu = _empty((self.wk_gu_bytes,), torch.uint8, dv)
        self.wk_dn_bytes = max(B.workspace_bytes(self.desc, T, B.MM_WS_DOWN), 256)
        self.wk_dn = _empty((self.wk_dn_bytes,), torch.uint8, dv)
        self.wk_fwd_bytes = max(B.workspace_bytes(self.desc, T, B.MM_WS_FORWARD), 256)
        self.wk_fwd = _empty((self.wk_fwd_bytes,), torch.uint8, dv)
        self.wk_sh_bytes = max(B.workspace_bytes(self.desc, T, B.MM_WS_SHARED), 256)
        self.wk_sh = _empty((self.wk_sh_bytes,), torch.uint8, dv)
        self._T = T

    # The seven calls, in order.  Each uses the current torch stream.
    def router(self, x, T):
        B.router_topk(self.desc, T, x, self.wr, self.bias, self.idx, self.topw)

    def route(self, T):
        B.route_permute(self.desc, T, self.idx, self.offsets, self.perm, self.inv, self.wk_route,
                        self.wk_route_bytes)

    def act_quant(self, x, T):
        B.act_quant_i8(T, self.d, x, self.xq, self.sx)

    def act(self, x):
        return (self.xq, self.sx) if self.wfmt == "int4g32" else (x, None)

    def gateup(self, x, T, isum=None):
        a, s = self.act(x)
        B.expert_gateup_swiglu(self.desc, T, a, s, self.perm, self.offsets, self.w_gu.c(), self.hbuf,
                               self.hscale, self.wk_gu, self.wk_gu_bytes, isum=isum)

    def gateup_f32(self, x, T, out):
        """Routed gate/up + SwiGLU without the re-quantisation: FP32 hidden
        rows [T*k, h] (sorted order) into `out` (INT4 weights only).  The
        matrix-core / weight-streaming kernel of gateup() on its own."""
        a, s = self.act(x)
        B.expert_gateup_swiglu(self.desc, T, a, s, self.perm, self.offsets, self.w_gu.c(), out,
                               None, None, 0)

    def gateup_pair_f32(self, T, xq16, h_r, h_s, isum_r=None, isum_s=None):
        """Routed and shared gate/up + SwiGLU in one launch, FP32 hidden rows
        into h_r [T*k, h] (sorted order) and h_s [T, h_s], from x_q as f16
        paired codes (with this layer's scales self.sx): the merged
        matrix-core kernel mm_moe_forward runs for larger batches, on its own
        (INT4 weights, shared expert).  isum_r / isum_s: also the exact group
        sums."""
        B.expert_gateup_pair_f32(self.desc, T, xq16, self.sx, self.perm, self.offsets,
                                 self.w_gu.c(), self.ws_gu.c(), h_r, h_s, isum_r=isum_r,
                                 isum_s=isum_s)

    def down_pair_f32(self, T, hq_r, hs_r, hq_s, hs_s, f, ys, isum_r=None, isum_s=None):
        """Routed and shared down products in one launch from f16 paired
        hidden codes: f [T*k, d] (sorted order) and ys [T, d]."""
        B.expert_down_pair_f32(self.desc, T, hq_r, hs_r, hq_s, hs_s, self.offsets, self.w_d.c(),
                               self.ws_d.c(), f, ys, isum_r=isum_r, isum_s=isum_s)

    def down(self, T, isum=None):
        B.expert_down(self.desc, T, self.hbuf, self.hscale, self.offsets, self.w_d.c(), self.f,
                      self.wk_dn, self.wk_dn_bytes, isum=isum)

    def shared(self, x, T):
        a, s = self.act(x)
        B.shared_expert(self.desc, T, a, s, self.ws_gu.c(), self.ws_d.c(), self.ys, self.wk_sh,
                        self.wk_sh_bytes)

    def combine(self, T):
        B.combine(self.desc, T, self.f, self.inv, self.topw, self.ys, self.y)

    def capture(self, x: torch.Tensor, fused: bool = False) -> "torch.cuda.CUDAGraph":
        """Records forward(x) for the static input buffer x into a HIP graph;
        replaying it recomputes y from whatever x holds at replay time.  The
        library allocates nothing and records no memset, so the graph holds
        only kernel nodes (and the shared-expert stream fork/join)."""
        T = x.shape[0]
        self.buffers(T)
        fwd = self.forward_fused if fused else self.forward
        warm = torch.cuda.Stream(device=self.device)
        warm.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(warm):
            fwd(x)
        torch.cuda.current_stream(self.device).wait_stream(warm)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd(x)
        return g

    def forward_fused(self, x: torch.Tensor, y_norm: Optional[torch.Tensor] = None,
                      norm_eps: float = 1e-5) -> torch.Tensor:
        """y = eq. (*) of x through the one-call entry (mm_moe_forward): same
        results as forward(), fewer launches, one stream.  Also fills idx/topw,
        and y_norm = RMSNorm(y) when given (the next layer's input in a stack)."""
        T = x.shape[0]
        self.buffers(T)
        none = B.weight(None, None)
        B.moe_forward(self.desc, T, x, self.wr, self.bias, self.w_gu.c(), self.w_d.c(),
                      self.ws_gu.c() if self.hs else none, self.ws_d.c() if self.hs else none,
                      self.idx, self.topw, self.y, self.wk_fwd, self.wk_fwd_bytes,
                      y_norm=y_norm, norm_eps=norm_eps if y_norm is not None else 0.0)
        return self.y

    def decode_supported(self, T: int) -> bool:
        """True when forward_decode has a one-launch form for T tokens."""
        return B.moe_decode_supported(self.desc, T)

    def forward_decode(self, x: torch.Tensor, y_norm: Optional[torch.Tensor] = None,
                       norm_eps: float = 1e-5) -> torch.Tensor:
        """forward_fused for 1..4 tokens as ONE kernel launch (mm_moe_decode):
        bit-identical results.  The layer keeps the call's state buffer
        (zeroed once here, left zeroed by every call)."""
        T = x.shape[0]
        self.buffers(T)
        if getattr(self, "wk_dec", None) is None:
            self.wk_dec_bytes = max(B.workspace_bytes(self.desc, 4, B.MM_WS_DECODE), 256)
            self.wk_dec = torch.zeros((self.wk_dec_bytes,), dtype=torch.uint8, device=self.device)
        none = B.weight(None, None)
        B.moe_decode(self.desc, T, x, self.wr, self.bias, self.w_gu.c(), self.w_d.c(),
                     self.ws_gu.c() if self.hs else none, self.ws_d.c() if self.hs else none,
                     self.idx, self.topw, self.y, self.wk_dec, self.wk_dec_bytes,
                     y_norm=y_norm, norm_eps=norm_eps if y_norm is not None else 0.0)
        return self.y

    def decode_status(self) -> int:
        """Waits inside mm_moe_decode that gave up so far (0 when healthy)."""
        if getattr(self, "wk_dec", None) is None:
            return 0
        return int(self.wk_dec[16:20].view(torch.int32).item())

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """y = eq. (*) of x [T, d] FP32 (device).  Returns the layer's y buffer."""
        T = x.shape[0]
        self.buffers(T)
        main = torch.cuda.current_stream(self.device)
        int4 = self.wfmt == "int4g32"
        if self.overlap_shared and self.hs:
            # side stream: activation quantisation, then the shared expert;
            # main stream: router and routing meanwhile, then the routed experts
            # once the quantised activations exist
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                if int4:
                    self.act_quant(x, T)
                    self._xq_ready.record(self.side)
                self.shared(x, T)
            self.router(x, T)
            self.route(T)
            if int4:
                main.wait_event(self._xq_ready)
            self.gateup(x, T)
            self.down(T)
            main.wait_stream(self.side)
        else:
            if int4:
                self.act_quant(x, T)
            self.router(x, T)
            self.route(T)
            self.gateup(x, T)
            self.down(T)
            if self.hs:
                self.shared(x, T)
        self.combine(T)
        return self.y


class DecoderBlock:
    """One MobileMoE decoder block for decode steps (one new token per
    sequence): the MoE-FFN layer with its neighbours ([P1] "MoE preliminaries
    and three design factors": each layer is grouped-query attention plus the
    FFN on the residual stream; "Quantisation-aware training": every linear
    layer in W4A8; eq. (5): the KV cache in 8 bits).

        a  = RMSNorm(x)
        q, k, v = W4A8 projections of a        (n_h, n_kv heads of 64)
        append k, v at pos[b] of the INT8 KV caches
        o  = GQA decode attention of q over positions 0 .. lens[b] - 1
        h  = x + W4A8(o) ;  a2 = RMSNorm(h)
        y  = h + MoE-FFN(a2)

    Positional encoding (RoPE) is the caller's: q and k are used as the
    projections give them.  Every step runs in the library's kernels through
    the C ABI; torch holds the buffers."""

    def __init__(self, moe: MoELayer, n_h: int, n_kv: int, wq, wk, wv, wo, batch: int, max_T: int,
                 eps: float = 1e-5):
        if moe.wfmt != "int4g32" or moe.desc.out_dtype != B.MM_OUT_F32:
            raise ValueError("the decoder block runs the INT4 layer with FP32 output")
        d, dev = moe.d, moe.device
        self.moe, self.n_h, self.n_kv, self.B, self.max_T, self.eps = moe, n_h, n_kv, batch, max_T, eps
        self.d, self.dh = d, 64
        qd, kd = n_h * 64, n_kv * 64
        if wq.shape != (qd, d) or wk.shape != (kd, d) or wv.shape != (kd, d) or wo.shape != (d, qd):
            raise ValueError("projection shapes do not match n_h, n_kv and d")
        self.wq, self.wk = prepare_weight(wq, "int4g32", dev), prepare_weight(wk, "int4g32", dev)
        self.wv, self.wo = prepare_weight(wv, "int4g32", dev), prepare_weight(wo, "int4g32", dev)
        f32, i8 = torch.float32, torch.int8
        self.a = _empty((batch, d), f32, dev)
        self.aq, self.asc = _empty((batch, d), i8, dev), _empty((batch,), f32, dev)
        self.q = _empty((batch, qd), f32, dev)
        self.k, self.v = _empty((batch, kd), f32, dev), _empty((batch, kd), f32, dev)
        self.o = _empty((batch, qd), f32, dev)
        self.oq, self.osc = _empty((batch, qd), i8, dev), _empty((batch,), f32, dev)
        self.attn = _empty((batch, d), f32, dev)
        self.h, self.a2, self.y = (_empty((batch, d), f32, dev) for _ in range(3))
        # caches [B][n_kv][max_T][64] codes and [B][n_kv][max_T] scales
        cb = B.kv_cache_bytes(batch, n_kv, 64, max_T, B.MM_KV_CODES)
        sb = B.kv_cache_bytes(batch, n_kv, 64, max_T, B.MM_KV_SCALES) // 4
        self.kc = torch.zeros((cb,), dtype=i8, device=dev)
        self.vc = torch.zeros((cb,), dtype=i8, device=dev)
        self.ks = torch.zeros((sb,), dtype=f32, device=dev)
        self.vs = torch.zeros((sb,), dtype=f32, device=dev)
        self.ws, self.ws_bytes, self._ws_len = None, 0, 0

    def load_context(self, kq: np.ndarray, vq: np.ndarray, ks: np.ndarray, vs: np.ndarray):
        """Copies an existing cache (codes [B, n_kv, max_T, 64] int8, scales
        [B, n_kv, max_T] FP32) to the device."""
        for dst, src in ((self.kc, kq), (self.vc, vq), (self.ks, ks), (self.vs, vs)):
            dst.copy_(_dev(src, self.moe.device).reshape(-1))

    def _attn_ws(self, max_len: int):
        if max_len > self._ws_len:
            nb = max(B.attn_workspace_bytes(self.B, self.n_kv, max_len), 256)
            self.ws = torch.empty((nb,), dtype=torch.uint8, device=self.moe.device)
            self.ws_bytes, self._ws_len = nb, max_len

    def decode(self, x: torch.Tensor, pos: torch.Tensor, lens: torch.Tensor, max_len: int) -> torch.Tensor:
        """One decode step: x [B, d] FP32; pos [B] int32 (cache slot of the new
        token; outside 0 .. max_T - 1 skips the append), lens [B] int32
        (positions attended after the append, 0 .. max_len), max_len
        <= max_T.  Returns the block output y [B, d]."""
        Bn, d = self.B, self.d
        qd, kd = self.n_h * 64, self.n_kv * 64
        if tuple(x.shape) != (Bn, d) or max_len < 1 or max_len > self.max_T:
            raise ValueError("x must be [B, d] and 1 <= max_len <= max_T")
        self._attn_ws(max_len)
        B.rmsnorm_f32(Bn, d, self.eps, x, self.a)
        B.act_quant_i8(Bn, d, self.a, self.aq, self.asc)
        B.linear_w4a8(Bn, d, qd, self.aq, self.asc, self.wq.c(), self.q)
        B.linear_w4a8(Bn, d, kd, self.aq, self.asc, self.wk.c(), self.k)
        B.linear_w4a8(Bn, d, kd, self.aq, self.asc, self.wv.c(), self.v)
        B.kv_append_i8(Bn, self.n_kv, 64, self.max_T, pos, self.k, self.v, self.kc, self.vc,
                       self.ks, self.vs)
        B.attn_decode_i8(Bn, self.n_h, self.n_kv, 64, self.max_T, max_len, lens, self.q, self.kc,
                         self.vc, self.ks, self.vs, self.o, self.ws, self.ws_bytes)
        B.act_quant_i8(Bn, qd, self.o, self.oq, self.osc)
        B.linear_w4a8(Bn, qd, d, self.oq, self.osc, self.wo.c(), self.attn)
        B.add_rmsnorm_f32(Bn, d, self.eps, x, self.attn, self.h, self.a2)
        m = self.moe.forward_decode(self.a2) if self.moe.decode_supported(Bn) else \
            self.moe.forward_fused(self.a2)
        B.add_rmsnorm_f32(Bn, d, self.eps, self.h, m, self.y, None)
        return self.y
