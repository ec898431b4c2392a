"""The decoder block around the MoE-FFN layer, run one decode step at a time
through the C ABI (RMSNorm, W4A8 q/k/v projections, INT8 KV append, GQA decode
attention, W4A8 output projection, residual add + RMSNorm, the MoE-FFN layer,
residual add), against the oracle.

Each step is checked teacher-forced: every stage is recomputed by the oracle
on the input the device stage received, and must match bit for bit (integer
codes, W4A8 products, the MoE layer, the FP32 residual adds) or within the
stated tolerance (RMSNorm: FP32 on the device against double, row error
<= 1e-6; attention: FP32 against double, per-head row error <= 1e-4).  Beside
it the composed oracle runs the whole block from x with its own cache, and the
block outputs must agree (tokens whose routing the two rounding orders do not
change: row error <= 1e-2; the test prints the largest)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from sparse_moe_ffn_amd import workloads as wl
from sparse_moe_ffn_amd.layer import DecoderBlock
from gpu_util import DEV, make_layer, np_, oracle_forward, row_rel_err

pytestmark = pytest.mark.gpu

EPS = 1e-5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _quant_vectors(x: np.ndarray, n_kv: int):
    """INT8 codes and scales of each 64-value key/value vector of x [B, n_kv*64]."""
    q, s = oracle.quant_act_i8(x.reshape(-1, 64))
    return q.reshape(x.shape[0], n_kv, 64), s.reshape(x.shape[0], n_kv)


def _attend(q: np.ndarray, kq, vq, ks, vs, lens, n_h: int) -> np.ndarray:
    """oracle.attn_decode per sequence -> [B, n_h, 64] double (zeros for lens 0)."""
    out = np.zeros((q.shape[0], n_h, 64))
    for b in range(q.shape[0]):
        if lens[b] > 0:
            out[b] = oracle.attn_decode(q[b:b + 1].reshape(1, n_h, 64), kq[b:b + 1], vq[b:b + 1],
                                        ks[b:b + 1], vs[b:b + 1], int(lens[b]))[0]
    return out


class OracleBlock:
    """The block composed from oracle functions, with a host cache; every
    tensor the device keeps in FP32 is rounded to FP32 here too."""

    def __init__(self, w, lw, aw, cache):
        self.w, self.lw, self.aw = w, lw, aw
        self.kq, self.vq, self.ks, self.vs = (c.copy() for c in cache)
        self.wq = oracle.quant_w4g32(aw.wq)
        self.wk = oracle.quant_w4g32(aw.wk)
        self.wv = oracle.quant_w4g32(aw.wv)
        self.wo = oracle.quant_w4g32(aw.wo)

    def step(self, x, pos, lens):
        f32 = np.float32
        a = oracle.rmsnorm(x, EPS).astype(f32)
        aq, asc = oracle.quant_act_i8(a)
        q = oracle.linear_w4a8(aq, asc, *self.wq).astype(f32)
        k = oracle.linear_w4a8(aq, asc, *self.wk).astype(f32)
        v = oracle.linear_w4a8(aq, asc, *self.wv).astype(f32)
        n_kv = self.aw.n_kv
        kq, ks = _quant_vectors(k, n_kv)
        vq, vs = _quant_vectors(v, n_kv)
        for b, p in enumerate(pos):
            self.kq[b, :, p], self.ks[b, :, p] = kq[b], ks[b]
            self.vq[b, :, p], self.vs[b, :, p] = vq[b], vs[b]
        o = _attend(q, self.kq, self.vq, self.ks, self.vs, lens, self.aw.n_h)
        o = o.reshape(x.shape[0], -1).astype(f32)
        oq, osc = oracle.quant_act_i8(o)
        attn = oracle.linear_w4a8(oq, osc, *self.wo).astype(f32)
        h = x + attn
        a2 = oracle.rmsnorm(h, EPS).astype(f32)
        r = oracle_forward(self.w, self.lw, a2)
        return h + r.y.astype(f32), r.idx


CASES = [
    # (layer shape, batch, context before the first step, steps)
    ("s_decode", 1, 37, 2),          # one-launch MoE layer
    ("s_decode", 8, 300, 2),         # one-call MoE layer; ragged contexts
    ("m_decode", 3, 1000, 1),
    ("l_decode", 1, 8191, 1),        # the 8K context: the step fills the last slot
    ("s_decode", 64, 128, 1),
]


@pytest.mark.parametrize("name,Bn,ctx,steps", CASES)
def test_decoder_block_decode(name, Bn, ctx, steps):
    w = wl.WORKLOADS[name].with_(T=Bn)
    lw = wl.layer_weights(w)
    aw = wl.attn_weights(w)
    max_T = ctx + steps
    cache = wl.kv_context(w, Bn, max_T)
    block = DecoderBlock(make_layer(w, lw), aw.n_h, aw.n_kv, aw.wq, aw.wk, aw.wv, aw.wo, Bn, max_T,
                         EPS)
    block.load_context(*cache)
    ref = OracleBlock(w, lw, aw, cache)
    wq, wk, wv, wo = ref.wq, ref.wk, ref.wv, ref.wo
    # ragged contexts: sequence b has ctx - 3b earlier positions (at least 1)
    start = np.maximum(ctx - 3 * np.arange(Bn), 1).astype(np.int32)
    worst = 0.0
    for s in range(steps):
        x = wl.tokens(w, step=s, T=Bn)
        pos = (start + s).astype(np.int32)
        lens = pos + 1
        y = np_(block.decode(dev(x), dev(pos), dev(lens), int(lens.max()))).copy()
        # --- teacher-forced stages
        a = np_(block.a)
        assert row_rel_err(a, oracle.rmsnorm(x, EPS)) <= 1e-6
        aq, asc = oracle.quant_act_i8(a)
        assert np.array_equal(np_(block.aq), aq) and np.array_equal(np_(block.asc), asc)
        q = np_(block.q)
        assert np.array_equal(q, oracle.linear_w4a8(aq, asc, *wq).astype(np.float32))
        k, v = np_(block.k), np_(block.v)
        assert np.array_equal(k, oracle.linear_w4a8(aq, asc, *wk).astype(np.float32))
        assert np.array_equal(v, oracle.linear_w4a8(aq, asc, *wv).astype(np.float32))
        kc = np_(block.kc).reshape(Bn, aw.n_kv, max_T, 64)
        vc = np_(block.vc).reshape(Bn, aw.n_kv, max_T, 64)
        ksd = np_(block.ks).reshape(Bn, aw.n_kv, max_T)
        vsd = np_(block.vs).reshape(Bn, aw.n_kv, max_T)
        kq_new, ks_new = _quant_vectors(k, aw.n_kv)
        vq_new, vs_new = _quant_vectors(v, aw.n_kv)
        for b in range(Bn):
            assert np.array_equal(kc[b, :, pos[b]], kq_new[b]) and np.array_equal(ksd[b, :, pos[b]], ks_new[b])
            assert np.array_equal(vc[b, :, pos[b]], vq_new[b]) and np.array_equal(vsd[b, :, pos[b]], vs_new[b])
        o = np_(block.o)
        o_ref = _attend(q, kc, vc, ksd, vsd, lens, aw.n_h)
        err = np.abs(o.reshape(o_ref.shape) - o_ref).max(2) / np.abs(o_ref).max(2)
        assert err.max() <= 1e-4, err.max()
        oq, osc = oracle.quant_act_i8(o)
        assert np.array_equal(np_(block.oq), oq) and np.array_equal(np_(block.osc), osc)
        attn = np_(block.attn)
        assert np.array_equal(attn, oracle.linear_w4a8(oq, osc, *wo).astype(np.float32))
        h = np_(block.h)
        assert np.array_equal(h, x + attn)
        a2 = np_(block.a2)
        assert row_rel_err(a2, oracle.rmsnorm(h, EPS)) <= 1e-6
        moe = oracle_forward(w, lw, a2)
        assert np.array_equal(np_(block.moe.idx), moe.idx)
        m = np_(block.moe.y)
        assert np.array_equal(m, moe.y.astype(np.float32))
        assert np.array_equal(y, h + m)
        # --- the composed oracle from x, with its own cache
        y_ref, idx_ref = ref.step(x, pos, lens)
        same = (np.sort(np_(block.moe.idx), 1) == np.sort(idx_ref, 1)).all(1)
        if same.any():
            e = row_rel_err(y[same], y_ref[same])
            worst = max(worst, e)
            assert e <= 1e-2, (s, e)
        assert (~same).sum() <= max(1, Bn // 8), (~same).sum()
    print(f"{name} B={Bn}: block output against the composed oracle, worst row error {worst:.2e}")
