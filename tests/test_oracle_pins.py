"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- closed forms, brute force on tiny inputs, double-precision
explicit dequantisation, library routines, invariants the method fixes, and
the sizes the MobileMoE close reading prints.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

from sparse_moe_ffn_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------- eq. (6), b=4
def _crafted_weights():
    g = rng(1)
    w = (g.standard_normal((24, 128)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                      # all-zero group
    w[1, :32] = 0.0
    w[1, 5] = 0.3                        # single non-zero element
    w[2, 32:64] = np.linspace(-1, 1, 32, dtype=np.float32)   # exact +-max
    w[3, :32] = -w[3, :32]
    w[4, 64:96] = 1e-30                  # tiny values
    return w


def test_quant_w4_range_and_error_bound(ora):
    w = _crafted_weights()
    q, s = ora.quant_w4g32(w)
    assert q.min() >= -8 and q.max() <= 7
    wq = w.reshape(24, 4, 32).astype(np.float64)
    qq = q.reshape(24, 4, 32).astype(np.float64)
    ss = s.astype(np.float64)[..., None]
    amax = np.abs(wq).max(-1, keepdims=True)
    # scale is 2*max/15 up to one FP32 rounding
    np.testing.assert_allclose(ss, 2 * amax / 15, rtol=2 ** -23, atol=0)
    err = np.abs(wq - ss * qq)
    # every element is within half a step, except +max which clips from 7.5 to 7
    is_pmax = (wq == amax) & (amax > 0)
    assert np.all(err[~is_pmax] <= ss.repeat(32, -1)[~is_pmax] * (0.5 + 1e-5))
    assert np.all(qq[is_pmax] == 7)
    # -max lands on -7.5 up to the rounding of s, so -8 (half-even) or -7
    is_nmax = (wq == -amax) & (amax > 0)
    assert np.all(np.isin(qq[is_nmax], (-8, -7)))
    # all-zero group -> zero scale and codes
    assert s[0, 0] == 0 and np.all(q[0, :32] == 0)
    # single non-zero element -> it is the max, code 7; the rest 0
    assert q[1, 5] == 7 and np.count_nonzero(q[1, :32]) == 1


def test_quant_w4_dequant_error_is_small(ora):
    """Group-32 symmetric INT4 reconstruction error is bounded by s/2 per element,
    i.e. relative RMS error well under the 4-bit step."""
    w = (rng(2).standard_normal((64, 256)) * 0.02).astype(np.float32)
    q, s = ora.quant_w4g32(w)
    wd = q.reshape(64, 8, 32) * s[..., None].astype(np.float64)
    rel = np.sqrt(((wd.reshape(64, 256) - w) ** 2).mean()) / np.sqrt((w.astype(np.float64) ** 2).mean())
    assert 0.02 < rel < 0.2


def test_quant_w4_grouping_axis(ora):
    """Groups run along the reduction (column) axis: scaling one 32-column block
    by 2 doubles only that block's scale and leaves codes unchanged."""
    w = (rng(3).standard_normal((8, 96)) * 0.02).astype(np.float32)
    q1, s1 = ora.quant_w4g32(w)
    w2 = w.copy()
    w2[:, 32:64] *= 2
    q2, s2 = ora.quant_w4g32(w2)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2[:, 1], s1[:, 1] * 2)
    assert np.array_equal(s2[:, [0, 2]], s1[:, [0, 2]])


# ----------------------------------------------------------------- INT8 activations
def test_quant_act_invariants(ora):
    g = rng(4)
    x = g.standard_normal((50, 768)).astype(np.float32)
    x[3] = 0.0
    q, s = ora.quant_act_i8(x)
    assert s[3] == 0 and np.all(q[3] == 0)
    xd = q.astype(np.float64) * s[:, None]
    amax = np.abs(x).max(1)
    nz = amax > 0
    np.testing.assert_allclose(s[nz], 2 * amax[nz].astype(np.float64) / 255, rtol=2 ** -23)
    err = np.abs(xd - x)
    pmax = (x == amax[:, None]) & nz[:, None]
    assert np.all(q[pmax] == 127)                      # +max maps to 127 (from 127.5)
    nmax = (x == -amax[:, None]) & nz[:, None]
    assert np.all(np.isin(q[nmax], (-128, -127)))
    assert np.all(err[~pmax] <= s[:, None].repeat(768, 1)[~pmax] * (0.5 + 1e-5))
    # power-of-two scaling of a row scales s exactly and keeps q
    q2, s2 = ora.quant_act_i8(x * np.float32(4))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * 4)


# ----------------------------------------------------------------- W4A8 linear
def test_linear_isum_bruteforce_and_dequant(ora):
    """int32 group sums equal an int64 brute-force product; the scaled output
    equals the explicitly dequantised product computed in double."""
    g = rng(5)
    rows, N, K = 7, 40, 192
    x = g.standard_normal((rows, K)).astype(np.float32)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, ws = ora.quant_w4g32(w)
    aq, sa = ora.quant_act_i8(x)
    out, isum = ora.linear_w4a8(aq, sa, wq, ws, want_isum=True)
    brute = np.einsum("rgc,ogc->rog", aq.reshape(rows, K // 32, 32).astype(np.int64),
                      wq.reshape(N, K // 32, 32).astype(np.int64))
    assert np.array_equal(isum.astype(np.int64), brute)
    assert np.abs(brute).max() <= 32 * 8 * 128
    wdq = (wq.reshape(N, K // 32, 32) * ws[..., None].astype(np.float64)).reshape(N, K)
    xdq = aq.astype(np.float64) * sa[:, None].astype(np.float64)
    ref = xdq @ wdq.T
    # FP32 scale application (fma chain over 6 groups, then one product)
    bound = 8 * 2.0 ** -24 * (np.abs(isum) * ws[None].astype(np.float64)).sum(-1) * sa[:, None]
    assert np.all(np.abs(out - ref) <= bound + 1e-30)


# ----------------------------------------------------------------- router
def _f32_round(fr: Fraction) -> Fraction:
    """Round an exact rational to the nearest FP32 value, ties to even (normal range)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def test_router_logit_exact_rational_emulation(ora):
    """Brute force: every fma and every tree addition of the router's fixed order
    evaluated in exact rational arithmetic with one FP32 rounding each."""
    g = rng(6)
    T, d, E = 3, 128, 5
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = g.standard_normal(E).astype(np.float32)
    _, _, logits = ora.router(x, wr, bias, k=2)
    for t in range(T):
        for e in range(E):
            p = [Fraction(0)] * 64
            for j in range(d):
                p[j % 64] = _f32_round(Fraction(float(x[t, j])) * Fraction(float(wr[e, j])) + p[j % 64])
            s = 1
            while s < 64:
                for l in range(0, 64, 2 * s):
                    p[l] = _f32_round(p[l] + p[l + s])
                s *= 2
            ref = _f32_round(p[0] + Fraction(float(bias[e])))
            assert Fraction(float(logits[t, e])) == ref


def test_router_against_double(ora):
    g = rng(7)
    T, d, E, k = 256, 768, 60, 4
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.02).astype(np.float32)
    idx, w, logits = ora.router(x, wr, None, k=k)
    l64 = x.astype(np.float64) @ wr.astype(np.float64).T
    bound = d * 2.0 ** -23 * (np.abs(x).astype(np.float64) @ np.abs(wr).astype(np.float64).T)
    assert np.all(np.abs(logits - l64) <= bound)
    # selection equals the double-precision ranking wherever the margin is clear
    srt = np.argsort(-l64, axis=1, kind="stable")
    clear = (np.take_along_axis(l64, srt[:, k - 1:k], 1) - np.take_along_axis(l64, srt[:, k:k + 1], 1))[:, 0] \
        > 4 * bound.max()
    for t in np.nonzero(clear)[0]:
        assert set(idx[t]) == set(srt[t, :k])
    assert clear.mean() > 0.9
    # idx listed by descending logit, distinct
    assert np.all(np.diff(np.take_along_axis(logits, idx, 1), axis=1) <= 0)
    assert all(len(set(r)) == k for r in idx)
    # gate weights: softmax over all E (library routine), not renormalised
    lg = logits.astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-6)
    assert np.all(w.sum(1) < 1.0)


def test_router_full_k_sums_to_one(ora):
    g = rng(8)
    x = g.standard_normal((16, 64)).astype(np.float32)
    wr = g.standard_normal((8, 64)).astype(np.float32)
    idx, w, logits = ora.router(x, wr, None, k=8)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.sort(idx, 1) == np.arange(8))


def test_router_ties_and_forced_bias(ora):
    g = rng(9)
    x = g.standard_normal((10, 128)).astype(np.float32)
    row = (g.standard_normal(128) * 0.02).astype(np.float32)
    wr = np.tile(row, (60, 1))
    idx, w, _ = ora.router(x, wr, None, k=4)
    assert np.all(idx == np.arange(4))             # equal logits: lowest index first
    np.testing.assert_allclose(w, 1 / 60, rtol=1e-6)
    wr2 = (g.standard_normal((60, 128)) * 0.02).astype(np.float32)
    bias = np.zeros(60, np.float32)
    bias[[7, 19, 33, 58]] = [100, 101, 102, 103]
    idx2, _, _ = ora.router(x, wr2, bias, k=4)
    assert np.all(idx2 == [58, 33, 19, 7])


def test_router_sigmoid_gate(ora):
    g = rng(10)
    x = g.standard_normal((32, 128)).astype(np.float32)
    wr = (g.standard_normal((60, 128)) * 0.1).astype(np.float32)
    i_s, w_s, lg = ora.router(x, wr, None, k=4, gating=0)
    i_g, w_g, _ = ora.router(x, wr, None, k=4, gating=1)
    assert np.array_equal(i_s, i_g)                # both gates are monotone in the logit
    sel = np.take_along_axis(lg.astype(np.float64), i_g, 1)
    ref = expit(sel) / expit(sel).sum(1, keepdims=True)
    np.testing.assert_allclose(w_g, ref, rtol=1e-6)


def test_router_selection_only_bias(ora):
    """Bias that steers the selection only (gating | 2): the ids are those of
    the biased ranking, the gate weights those of the unbiased logits."""
    g = rng(12)
    x = g.standard_normal((32, 128)).astype(np.float32)
    wr = (g.standard_normal((60, 128)) * 0.1).astype(np.float32)
    bias = (g.standard_normal(60) * 0.5).astype(np.float32)
    _, _, raw = ora.router(x, wr, None, k=4, gating=0)            # logits without the bias
    raw64 = raw.astype(np.float64)
    for base in (0, 1):
        i_b, _, _ = ora.router(x, wr, bias, k=4, gating=base)     # bias in selection and gate
        i_s, w_s, _ = ora.router(x, wr, bias, k=4, gating=base | 2)
        assert np.array_equal(i_s, i_b)                          # the same ranking
        biased = raw64 + bias.astype(np.float64)
        assert np.array_equal(i_s[:, 0], np.argmax(biased, 1))
        sel = np.take_along_axis(raw64, i_s, 1)
        if base == 0:
            p = np.exp(raw64 - raw64.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            ref = np.take_along_axis(p, i_s, 1)
        else:
            ref = expit(sel) / expit(sel).sum(1, keepdims=True)
        np.testing.assert_allclose(w_s, ref, rtol=1e-6)
        # a zero bias changes nothing
        i0, w0, _ = ora.router(x, wr, np.zeros(60, np.float32), k=4, gating=base | 2)
        i1, w1, _ = ora.router(x, wr, None, k=4, gating=base)
        assert np.array_equal(i0, i1) and np.array_equal(w0, w1)
    # a large bias forces the routing but not the gate values
    forced = np.zeros(60, np.float32)
    forced[[7, 19, 33, 58]] = [100, 110, 120, 130]                # gaps far above the logits' spread
    i_f, w_f, _ = ora.router(x, wr, forced, k=4, gating=2)
    assert np.all(i_f == [58, 33, 19, 7])
    p = np.exp(raw64 - raw64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(w_f, p[:, [58, 33, 19, 7]], rtol=1e-6)


# ----------------------------------------------------------------- routing
def test_route_invariants_and_stable_sort(ora):
    g = rng(11)
    T, E, k = 300, 60, 4
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, perm, inv = ora.route(idx, E)
    flat = idx.reshape(-1)
    assert off[0] == 0 and off[E] == T * k
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))  # library stable sort
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_route_rejects_bad_ids(ora):
    with pytest.raises(ValueError):
        ora.route(np.array([[0, 61]], np.int32), 60)


# ----------------------------------------------------------------- FFN and layer
def _dense_swiglu(x, wgu, wd):
    h = wd.shape[1]
    gu = x @ wgu.T
    a = gu[:, :h] * expit(gu[:, :h]) * gu[:, h:]
    return a @ wd.T


def _mk(E, d, h, hs, seed, std=0.02):
    g = rng(seed)
    wr = (g.standard_normal((E, d)) * std).astype(np.float32)
    wgu = (g.standard_normal((E, 2 * h, d)) * std).astype(np.float32)
    wd = (g.standard_normal((E, d, h)) * std).astype(np.float32)
    sgu = (g.standard_normal((2 * hs, d)) * std).astype(np.float32) if hs else None
    sd = (g.standard_normal((d, hs)) * std).astype(np.float32) if hs else None
    return wr, wgu, wd, sgu, sd


def test_ffn_w4a8_against_dequantised_double(ora):
    g = rng(12)
    d, h, rows = 256, 128, 24
    x = g.standard_normal((rows, d)).astype(np.float32)
    wgu = (g.standard_normal((2 * h, d)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((d, h)) * 0.02).astype(np.float32)
    guq, gus = ora.quant_w4g32(wgu)
    dq, ds = ora.quant_w4g32(wd)
    xq, sx = ora.quant_act_i8(x)
    hq, hs, f = ora.ffn_w4a8(xq, sx, guq, gus, dq, ds)
    W = lambda q, s: (q.reshape(q.shape[0], -1, 32) * s[..., None].astype(np.float64)).reshape(q.shape)
    xd = xq * sx[:, None].astype(np.float64)
    gu = xd @ W(guq, gus).T
    a = gu[:, :h] * expit(gu[:, :h]) * gu[:, h:]
    # hidden row re-quantised per row, then the down product on the dequantised row
    hd = hq * hs[:, None].astype(np.float64)
    amax = np.abs(a).max(1)
    np.testing.assert_allclose(hs, 2 * amax / 255, rtol=1e-6)
    assert np.all(np.abs(hd - a) <= hs[:, None] * 0.5 * (1 + 1e-4))
    fd = hd @ W(dq, ds).T
    assert (np.abs(f - fd).max(1) / np.abs(fd).max(1)).max() < 1e-5
    # the exposed FP32 hidden row: close to the double SwiGLU, and its own
    # per-row quantisation is exactly the hidden code row
    a32 = ora.ffn_w4a8(xq, sx, guq, gus, dq, ds, want_a=True)[3]
    assert (np.abs(a32 - a).max(1) / np.abs(a).max(1)).max() < 1e-5
    hq2, hs2 = ora.quant_act_i8(a32)
    assert np.array_equal(hq2, hq) and np.array_equal(hs2, hs)
    # and the whole thing is close to the unquantised FP32 FFN
    ref = _dense_swiglu(x.astype(np.float64), wgu.astype(np.float64), wd.astype(np.float64))
    assert np.abs(f - ref).max() / np.abs(ref).max() < 0.3


def test_degenerate_single_expert_is_dense_swiglu(ora):
    """E = 1, k = 1, no shared expert: the gate is exp(0)/1 = 1 and the layer is
    a plain dense SwiGLU FFN."""
    g = rng(13)
    d, h, T = 128, 64, 20
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, _, _ = _mk(1, d, h, 0, 14)
    r = ora.forward(x, wr, None, wgu, wd, None, None, k=1, wfmt="f32")
    assert np.all(r.w == 1.0) and np.all(r.idx == 0)
    ref = _dense_swiglu(x.astype(np.float64), wgu[0].astype(np.float64), wd[0].astype(np.float64))
    np.testing.assert_allclose(r.y, ref, rtol=1e-12, atol=1e-15)
    ri = ora.forward(x, wr, None, wgu, wd, None, None, k=1, wfmt="int4g32")
    assert np.abs(ri.y - ref).max() / np.abs(ref).max() < 0.3


def test_k_equals_E_is_dense_softmax_mixture(ora):
    g = rng(15)
    E, d, h, hs, T = 6, 64, 64, 64, 12
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 16, std=0.2)
    r = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=E, wfmt="f32")
    lg = r.logits.astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    X = x.astype(np.float64)
    ref = sum(p[:, e:e + 1] * _dense_swiglu(X, wgu[e].astype(np.float64), wd[e].astype(np.float64))
              for e in range(E))
    ref += _dense_swiglu(X, sgu.astype(np.float64), sd.astype(np.float64))
    assert (np.abs(r.y - ref).max(1) / np.abs(ref).max(1)).max() < 1e-6


@pytest.mark.parametrize("wfmt", ["f32", "int4g32"])
def test_dense_masked_bruteforce(ora, wfmt):
    """Every expert evaluated on every token, then masked by the top-k choice,
    equals the sparse layer."""
    g = rng(17)
    E, d, h, hs, T, k = 8, 64, 64, 64, 16, 3
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 18, std=0.1)
    r = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=k, wfmt=wfmt)
    lg = r.logits.astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, r.idx, 1.0, 1)
    if wfmt == "f32":
        X = x.astype(np.float64)
        allf = np.stack([_dense_swiglu(X, wgu[e].astype(np.float64), wd[e].astype(np.float64))
                         for e in range(E)], 1)
        ys = _dense_swiglu(X, sgu.astype(np.float64), sd.astype(np.float64))
        exact_parts = False
    else:
        xq, sx = ora.quant_act_i8(x)
        allf = np.stack([ora.ffn_w4a8(xq, sx, *ora.quant_w4g32(wgu[e]), *ora.quant_w4g32(wd[e]))[2]
                         for e in range(E)], 1).astype(np.float64)
        ys = ora.ffn_w4a8(xq, sx, *ora.quant_w4g32(sgu), *ora.quant_w4g32(sd))[2].astype(np.float64)
        exact_parts = True
    ref = np.einsum("te,ted->td", mask * p, allf) + ys
    # gate weights and the combine are FP32 in the INT4 path
    assert (np.abs(r.y - ref).max(1) / np.abs(ref).max(1)).max() < 1e-6
    sel = np.take_along_axis(allf, r.idx[..., None], 1)
    if exact_parts:          # same FP32 arithmetic, evaluated expert by expert
        assert np.array_equal(r.ys, ys) and np.array_equal(r.f, sel)
    else:
        np.testing.assert_allclose(r.ys, ys, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r.f, sel, rtol=1e-12, atol=1e-15)


def test_shared_expert_reaches_every_token(ora):
    g = rng(19)
    E, d, h, hs, T = 60, 128, 64, 256, 40
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 20)
    for wfmt in ("f32", "int4g32"):
        r = ora.forward(x, wr, None, wgu, np.zeros_like(wd), sgu, sd, k=4, wfmt=wfmt)
        assert np.array_equal(r.y, r.ys) and np.all(np.abs(r.ys).max(1) > 0)
        r0 = ora.forward(x, wr, None, wgu, wd, np.zeros_like(sgu), np.zeros_like(sd), k=4, wfmt=wfmt)
        assert np.all(r0.ys == 0)


def test_token_permutation_equivariance(ora):
    g = rng(21)
    E, d, h, hs, T = 60, 128, 64, 256, 33
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 22)
    pi = g.permutation(T)
    a = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=4)
    b = ora.forward(x[pi], wr, None, wgu, wd, sgu, sd, k=4)
    assert np.array_equal(a.y[pi], b.y) and np.array_equal(a.idx[pi], b.idx)


def test_expert_relabelling(ora):
    g = rng(23)
    E, d, h, hs, T = 60, 128, 64, 128, 25
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 24)
    sigma = g.permutation(E)              # new label i holds old expert sigma[i]
    a = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=4)
    b = ora.forward(x, wr[sigma], None, wgu[sigma], wd[sigma], sgu, sd, k=4)
    assert np.array_equal(sigma[b.idx], a.idx)
    # the softmax denominator's summation tree follows expert labels, so only
    # rounding may differ
    assert (np.abs(b.y - a.y).max(1) / np.abs(a.y).max(1)).max() < 1e-6


def test_layer_routing_properties(ora):
    g = rng(25)
    E, d, h, hs, T, k = 60, 256, 64, 256, 64, 4
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 26)
    r = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=k)
    assert all(len(set(row)) == k for row in r.idx)      # k distinct experts per token
    off, perm, inv = ora.route(r.idx, E)
    assert off[E] == T * k and np.bincount(r.idx.reshape(-1), minlength=E).sum() == T * k


def test_bf16_rounding_matches_torch(ora):
    torch = pytest.importorskip("torch")
    x = (rng(27).standard_normal(100_000) * 10).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ora.round_bf16(x), ref)


def test_bf16_layer_close_to_f32(ora):
    g = rng(28)
    E, d, h, hs, T = 60, 128, 64, 256, 16
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 29)
    a = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=4, wfmt="f32")
    b = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=4, wfmt="bf16")
    assert np.array_equal(a.idx, b.idx)
    assert np.all(ora.round_bf16(b.y.astype(np.float32)) == b.y)
    assert np.abs(a.y - b.y).max() / np.abs(a.y).max() < 2e-2


def _bf16_ffn_torch(x, wgu, wd, round_x=True, round_w=True, round_a=True):
    """BF16-weight SwiGLU FFN evaluated independently of the oracle: torch's
    bfloat16 conversion (round to nearest even) of x, of both weights and of
    the hidden row (through FP32, as an FP32 kernel rounds it), every product
    and sum in float64.  The flags drop one rounding each, to show that the
    pin below can see it."""
    torch = pytest.importorskip("torch")
    bf = lambda a, on: (torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
                        .to(torch.float64) if on else torch.from_numpy(a.astype(np.float64)))
    h = wd.shape[1]
    gu = bf(x, round_x) @ bf(wgu, round_w).T
    g, u = gu[:, :h], gu[:, h:]
    a = g * torch.sigmoid(g) * u
    if round_a:
        a = a.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    return (a @ bf(wd, round_w).T).numpy()


def test_bf16_ffn_against_torch_casts(ora):
    """The BF16 path (R15: x, weights and the hidden row rounded to BF16,
    sums in higher precision) equals an independent torch evaluation to
    1e-9 of each row's maximum; evaluations without one of the three
    roundings miss it by orders of magnitude more."""
    g = rng(40)
    d, h, rows = 256, 128, 24
    x = g.standard_normal((rows, d)).astype(np.float32)
    wgu = (g.standard_normal((2 * h, d)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((d, h)) * 0.02).astype(np.float32)
    got = ora.ffn_float(x, wgu, wd, bf16=True)
    rel = lambda a, b: float((np.abs(a - b).max(1) / np.abs(b).max(1)).max())
    assert rel(got, _bf16_ffn_torch(x, wgu, wd)) < 1e-9
    for drop in ("round_x", "round_w", "round_a"):
        assert rel(got, _bf16_ffn_torch(x, wgu, wd, **{drop: False})) > 1e-5, drop


def test_bf16_layer_against_torch_casts(ora):
    """Whole BF16 layer: each selected expert and the shared expert from the
    independent torch evaluation, combined with the router's weights in
    float64, the output rounded to BF16 (through FP32) -- equal to the
    oracle's layer except where a value sits within rounding of a BF16 tie."""
    torch = pytest.importorskip("torch")
    g = rng(41)
    E, d, h, hs, T, k = 8, 128, 64, 256, 12, 4
    x = g.standard_normal((T, d)).astype(np.float32)
    wr, wgu, wd, sgu, sd = _mk(E, d, h, hs, 42)
    r = ora.forward(x, wr, None, wgu, wd, sgu, sd, k=k, wfmt="bf16")
    ys = _bf16_ffn_torch(x, sgu, sd)
    y = ys.copy()
    for t in range(T):
        for j in range(k):
            e = r.idx[t, j]
            y[t] += r.w[t, j] * _bf16_ffn_torch(x[t:t + 1], wgu[e], wd[e])[0]
    yb = torch.from_numpy(y).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert float((np.abs(r.ys - ys).max(1) / np.abs(ys).max(1)).max()) < 1e-9
    # one BF16 ulp is 2^-8 relative: rounding may differ only for y within 1e-9 of a tie
    diff = r.y != yb
    assert diff.mean() < 1e-3
    assert np.all(np.abs(r.y - yb)[diff] <= np.abs(yb)[diff] * 2.0 ** -7)


def test_exp_ref_accuracy(ora):
    x = np.linspace(-87.3, 88.7, 3_000_001, dtype=np.float32)
    y = ora.exp_ref(x).astype(np.float64)
    r = np.exp(x.astype(np.float64))
    assert (np.abs(y - r) / r).max() < 2.5 * 2.0 ** -24      # within ~2 ulp
    sp = ora.exp_ref(np.array([0.0, 1.0, -1.0, 89.0, -88.0, 1e-8], np.float32))
    assert sp[0] == 1.0 and sp[3] == np.inf and sp[4] == 0.0 and sp[5] == 1.0
    assert abs(sp[1] - np.e) <= 2.5e-7 * np.e and abs(sp[2] - 1 / np.e) <= 2.5e-7 / np.e


def test_combine_f32_against_double(ora):
    g = rng(32)
    f = g.standard_normal((7, 4, 64)).astype(np.float32)
    w = g.random((7, 4)).astype(np.float32)
    ys = g.standard_normal((7, 64)).astype(np.float32)
    ref = np.einsum("tj,tjd->td", w.astype(np.float64), f.astype(np.float64)) + ys
    got = ora.combine_f32(f, w, ys)
    assert np.abs(got - ref).max() < 1e-5
    assert np.array_equal(ora.combine_f32(f, w, None) + ys, got) or np.abs(
        ora.combine_f32(f, w, None) + ys - got).max() == 0


def test_combine_closed_form(ora):
    g = rng(30)
    f = g.standard_normal((5, 4, 16))
    w = g.random((5, 4))
    ys = g.standard_normal((5, 16))
    np.testing.assert_allclose(ora.combine(f, w, ys), np.einsum("tj,tjd->td", w, f) + ys, rtol=1e-14)
    np.testing.assert_allclose(ora.combine(f, w, None), np.einsum("tj,tjd->td", w, f), rtol=1e-14)


def test_rmsnorm_closed_form(ora):
    x = np.full((2, 64), 3.0, np.float32)
    x[1] = -3.0
    y = ora.rmsnorm(x, eps=0.0)
    np.testing.assert_allclose(y, np.sign(x), rtol=1e-15)
    z = rng(31).standard_normal((4, 96)).astype(np.float32)
    yz = ora.rmsnorm(z, eps=0.0)
    np.testing.assert_allclose((yz ** 2).mean(1), 1.0, rtol=1e-12)


def test_rmsnorm_eps_closed_form(ora):
    """With eps > 0 a constant row c gives c / sqrt(c^2 + eps) in every
    column (eps inside the square root, added to the mean square); at
    c^2 = 10 eps that is 4.7 % below the eps = 0 value, so a dropped or
    misplaced eps fails."""
    for c, eps in ((0.01, 1e-5), (-0.03, 1e-5), (2.0, 0.5)):
        x = np.full((3, 128), c, np.float32)
        y = ora.rmsnorm(x, eps=eps)
        c64 = float(np.float32(c))
        np.testing.assert_allclose(y, c64 / np.sqrt(c64 * c64 + eps), rtol=1e-14)
    # a row with a known mean square: values +-a, mean square a^2
    a = np.float32(0.02)
    x = np.tile(np.array([a, -a], np.float32), (2, 48))
    y = ora.rmsnorm(x, eps=1e-4)
    np.testing.assert_allclose(np.abs(y), float(a) / np.sqrt(float(a) ** 2 + 1e-4), rtol=1e-14)


def test_oracle_rejects_bad_shapes(ora):
    with pytest.raises(ValueError):
        ora.quant_w4g32(np.zeros((2, 40), np.float32))
    with pytest.raises(ValueError):
        ora.router(np.zeros((2, 100), np.float32), np.zeros((4, 100), np.float32), None, k=2)


# ----------------------------------------------------------------- printed sizes
def test_layer_shapes_reproduce_printed_parameter_counts():
    """Routed hidden d/2 (d_ff = 4d split g = 8 ways), shared hidden 4x that,
    60 experts, top-4, FP32 router [E, d], GQA with 4 KV heads of 64, and a
    128K tied vocabulary reproduce the printed active and total counts of
    MobileMoE-S/M/L, with 20/26/32 layers (d/n_l close to 40)."""
    g = {e["key"]: e for e in json.load(open(os.path.join(GOLDEN, "mobilemoe_printed_shapes.json")))["entries"]}
    s = wl.WORKLOADS["s_prefill"]
    assert (s.d, s.h) == tuple(g["s_expert_shape"]["value"])
    assert s.E == g["routed_experts"]["value"] and s.k == g["top_k"]["value"]
    for name, key, n_l in (("s_prefill", "S", 20), ("m_prefill", "M", 26), ("l_prefill", "L", 32)):
        w = wl.WORKLOADS[name]
        assert w.h * g["granularity"]["value"] == g["ffn_expansion_ratio"]["value"] * w.d
        assert w.hs == g["shared_expert_size_ratio"]["value"] * w.h
        act, tot = wl.param_counts(w.d, n_l, n_kv=g["kv_heads"]["value"], d_head=g["head_dim"]["value"])
        assert abs(act - g[f"active_params_{key}"]["value"]) <= g[f"active_params_{key}"]["tol"]
        assert abs(tot - g[f"total_params_{key}"]["value"]) <= g[f"total_params_{key}"]["tol"]
        assert abs(w.d / n_l - g["aspect_ratio_d_over_layers"]["value"]) <= g["aspect_ratio_d_over_layers"]["tol"]


# ----------------------------------------------------------------- GQA decode attention
def _kv_case(g, B, nh, nkv, dh, maxT):
    q = g.standard_normal((B, nh, dh)).astype(np.float32)
    kq = g.integers(-128, 128, (B, nkv, maxT, dh)).astype(np.int8)
    vq = g.integers(-128, 128, (B, nkv, maxT, dh)).astype(np.int8)
    ks = (g.uniform(0.5, 1.5, (B, nkv, maxT)) / 127).astype(np.float32)
    vs = (g.uniform(0.5, 1.5, (B, nkv, maxT)) / 127).astype(np.float32)
    return q, kq, vq, ks, vs


def test_attn_decode_against_library_sdpa(ora):
    """Dequantised cache through torch's scaled dot-product attention (float64,
    key/value heads repeated for the query-head groups)."""
    import torch
    g = rng(20)
    B, nh, nkv, dh, maxT, T = 2, 12, 4, 64, 40, 33
    q, kq, vq, ks, vs = _kv_case(g, B, nh, nkv, dh, maxT)
    out = ora.attn_decode(q, kq, vq, ks, vs, T)
    k = torch.from_numpy(kq[:, :, :T].astype(np.float64) * ks[:, :, :T, None].astype(np.float64))
    v = torch.from_numpy(vq[:, :, :T].astype(np.float64) * vs[:, :, :T, None].astype(np.float64))
    grp = nh // nkv
    k = k.repeat_interleave(grp, dim=1)
    v = v.repeat_interleave(grp, dim=1)
    qq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v)[:, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_attn_decode_special_cases(ora):
    g = rng(21)
    B, nh, nkv, dh, maxT = 1, 8, 4, 64, 16
    q, kq, vq, ks, vs = _kv_case(g, B, nh, nkv, dh, maxT)
    deq_v = vq.astype(np.float64) * vs[..., None].astype(np.float64)
    # one position: every head returns its group's value row
    out = ora.attn_decode(q, kq, vq, ks, vs, 1)
    for h in range(nh):
        np.testing.assert_array_equal(out[0, h], deq_v[0, h // 2, 0])
    # identical keys: uniform weights, the mean of the values
    kq2 = np.broadcast_to(kq[:, :, :1], kq.shape).copy()
    ks2 = np.broadcast_to(ks[:, :, :1], ks.shape).copy()
    out = ora.attn_decode(q, kq2, vq, ks2, vs, 10)
    for h in range(nh):
        np.testing.assert_allclose(out[0, h], deq_v[0, h // 2, :10].mean(0), rtol=1e-12, atol=1e-15)
    # positions past T never matter
    kq3, vq3 = kq.copy(), vq.copy()
    kq3[:, :, 10:] = 127
    vq3[:, :, 10:] = -128
    np.testing.assert_array_equal(ora.attn_decode(q, kq3, vq3, ks, vs, 10),
                                  ora.attn_decode(q, kq, vq, ks, vs, 10))
    # grouped heads: equal queries in one group give equal outputs; another group differs
    q4 = q.copy()
    q4[0, 1] = q4[0, 0]
    o4 = ora.attn_decode(q4, kq, vq, ks, vs, 12)
    np.testing.assert_array_equal(o4[0, 0], o4[0, 1])
    q4[0, 2] = q4[0, 0]
    o5 = ora.attn_decode(q4, kq, vq, ks, vs, 12)
    assert not np.allclose(o5[0, 2], o5[0, 0])


# ----------------------------------------------------------------- training side
def test_bias_update_pins(ora):
    """Aux-loss-free balancing: balanced load leaves the bias bit-identical;
    otherwise each bias moves by exactly +-lambda (FP32) towards balance, the
    direction decided by the exact load against the mean (np.bincount)."""
    E, k, lam = 60, 4, np.float32(1e-3)
    g = rng(40)
    bias = g.standard_normal(E).astype(np.float32)
    T = 60
    idx = ((np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    nb, load = ora.bias_update(idx, bias, E, float(lam))
    assert np.array_equal(load, np.full(E, 4)) and np.array_equal(nb.view(np.int32), bias.view(np.int32))
    T = 333
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:50, 0] = 7                                            # make expert 7 overloaded
    idx[:50] = np.where((idx[:50] == 7) & (np.arange(k) > 0), (idx[:50] + 1) % E, idx[:50])
    nb, load = ora.bias_update(idx, bias, E, float(lam))
    cnt = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(load, cnt)
    mean = Fraction(T * k, E)
    for e in range(E):
        want = bias[e] + lam if cnt[e] < mean else (bias[e] - lam if cnt[e] > mean else bias[e])
        assert nb[e] == np.float32(want)
    assert nb[7] == np.float32(bias[7] - lam)
    # all load on two experts of four
    nb, _ = ora.bias_update(np.array([[0, 1]] * 10, np.int32), np.zeros(4, np.float32), 4, 0.5)
    assert list(nb) == [-0.5, -0.5, 0.5, 0.5]
    with pytest.raises(ValueError):
        ora.bias_update(np.array([[0, 4]], np.int32), np.zeros(4, np.float32), 4)


def test_drop_pad_capacity_pin(ora):
    import math
    for T, k, E in [(2048, 4, 60), (8192, 4, 60), (1, 4, 60), (7, 2, 3), (100, 1, 100)]:
        assert ora.capacity(T, k, E) == math.ceil(Fraction(3, 2) * T * k / E)
    assert ora.capacity(2048, 4, 60) == 205


def test_drop_pad_pins(ora):
    """Drop-and-pad against a sort-based construction (np.flatnonzero per
    expert), and against the dropless count sort when nothing overflows."""
    g = rng(41)
    E, k, T = 12, 3, 50
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:20, 0] = 5                                   # expert 5 over capacity
    idx[:20] = np.where((idx[:20] == 5) & (np.arange(k) > 0), (idx[:20] + 1) % E, idx[:20])
    C = ora.capacity(T, k, E)
    buf, offs, perm, inv = ora.drop_pad(idx, E, C)
    flat = idx.ravel()
    kept_total = 0
    for e in range(E):
        ids = np.flatnonzero(flat == e)               # assignment ids in token order
        kept = ids[:C]
        assert np.array_equal(buf[e, :len(kept)], kept) and np.all(buf[e, len(kept):] == -1)
        assert offs[e] == kept_total and np.array_equal(perm[kept_total:kept_total + len(kept)], kept)
        assert np.array_equal(inv[kept], kept_total + np.arange(len(kept)))
        assert np.all(inv[ids[C:]] == -1)
        kept_total += len(kept)
    assert offs[E] == kept_total and np.all(perm[kept_total:] == -1)
    assert (flat == 5).sum() > C and kept_total < T * k      # something was dropped
    # capacity above every load: the dropless count sort
    ro, rp, ri = ora.route(idx, E)
    buf, offs, perm, inv = ora.drop_pad(idx, E, T * k)
    assert np.array_equal(offs, ro) and np.array_equal(perm, rp) and np.array_equal(inv, ri)
    # capacity 0 drops everything
    buf, offs, perm, inv = ora.drop_pad(idx, E, 0)
    assert buf.size == 0 and np.all(offs == 0) and np.all(perm == -1) and np.all(inv == -1)


def test_fake_quant_forward_pins(ora):
    """Forward equals the eq. (6) codes of the quantisers times their scales
    (weights: b=4, group 32; activations: b=8, one group per row); error at
    most s/2 except a clipped positive maximum."""
    w = _crafted_weights()
    q, s = ora.quant_w4g32(w)
    want = (np.repeat(s, 32, axis=1) * q.astype(np.float32)).astype(np.float32)
    wb = ora.fake_quant(w, 4, 32)
    assert np.array_equal(wb, want)
    assert np.all(wb[0, :32] == 0.0)
    x = (rng(42).standard_normal((9, 200)) * 3).astype(np.float32)
    x[3] = 0.0
    qa, sa = ora.quant_act_i8(x)
    xb = ora.fake_quant(x, 8, 200)
    assert np.array_equal(xb, (sa[:, None] * qa.astype(np.float32)).astype(np.float32))
    err = np.abs(xb.astype(np.float64) - x)
    clipped = (xb == (sa[:, None] * np.float32(127)).astype(np.float32)) & (x > 0)
    assert np.all(err[~clipped] <= sa[:, None].repeat(200, 1)[~clipped] * 0.5 * (1 + 1e-6))
    with pytest.raises(ValueError):
        ora.fake_quant(x, 5, 200)


def test_fake_quant_ste_against_torch(ora):
    """Straight-through gradient against torch's per-channel fake quantiser
    (autograd), one channel per group of 32, scale s_g, zero point 0, range
    [-8, 7]; all-zero groups pass the gradient.  torch scales by the
    reciprocal where eq. (6) divides; the two quotients round differently
    only at a group maximum, whose quotient lies within an ulp of 7.5, and
    those entries are compared with the division's own decision instead."""
    import torch
    g = rng(43)
    w = (g.standard_normal((64, 256)) * 0.05).astype(np.float32)
    # groups whose positive maximum sits exactly on 7.5 * s or just off it
    w[0, :32] = np.linspace(-0.7, 1.0, 32, dtype=np.float32)
    w[1, :32] = np.linspace(-1.0, 0.9, 32, dtype=np.float32)
    w[2, 32:64] = 0.0
    gout = g.standard_normal(w.shape).astype(np.float32)
    wb, gin = ora.fake_quant(w, 4, 32, gout)
    _, s = ora.quant_w4g32(w)
    xs = torch.from_numpy(w.reshape(-1, 32)).requires_grad_(True)
    sc = torch.from_numpy(s.reshape(-1).copy())
    nz = sc > 0
    sc_t = torch.where(nz, sc, torch.ones_like(sc))
    y = torch.fake_quantize_per_channel_affine(xs, sc_t, torch.zeros_like(sc, dtype=torch.int32), 0, -8, 7)
    y.backward(torch.from_numpy(gout.reshape(-1, 32)))
    gt = xs.grad.numpy().copy()
    gt[~nz.numpy()] = gout.reshape(-1, 32)[~nz.numpy()]
    q_div = np.rint(w.reshape(-1, 32) / np.where(s.reshape(-1, 1) > 0, s.reshape(-1, 1), 1)).astype(np.float32)
    q_mul = np.rint(w.reshape(-1, 32) * (np.float32(1) / np.where(s.reshape(-1, 1) > 0, s.reshape(-1, 1), 1)).astype(np.float32))
    same = q_div == q_mul
    gm = np.abs(w.reshape(-1, 32)).max(1, keepdims=True)
    is_max = np.abs(w.reshape(-1, 32)) == gm
    assert np.all(is_max[~same])
    assert np.array_equal(gin.reshape(-1, 32)[same], gt[same])
    assert np.array_equal(wb.reshape(-1, 32)[same], y.detach().numpy()[same])
    # at the excluded maxima the gradient passes iff the quotient rounds into range
    g_div = np.where(q_div <= 7, gout.reshape(-1, 32), 0.0)
    assert np.array_equal(gin.reshape(-1, 32)[~same], g_div[~same])
    clipped = (gin == 0) & (gout != 0)
    # only positive group maxima are ever clipped, and they are (a quotient
    # at or above 7.5 is common: s is rounded to FP32)
    assert np.all((is_max & (w.reshape(-1, 32) > 0))[clipped.reshape(-1, 32)])
    assert clipped.sum() > 10


def _expert_case(g, E=3, d=64, h=32, counts=(5, 0, 7)):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    xs = g.standard_normal((R, d)).astype(np.float32)
    wgu = (g.standard_normal((E, 2 * h, d)) * 0.2).astype(np.float32)
    wd = (g.standard_normal((E, d, h)) * 0.2).astype(np.float32)
    return offs, xs, wgu, wd


def _act32(ora, gu, h):
    g, u = gu[:, :h], gu[:, h:]
    return ((g / (np.float32(1) + ora.exp_ref(-g))).astype(np.float32) * u).astype(np.float32)


def test_expert_train_forward_pins(ora):
    """QAT expert forward: gate/up and down products equal float64 matrix
    products per expert; abar equals the pinned activation fake quantiser
    applied to the FP32 SwiGLU."""
    g = rng(50)
    offs, xs, wgu, wd = _expert_case(g)
    gu, abar, f = ora.expert_train_forward(offs, xs, wgu, wd)
    h = wgu.shape[1] // 2
    for e in range(len(offs) - 1):
        r0, r1 = offs[e], offs[e + 1]
        want = xs[r0:r1].astype(np.float64) @ wgu[e].astype(np.float64).T
        np.testing.assert_allclose(gu[r0:r1], want, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(f[r0:r1], abar[r0:r1].astype(np.float64) @ wd[e].astype(np.float64).T,
                                   rtol=1e-6, atol=1e-6)
    assert np.array_equal(abar, ora.fake_quant(_act32(ora, gu, h), 8, h))


def test_expert_backward_against_autograd(ora):
    """QAT expert backward against torch autograd (float64) of the same
    forward, with the activation quantiser as a straight-through node whose
    values and pass mask come from the pinned fake quantiser; an expert
    without rows gets zero weight gradients."""
    import torch
    g = rng(51)
    offs, xs, wgu, wd = _expert_case(g)
    gu, abar, _ = ora.expert_train_forward(offs, xs, wgu, wd)
    h = wgu.shape[1] // 2
    a32 = _act32(ora, gu, h)
    # planted clips: make some rows' maximum exactly hit the clamp path
    _, pass_ = ora.fake_quant(a32, 8, h, np.ones_like(a32))
    df = g.standard_normal((xs.shape[0], xs.shape[1])).astype(np.float32)
    dxs, dwgu, dwd = ora.expert_backward(offs, xs, wgu, wd, gu, df)
    X = torch.tensor(xs, dtype=torch.float64, requires_grad=True)
    Wg = torch.tensor(wgu, dtype=torch.float64, requires_grad=True)
    Wd = torch.tensor(wd, dtype=torch.float64, requires_grad=True)
    loss = 0.0
    for e in range(len(offs) - 1):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 == r0:
            continue
        GU = X[r0:r1] @ Wg[e].T
        G, U = GU[:, :h], GU[:, h:]
        A = G * torch.sigmoid(G) * U
        Ab = torch.tensor(abar[r0:r1], dtype=torch.float64) + (A - A.detach()) * torch.tensor(pass_[r0:r1], dtype=torch.float64)
        F = Ab @ Wd[e].T
        loss = loss + (F * torch.tensor(df[r0:r1], dtype=torch.float64)).sum()
    loss.backward()
    np.testing.assert_allclose(dxs, X.grad.numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dwgu, Wg.grad.numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dwd, Wd.grad.numpy(), rtol=1e-9, atol=1e-9)
    assert np.all(dwgu[1] == 0) and np.all(dwd[1] == 0)
    assert (pass_ == 0).sum() >= 1          # some row maximum clips


@pytest.mark.parametrize("gating", [0, 1, 2, 3])
def test_router_backward_against_autograd(ora, gating):
    """Router backward against torch autograd (float64) of the gate and the
    z-loss: y_t = sum_j w_tj f_tj with the expert outputs held fixed,
    loss = sum y . dy + (lambda_z / T) sum_t lse(z_t)^2; dropped assignments
    contribute nothing; the bias gets no gradient."""
    import torch
    g = rng(60 + gating)
    T, d, E, k = 9, 32, 12, 3
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.3).astype(np.float32)
    bias = g.standard_normal(E).astype(np.float32)
    z_sel = x.astype(np.float64) @ wr.T.astype(np.float64) + bias
    idx = np.argsort(-z_sel, axis=1, kind="stable")[:, :k].astype(np.int32)
    inv = g.permutation(T * k).astype(np.int32)
    inv[[2, 7]] = -1                                   # two dropped assignments
    f = g.standard_normal((T * k, d)).astype(np.float32)
    dy = g.standard_normal((T, d)).astype(np.float32)
    lz = 0.05
    dz, dwr, dx = ora.router_backward(x, wr, bias, idx, f, inv, dy, gating, lz)
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W = torch.tensor(wr, dtype=torch.float64, requires_grad=True)
    Z = X @ W.T + (0.0 if gating & 2 else torch.tensor(bias, dtype=torch.float64))
    Z.retain_grad()
    I = torch.tensor(idx, dtype=torch.int64)
    if gating & 1:
        s = torch.sigmoid(Z).gather(1, I)
        wts = s / s.sum(1, keepdim=True)
    else:
        wts = torch.softmax(Z, 1).gather(1, I)
    fr = torch.tensor(np.where(inv[:, None] >= 0, f[np.maximum(inv, 0)], 0.0), dtype=torch.float64).reshape(T, k, d)
    y = (wts[:, :, None] * fr).sum(1)
    loss = (y * torch.tensor(dy, dtype=torch.float64)).sum() + lz / T * (torch.logsumexp(Z, 1) ** 2).sum()
    loss.backward()
    np.testing.assert_allclose(dz, Z.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dwr, W.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dx, X.grad.numpy(), rtol=1e-9, atol=1e-12)
