"""GPU parity of the HIP path (called through the C ABI) against the CPU
oracle, stage by stage and end to end, on seeded synthetic inputs.

Bars: bit-exact for integer work (weight codes and scales, activation codes
and scales, top-k ids, routing offsets / permutation, int32 group sums).  The
INT4/INT8 path fixes its FP32 operation order (scale fma chain over groups,
SwiGLU with the shared-method exponential, softmax tree, combine fma chain), so
its gate weights, hidden codes, expert outputs and y are compared bit for bit
as well.  FP32- and BF16-weight paths: per token row max|gpu - oracle| /
max|oracle| <= 1e-3 (FP32 output) or 2e-2 (BF16 output)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_ffn_amd import binding as B
from sparse_moe_ffn_amd import workloads as wl
from gpu_util import (DEV, bf16_bits_to_f32, decode_f16_paired, decode_prepacked, layer_output,
                      make_layer, np_, oracle_forward, row_rel_err, unpack_canonical)

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-3, 2e-2


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ------------------------------------------------------------ weights: eq. (6)
@pytest.mark.parametrize("n,rows,cols", [(1, 32, 32), (3, 64, 128), (2, 768, 384)])
def test_quantize_and_prepack_bitexact(n, rows, cols):
    g = rng(100 + rows)
    w = (g.standard_normal((n, rows, cols)) * 0.02).astype(np.float32)
    w[0, 0, :32] = 0.0                                      # all-zero group
    w[0, 1, :32] = np.linspace(-1, 1, 32, dtype=np.float32)  # exact +-max
    qc = torch.empty((n * rows, cols // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((n * rows, cols // 32), dtype=torch.float32, device=DEV)
    B.quantize_int4g32(n * rows, cols, dev(w), qc, sc)
    q_ref, s_ref = oracle.quant_w4g32(w.reshape(n * rows, cols))
    assert np.array_equal(unpack_canonical(np_(qc)), q_ref)
    assert np.array_equal(np_(sc), s_ref)
    qp = torch.empty((n * B.prepacked_bytes(rows, cols),), dtype=torch.uint8, device=DEV)
    sp = torch.empty((n * B.prepacked_scale_bytes(rows, cols) // 4,), dtype=torch.float32, device=DEV)
    B.prepack_int4g32(n, rows, cols, qc, sc, qp, sp)
    q2, s2 = decode_prepacked(np_(qp), np_(sp), n, rows, cols)
    assert np.array_equal(q2.reshape(n * rows, cols), q_ref)
    assert np.array_equal(s2.reshape(n * rows, -1), s_ref)


# ------------------------------------------------------------ activations
@pytest.mark.parametrize("rows,cols", [(1, 64), (333, 768), (64, 1280), (5, 2560)])
def test_act_quant_bitexact(rows, cols):
    x = rng(rows).standard_normal((rows, cols)).astype(np.float32)
    x[0, :] = 0.0
    if rows > 2:
        x[2] *= 1e-20
    q = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
    s = torch.empty((rows,), dtype=torch.float32, device=DEV)
    B.act_quant_i8(rows, cols, dev(x), q, s)
    q_ref, s_ref = oracle.quant_act_i8(x)
    assert np.array_equal(np_(q), q_ref)
    assert np.array_equal(np_(s), s_ref)


def halfway_rows(cols, amaxes, seed):
    """Rows whose entries sit on and next to the rounding boundaries of the
    INT8 rule: fl((k + 1/2) * s) and its neighbours 1 and 2 ulps away, for
    every k with |k + 1/2| <= 126.5, s = fl(2 * amax / 255), amax the row's
    first entry (the rest random below it)."""
    g = rng(seed)
    rows = []
    for A in amaxes:
        A = np.float32(A)
        s = np.float32(np.float32(2.0) * A) / np.float32(255.0)
        mid = (np.arange(-127, 127, dtype=np.float32) + np.float32(0.5)) * s
        vals = [mid]
        for n in (1, 2):
            up, dn = mid.copy(), mid.copy()
            for _ in range(n):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            vals += [up, dn]
        v = np.concatenate(vals).astype(np.float32)
        v = v[np.abs(v) <= A]
        row = (g.uniform(-1, 1, cols) * A * 0.9).astype(np.float32)
        m = min(cols - 1, v.size)
        row[1:1 + m] = v[:m]
        row[0] = A
        g.shuffle(row[1:])
        rows.append(row)
    return np.stack(rows)


# Quotients on or within two ulps of a half-integer (the codes there depend on
# the exact FP32 quotient), tiny rows (scale below 2^-100) and a subnormal row.
@pytest.mark.parametrize("cols", [768, 1536])
def test_act_quant_halfway_bitexact(cols):
    x = halfway_rows(cols, [1.0, 3.7, 1e-3, 123.456, 2.5e-30, 7e-36, 0.1, 5e4, 1.1754944e-38 * 3], 7)
    rows = x.shape[0]
    q_ref, s_ref = oracle.quant_act_i8(x)
    for layout in (B.MM_ACT_ROW_MAJOR, B.MM_ACT_GROUP_MAJOR, B.MM_ACT_F16_PAIRED):
        f16 = layout == B.MM_ACT_F16_PAIRED
        q = torch.empty((rows, cols), dtype=torch.int16 if f16 else torch.int8, device=DEV)
        s = torch.empty((rows,), dtype=torch.float32, device=DEV)
        B.act_quant_i8_layout(rows, cols, dev(x), q, s, layout)
        qh = np_(q)
        if layout == B.MM_ACT_GROUP_MAJOR:  # byte (g * rows + r) * 32 + c % 32
            qh = qh.reshape(cols // 32, rows, 32).transpose(1, 0, 2).reshape(rows, cols)
        elif f16:
            qh = decode_f16_paired(qh, cols)
        assert np.array_equal(s_ref, np_(s))
        assert np.array_equal(qh, q_ref)


# ------------------------------------------------------------ dense W4A8 linear
@pytest.mark.parametrize("rows,K,N", [
    (1, 768, 256), (7, 768, 768), (8, 1280, 256),    # weight-streaming (decode rows)
    (9, 768, 256), (64, 1280, 256),                  # matrix cores from 9 rows
    (65, 1024, 1024), (300, 1280, 1280), (2048, 768, 768), (130, 3072, 640),
    (3, 3072, 128),                                    # row-tile kernel (K beyond the streaming form)
])
def test_linear_w4a8_bitexact(rows, K, N):
    """mm_linear_w4a8 (an attention / embedding projection in W4A8) against the
    oracle's linear, bit for bit, from device-quantised weights and rows."""
    from sparse_moe_ffn_amd.layer import prepare_weight
    g = rng(rows * 7 + K + N)
    x = g.standard_normal((rows, K)).astype(np.float32)
    wt = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xq_ref, sx_ref = oracle.quant_act_i8(x)
    wq_ref, ws_ref = oracle.quant_w4g32(wt)
    y_ref = oracle.linear_w4a8(xq_ref, sx_ref, wq_ref, ws_ref)
    dw = prepare_weight(wt, "int4g32", DEV)
    xq = torch.empty((rows, K), dtype=torch.int8, device=DEV)
    sx = torch.empty((rows,), dtype=torch.float32, device=DEV)
    B.act_quant_i8(rows, K, dev(x), xq, sx)
    y = torch.empty((rows, N), dtype=torch.float32, device=DEV)
    B.linear_w4a8(rows, K, N, xq, sx, dw.c(), y)
    assert np.array_equal(np_(y), y_ref)


@pytest.mark.parametrize("rows", [1, 65])
def test_linear_w4a8_tiny_scales(rows):
    """Weight groups whose scale s falls below 2^-122 (the prepacked s / 16 is
    then subnormal, include/mobmoe.h): every output column whose groups all
    have s >= 2^-122 stays bit-exact; the columns with tiny groups stay within
    the documented rounding of s / 16 (2^-149 / (s / 16) relative per group)."""
    from sparse_moe_ffn_amd.layer import prepare_weight
    K, N = 768, 256
    g = rng(4242 + rows)
    x = g.standard_normal((rows, K)).astype(np.float32)
    wt = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    wt[0] *= np.float32(5e-36)       # s about 1.3e-38: s / 16 subnormal
    wt[1, :32] *= np.float32(5e-36)  # one tiny group in an otherwise normal row
    wt[2] *= np.float32(2.0 ** -110)  # s about 2^-114: exact
    xq_ref, sx_ref = oracle.quant_act_i8(x)
    wq_ref, ws_ref = oracle.quant_w4g32(wt)
    assert ws_ref[0].max() < 2.0 ** -122 and ws_ref[2].min() > 2.0 ** -122
    y_ref = oracle.linear_w4a8(xq_ref, sx_ref, wq_ref, ws_ref)
    dw = prepare_weight(wt, "int4g32", DEV)
    xq = torch.empty((rows, K), dtype=torch.int8, device=DEV)
    sx = torch.empty((rows,), dtype=torch.float32, device=DEV)
    B.act_quant_i8(rows, K, dev(x), xq, sx)
    yd = torch.empty((rows, N), dtype=torch.float32, device=DEV)
    B.linear_w4a8(rows, K, N, xq, sx, dw.c(), yd)
    y = np_(yd)
    tiny = (ws_ref < 2.0 ** -122).any(axis=1)
    assert list(np.flatnonzero(tiny)) == [0, 1]
    assert np.array_equal(y[:, ~tiny], y_ref[:, ~tiny])
    for c in (0, 1):
        err = np.abs(y[:, c].astype(np.float64) - y_ref[:, c]).max()
        assert err <= 1e-5 * np.abs(y_ref[:, c]).max() + 2.0 ** -149


# ------------------------------------------------------------ GQA decode attention, INT8 KV cache
def _quant_rows_i8(x):
    """Cache contents for float vectors [..., 64] by the oracle's INT8 row rule."""
    q, s = oracle.quant_act_i8(x.reshape(-1, x.shape[-1]))
    return q.reshape(x.shape), s.reshape(x.shape[:-1])


@pytest.mark.parametrize("B_,nh,nkv,maxT,lens", [
    (1, 12, 4, 64, [1]),                         # S heads, one position
    (2, 12, 4, 300, [300, 17]),                  # ragged lengths, partial chunks
    (3, 16, 4, 1024, [1000, 256, 257]),          # M heads, chunk edges
    (1, 20, 4, 8192, [8192]),                    # L heads at the 8K context
    (4, 8, 8, 128, [5, 128, 64, 0]),             # one query head per key/value head; empty row
])
def test_attn_decode_i8(B_, nh, nkv, maxT, lens):
    """mm_attn_decode_i8 against the oracle's double evaluation per sequence;
    per (sequence, head) row max|gpu - oracle| / max|oracle| <= 1e-4."""
    g = rng(sum(lens) + nh)
    q = g.standard_normal((B_, nh, 64)).astype(np.float32)
    kf = g.standard_normal((B_, nkv, maxT, 64)).astype(np.float32)
    vf = g.standard_normal((B_, nkv, maxT, 64)).astype(np.float32)
    kq, ks = _quant_rows_i8(kf)
    vq, vs = _quant_rows_i8(vf)
    max_len = max(max(lens), 1)
    ws_bytes = B.attn_workspace_bytes(B_, nkv, max_len)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=DEV)
    out = torch.empty((B_, nh, 64), dtype=torch.float32, device=DEV)
    lens_d = dev(np.array(lens, np.int32))
    B.attn_decode_i8(B_, nh, nkv, 64, maxT, max_len, lens_d, dev(q), dev(kq), dev(vq), dev(ks),
                     dev(vs), out, ws, ws_bytes)
    got = np_(out)
    for b in range(B_):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0)
            continue
        ref = oracle.attn_decode(q[b:b + 1], kq[b:b + 1], vq[b:b + 1], ks[b:b + 1], vs[b:b + 1],
                                 lens[b])[0]
        err = np.abs(got[b] - ref).max(1) / np.abs(ref).max(1)
        assert err.max() <= 1e-4, (b, err.max())


def test_kv_append_i8_bitexact():
    """mm_kv_append_i8 writes each new vector's codes and scale (the oracle's
    INT8 row rule) at its sequence's position and nothing else."""
    g = rng(31)
    B_, nkv, maxT = 3, 4, 50
    kn = g.standard_normal((B_, nkv, 64)).astype(np.float32)
    vn = g.standard_normal((B_, nkv, 64)).astype(np.float32)
    vn[1, 2] = 0.0                                           # an all-zero vector: scale 0, codes 0
    pos = np.array([0, 37, 49], np.int32)
    kc = torch.full((B_, nkv, maxT, 64), 77, dtype=torch.int8, device=DEV)
    vc = torch.full((B_, nkv, maxT, 64), 77, dtype=torch.int8, device=DEV)
    ksd = torch.full((B_, nkv, maxT), -1.0, dtype=torch.float32, device=DEV)
    vsd = torch.full((B_, nkv, maxT), -1.0, dtype=torch.float32, device=DEV)
    B.kv_append_i8(B_, nkv, 64, maxT, dev(pos), dev(kn), dev(vn), kc, vc, ksd, vsd)
    kq, ks = _quant_rows_i8(kn)
    vq, vs = _quant_rows_i8(vn)
    kch, vch, ksh, vsh = np_(kc), np_(vc), np_(ksd), np_(vsd)
    for b in range(B_):
        assert np.array_equal(kch[b, :, pos[b]], kq[b]) and np.array_equal(vch[b, :, pos[b]], vq[b])
        assert np.array_equal(ksh[b, :, pos[b]], ks[b]) and np.array_equal(vsh[b, :, pos[b]], vs[b])
        others = [t for t in range(maxT) if t != pos[b]]
        assert np.all(kch[b, :, others] == 77) and np.all(ksh[b, :, others] == -1.0)
    # positions outside the cache are skipped
    before = np_(kc).copy()
    B.kv_append_i8(B_, nkv, 64, maxT, dev(np.array([-1, maxT, maxT + 5], np.int32)), dev(kn),
                   dev(vn), kc, vc, ksd, vsd)
    assert np.array_equal(np_(kc), before)


# ------------------------------------------------------------ router
@pytest.mark.parametrize("T,d,E,k,use_bias,gating", [
    (1000, 768, 60, 4, False, 0), (257, 1280, 60, 4, True, 0), (33, 64, 8, 2, False, 0),
    (130, 256, 60, 4, False, 0), (64, 1024, 64, 8, True, 0), (77, 768, 60, 4, True, 1),
    (5, 3072, 60, 4, False, 0),
    # decode batches (one workgroup per token)
    (1, 768, 60, 4, False, 0), (8, 1280, 60, 4, True, 0), (64, 768, 60, 4, True, 1),
    (3, 256, 33, 3, False, 0)])
def test_router_bitexact(T, d, E, k, use_bias, gating):
    g = rng(T + d)
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = wl.zipf_bias(wl.WORKLOADS["l_prefill"].with_(E=E)) if use_bias else None
    ds = B.desc(d, E, 64, 0, k, "int4g32", gating)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.router_topk(ds, T, dev(x), dev(wr), None if bias is None else dev(bias), idx, wt)
    i_ref, w_ref, _ = oracle.router(x, wr, bias, k=k, gating=gating)
    assert np.array_equal(np_(idx), i_ref)
    assert np.array_equal(np_(wt), w_ref.astype(np.float32))


def test_router_ties_pick_lowest_index():
    g = rng(7)
    T, d, E, k = 50, 256, 60, 4
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = np.tile((g.standard_normal(d) * 0.02).astype(np.float32), (E, 1))
    ds = B.desc(d, E, 64, 0, k)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    wt = torch.empty((T, k), dtype=torch.float32, device=DEV)
    B.router_topk(ds, T, dev(x), dev(wr), None, idx, wt)
    assert np.all(np_(idx) == np.arange(k))
    np.testing.assert_allclose(np_(wt), 1 / E, rtol=1e-6)


# ------------------------------------------------------------ routing
@pytest.mark.parametrize("T,E,k,skew", [(3000, 60, 4, False), (2048, 60, 4, True), (1, 60, 4, False),
                                         (513, 1, 1, False), (100, 64, 8, True), (8192, 60, 4, True),
                                         (400, 60, 4, False)])  # one workgroup for 257..2048 slots, else one block or two kernels
def test_route_permute_bitexact(T, E, k, skew):
    g = rng(T * 7 + E)
    if skew:
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
        p /= p.sum()
        idx = np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ds = B.desc(64, E, 64, 0, k)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    inv = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    nb = B.workspace_bytes(ds, T, B.MM_WS_ROUTE)
    ws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    B.route_permute(ds, T, dev(idx), off, perm, inv, ws, nb)
    o_ref, p_ref, i_ref = oracle.route(idx, E)
    assert np.array_equal(np_(off), o_ref)
    assert np.array_equal(np_(perm), p_ref)
    assert np.array_equal(np_(inv), i_ref)


# ------------------------------------------------------------ training side
def _skewed_ids(g, T, E, k):
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    p /= p.sum()
    return np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(2048, 60, 4), (1, 60, 4), (65536, 60, 4), (15, 4, 2)])
def test_bias_update_bitexact(T, E, k):
    """mm_bias_update: loads and updated biases bit-identical to the oracle."""
    g = rng(T + E)
    idx = _skewed_ids(g, T, E, k)
    bias = g.standard_normal(E).astype(np.float32)
    bd = dev(bias)
    load = torch.empty((E,), dtype=torch.int32, device=DEV)
    B.bias_update(T, E, k, dev(idx), 1e-3, bd, load)
    ref, ref_load = oracle.bias_update(idx, bias, E, 1e-3)
    assert np.array_equal(np_(load), ref_load)
    assert np.array_equal(np_(bd).view(np.int32), ref.view(np.int32))
    # balanced routing: biases unchanged
    idx = ((np.arange(E)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    bd = dev(bias)
    B.bias_update(E, E, k, dev(idx), 1e-3, bd)
    assert np.array_equal(np_(bd).view(np.int32), bias.view(np.int32))


@pytest.mark.parametrize("T,E,k", [(2048, 60, 4), (8192, 60, 4), (3, 60, 4), (37, 8, 2)])
def test_drop_pad_bitexact(T, E, k):
    """mm_drop_pad after mm_route_permute: padded table and kept routing
    bit-identical to the oracle at capacity factor 1.5, 0, 1 and above every load."""
    g = rng(T * 3 + E)
    idx = _skewed_ids(g, T, E, k)
    ds = B.desc(64, E, 64, 0, k)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    inv = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    nb = B.workspace_bytes(ds, T, B.MM_WS_ROUTE)
    ws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    idx_d = dev(idx)
    B.route_permute(ds, T, idx_d, off, perm, inv, ws, nb)
    cap = B.drop_pad_capacity(T, k, E)
    assert cap == oracle.capacity(T, k, E)
    dropped_some = False
    for C in [cap, 0, 1, T * k]:
        buf = torch.full((max(E * C, 1),), 7, dtype=torch.int32, device=DEV)
        offc = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
        permc = torch.full((T * k,), 7, dtype=torch.int32, device=DEV)
        invc = torch.full((T * k,), 7, dtype=torch.int32, device=DEV)
        B.drop_pad(T, E, k, C, idx_d, off, perm, inv, buf, offc, permc, invc)
        rb, ro, rp, ri = oracle.drop_pad(idx, E, C)
        assert np.array_equal(np_(buf)[:E * C], rb.ravel()), C
        assert np.array_equal(np_(offc), ro), C
        assert np.array_equal(np_(permc), rp), C
        assert np.array_equal(np_(invc), ri), C
        dropped_some |= C == cap and ro[E] < T * k
    if T >= 2048:
        assert dropped_some          # the skewed routing overflows some expert at factor 1.5


@pytest.mark.parametrize("rows,cols,bits,group", [(4096, 384, 4, 32), (771, 768, 4, 32),
                                                  (2053, 768, 8, 768), (5, 4, 8, 4),
                                                  (64, 1536, 4, 1536), (8, 32, 8, 32)])
def test_fake_quant_bitexact(rows, cols, bits, group):
    """mm_fake_quant forward and straight-through backward bit-identical to
    the oracle, with all-zero groups, exact +-maxima and tiny values."""
    g = rng(rows + cols + bits)
    x = (g.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    x[0, :min(group, cols)] = 0.0
    if rows > 2:
        x[1, :min(32, cols)] = np.linspace(-1, 1, min(32, cols), dtype=np.float32)
        x[2, :min(32, cols)] = 1e-30
    go = g.standard_normal((rows, cols)).astype(np.float32)
    xb = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    gi = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    xd, god = dev(x), dev(go)
    B.fake_quant(rows, cols, bits, group, xd, xb, god, gi)
    rxb, rgi = oracle.fake_quant(x, bits, group, go)
    assert np.array_equal(np_(xb).view(np.int32), rxb.view(np.int32))
    assert np.array_equal(np_(gi).view(np.int32), rgi.view(np.int32))
    assert (rgi == 0).sum() > 0 or bits == 8     # some positive maxima clip at b = 4
    # forward only, and backward only
    xb2 = torch.empty_like(xb)
    B.fake_quant(rows, cols, bits, group, xd, xb2)
    assert torch.equal(xb2, xb)
    gi2 = torch.empty_like(gi)
    B.fake_quant(rows, cols, bits, group, xd, None, god, gi2)
    assert torch.equal(gi2, gi)


def _expert_rows_case(g, E, d, h, counts):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offs[-1])
    xs = (g.standard_normal((R, d))).astype(np.float32)
    wgu = (g.standard_normal((E, 2 * h, d)) * (1.0 / np.sqrt(d))).astype(np.float32)
    wd = (g.standard_normal((E, d, h)) * (1.0 / np.sqrt(h))).astype(np.float32)
    return offs, xs, wgu, wd


def _row_rel(got, ref):
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    got = got.reshape(ref.shape).astype(np.float64)
    den = np.maximum(np.abs(ref).max(1), 1e-30)
    return np.abs(got - ref).max(1) / den


EXPERT_SHAPES = [(3, 64, 32, [5, 0, 70]), (60, 768, 384, None), (4, 128, 1536 // 4, [0, 1, 129, 64]),
                 (1, 768, 1536, [197])]          # the S shared expert: one group of every token


@pytest.mark.parametrize("E,d,h,counts", EXPERT_SHAPES)
def test_expert_train_forward(E, d, h, counts):
    """mm_expert_train_forward_f32 against the oracle: gate/up and down
    products within 1e-4 per row.  The INT8 activation codes are decided on
    FP32 products on the device and double products in the oracle, so a code
    whose quotient lies within FP32 rounding of a half-integer may differ by
    one step (the derived bound of the fake-quantised training activations):
    at most 0.1 % of the codes (and at least 2 allowed), each within one step
    s_r of the oracle's value; rows without such a code get 1e-4 on f, rows
    with one get 1e-4 of the row maximum plus one step times the sum of
    |W_d| over the flipped columns."""
    g = rng(E + d + h)
    if counts is None:
        counts = list(np.bincount(_skewed_ids(g, 150, E, 4).ravel(), minlength=E))
    offs, xs, wgu, wd = _expert_rows_case(g, E, d, h, counts)
    R = xs.shape[0]
    gu = torch.empty((R, 2 * h), device=DEV)
    ab = torch.empty((R, h), device=DEV)
    f = torch.empty((R, d), device=DEV)
    B.expert_train_forward_f32(E, d, h, R, dev(offs), dev(xs), dev(wgu), dev(wd), gu, ab, f)
    rgu, rab, rf = oracle.expert_train_forward(offs, xs, wgu, wd)
    assert _row_rel(np_(gu), rgu).max() <= 1e-4
    gab = np_(ab)
    s = (2.0 * np.abs(rab).max(1) / 255.0).astype(np.float32)  # an upper bound of each row's step
    # the row scale follows the row's FP32 products, so s * code may differ
    # in its last bits everywhere; a code that differs moves by a whole step
    rowmax = np.maximum(np.abs(rab).max(1, keepdims=True), 1e-30)
    diff = np.abs(gab.astype(np.float64) - rab) > 1e-4 * rowmax
    assert diff.sum() <= max(2, diff.size // 1000)
    assert np.all(np.abs(gab - rab)[diff] <= 1.01 * np.repeat(np.maximum(s, 1e-30)[:, None], h, 1)[diff])
    flip_rows = diff.any(1)
    err = _row_rel(np_(f), rf)
    assert err[~flip_rows].max(initial=0) <= 1e-4
    # a flipped code j of row r moves f[r][c] by one step s_r times |wd_e[c][j]|
    gf = np_(f).astype(np.float64)
    expert_of = np.repeat(np.arange(E), counts)
    for r in np.flatnonzero(flip_rows):
        js = np.flatnonzero(diff[r])
        bound = 1e-4 * np.abs(rf[r]).max() + 1.01 * s[r] * np.abs(wd[expert_of[r]][:, js]).sum(1)
        assert np.all(np.abs(gf[r] - rf[r]) <= bound), r


@pytest.mark.parametrize("E,d,h,counts", EXPERT_SHAPES)
def test_expert_backward(E, d, h, counts):
    """mm_expert_backward_f32 against the oracle's double backward on the
    oracle's own forward state: dxs per row and every expert's weight
    gradients within 1e-4 (of the row / matrix maximum); zero for experts
    without rows."""
    g = rng(E * 3 + d + h)
    if counts is None:
        counts = list(np.bincount(_skewed_ids(g, 150, E, 4).ravel(), minlength=E))
    offs, xs, wgu, wd = _expert_rows_case(g, E, d, h, counts)
    R = xs.shape[0]
    rgu, rab, _ = oracle.expert_train_forward(offs, xs, wgu, wd)
    df = g.standard_normal((R, d)).astype(np.float32)
    rdx, rdwgu, rdwd = oracle.expert_backward(offs, xs, wgu, wd, rgu, df)
    dx = torch.empty((R, d), device=DEV)
    dwgu = torch.full((E, 2 * h, d), 7.0, device=DEV)
    dwd = torch.full((E, d, h), 7.0, device=DEV)
    wsb = B.expert_backward_workspace_bytes(R, h)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=DEV)
    B.expert_backward_f32(E, d, h, R, dev(offs), dev(xs), dev(wgu), dev(wd), dev(rgu), dev(rab),
                          dev(df), dx, dwgu, dwd, ws, wsb)
    assert _row_rel(np_(dx), rdx).max() <= 1e-4
    gw, gd = np_(dwgu), np_(dwd)
    for e in range(E):
        if counts[e] == 0:
            assert np.all(gw[e] == 0) and np.all(gd[e] == 0)
            continue
        for got, ref in ((gw[e], rdwgu[e]), (gd[e], rdwd[e])):
            assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max(), e


def test_expert_backward_zero_rows():
    """No kept rows at all (drop-and-pad with capacity 0 gives offsets of
    zeros): the call still writes zero weight gradients for every expert and
    touches no row buffer (those may be NULL)."""
    E, d, h = 3, 64, 32
    offs = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    g = rng(77)
    wgu = dev((g.standard_normal((E, 2 * h, d)) * 0.02).astype(np.float32))
    wd = dev((g.standard_normal((E, d, h)) * 0.02).astype(np.float32))
    dwgu = torch.full((E, 2 * h, d), 7.0, device=DEV)
    dwd = torch.full((E, d, h), 7.0, device=DEV)
    B.expert_backward_f32(E, d, h, 0, offs, None, wgu, wd, None, None, None, None, dwgu, dwd, None, 0)
    assert np.all(np_(dwgu) == 0) and np.all(np_(dwd) == 0)


def test_expert_training_full_size_sampled():
    """The S training step at T = 2048 in the launch configuration of
    bench.py --op train_step (routing with expert probability ~ rank^-0.3,
    capacity 1.5, compacted rows bounded by T*k): drop-and-pad exact on the
    whole batch; forward and backward of three whole experts (rows and weight
    gradients) against the oracle."""
    T, E, k, d, h = 2048, 60, 4, 768, 384
    g = rng(2048)
    p = np.arange(1, E + 1, dtype=np.float64) ** -0.3
    p = p[g.permutation(E)]
    p /= p.sum()
    idx = np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    ds = B.desc(d, E, h, 0, k)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    inv = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    nb = B.workspace_bytes(ds, T, B.MM_WS_ROUTE)
    rws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    idx_d = dev(idx)
    B.route_permute(ds, T, idx_d, off, perm, inv, rws, nb)
    C = B.drop_pad_capacity(T, k, E)
    buf = torch.empty((E * C,), dtype=torch.int32, device=DEV)
    offc = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    permc = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    invc = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    B.drop_pad(T, E, k, C, idx_d, off, perm, inv, buf, offc, permc, invc)
    rb, ro, rp, ri = oracle.drop_pad(idx, E, C)
    assert np.array_equal(np_(offc), ro) and np.array_equal(np_(permc), rp)
    assert np.array_equal(np_(invc), ri) and np.array_equal(np_(buf), rb.ravel())
    Tk = T * k
    x = g.standard_normal((T, d)).astype(np.float32)
    wgu = (g.standard_normal((E, 2 * h, d)) / np.sqrt(d)).astype(np.float32)
    wd = (g.standard_normal((E, d, h)) / np.sqrt(h)).astype(np.float32)
    xs = torch.empty((Tk, d), device=DEV)
    B.gather_rows(Tk, d, k, permc, None, dev(x), xs)
    gu = torch.empty((Tk, 2 * h), device=DEV)
    ab = torch.empty((Tk, h), device=DEV)
    f = torch.empty((Tk, d), device=DEV)
    B.expert_train_forward_f32(E, d, h, Tk, offc, xs, dev(wgu), dev(wd), gu, ab, f)
    df = g.standard_normal((Tk, d)).astype(np.float32)
    dxs = torch.empty((Tk, d), device=DEV)
    dwgu = torch.empty((E, 2 * h, d), device=DEV)
    dwd = torch.empty((E, d, h), device=DEV)
    wsb = B.expert_backward_workspace_bytes(Tk, h)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=DEV)
    # the backward runs on the oracle's forward state for the sampled experts
    ref_state = {}
    xs_h = x[np.maximum(rp, 0) // k]
    for e in (0, 17, 59):
        r0, r1 = int(ro[e]), int(ro[e + 1])
        o = np.array([0, r1 - r0], np.int32)
        ref_state[e] = (r0, r1, o) + oracle.expert_train_forward(o, xs_h[r0:r1], wgu[e:e + 1], wd[e:e + 1])
    gu_in = np_(gu).copy()
    ab_in = np_(ab).copy()
    for e, (r0, r1, o, rgu, rab, rf) in ref_state.items():
        assert _row_rel(gu_in[r0:r1], rgu).max() <= 1e-4
        gu_in[r0:r1], ab_in[r0:r1] = rgu, rab
        ferr = _row_rel(np_(f)[r0:r1], rf)
        diff = np.abs(np_(ab)[r0:r1].astype(np.float64) - rab) > 1e-4 * np.maximum(
            np.abs(rab).max(1, keepdims=True), 1e-30)
        assert diff.sum() <= max(2, diff.size // 1000)
        flips = diff.any(1)
        assert ferr[~flips].max(initial=0) <= 1e-4
        step = (2.0 * np.abs(rab).max(1) / 255.0).astype(np.float32)
        for r in np.flatnonzero(flips):
            js = np.flatnonzero(diff[r])
            bound = 1e-4 * np.abs(rf[r]).max() + 1.01 * step[r] * np.abs(wd[e][:, js]).sum(1)
            assert np.all(np.abs(np_(f)[r0 + r].astype(np.float64) - rf[r]) <= bound)
    B.expert_backward_f32(E, d, h, Tk, offc, xs, dev(wgu), dev(wd), dev(gu_in), dev(ab_in), dev(df),
                          dxs, dwgu, dwd, ws, wsb)
    gdx, gw, gd = np_(dxs), np_(dwgu), np_(dwd)
    for e, (r0, r1, o, rgu, rab, rf) in ref_state.items():
        rdx, rdw, rdd = oracle.expert_backward(o, xs_h[r0:r1], wgu[e:e + 1], wd[e:e + 1], rgu, df[r0:r1])
        assert _row_rel(gdx[r0:r1], rdx).max() <= 1e-4
        assert np.abs(gw[e] - rdw[0]).max() <= 1e-4 * np.abs(rdw[0]).max()
        assert np.abs(gd[e] - rdd[0]).max() <= 1e-4 * np.abs(rdd[0]).max()


def test_attn_decode_full_size_sampled():
    """Decode attention in the launch configuration of bench.py --op
    attn_decode (32 sequences, 12 query heads over 4 key/value heads, 8192
    positions, workspace for the whole batch), checked on three sequences."""
    Bn, nh, nkv, T = 32, 12, 4, 8192
    g = rng(8192)
    kc = torch.randint(-127, 128, (Bn, nkv, T, 64), dtype=torch.int8, device=DEV)
    vc = torch.randint(-127, 128, (Bn, nkv, T, 64), dtype=torch.int8, device=DEV)
    ks = dev((g.random((Bn, nkv, T)) * 0.04 + 1e-3).astype(np.float32))
    vs = dev((g.random((Bn, nkv, T)) * 0.04 + 1e-3).astype(np.float32))
    q = g.standard_normal((Bn, nh, 64)).astype(np.float32)
    lens = np.full(Bn, T, np.int32)
    lens[5] = 4097
    wsb = B.attn_workspace_bytes(Bn, nkv, T)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=DEV)
    out = torch.empty((Bn, nh, 64), device=DEV)
    B.attn_decode_i8(Bn, nh, nkv, 64, T, T, dev(lens), dev(q), kc, vc, ks, vs, out, ws, wsb)
    got = np_(out)
    for b in (0, 5, 31):
        ref = oracle.attn_decode(q[b:b + 1], np_(kc[b:b + 1]), np_(vc[b:b + 1]), np_(ks[b:b + 1]),
                                 np_(vs[b:b + 1]), int(lens[b]))[0]
        err = np.abs(got[b] - ref).max(1) / np.abs(ref).max(1)
        assert err.max() <= 1e-4, (b, err.max())


def test_combine_after_drop_pad():
    """A dropped batch: mm_combine over the kept routing of mm_drop_pad
    (inverse with -1 for dropped assignments) equals the oracle's FP32
    combine with the dropped gate weights set to zero, bit for bit."""
    g = rng(77)
    T, E, k, d = 300, 8, 4, 256
    idx = _skewed_ids(g, T, E, k)
    ds = B.desc(d, E, 64, 0, k)
    off = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    inv = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    nb = B.workspace_bytes(ds, T, B.MM_WS_ROUTE)
    ws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    idx_d = dev(idx)
    B.route_permute(ds, T, idx_d, off, perm, inv, ws, nb)
    C = B.drop_pad_capacity(T, k, E, 1, 1)       # capacity factor 1: the skewed routing overflows
    buf = torch.empty((E * C,), dtype=torch.int32, device=DEV)
    offc = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    permc = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    invc = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    B.drop_pad(T, E, k, C, idx_d, off, perm, inv, buf, offc, permc, invc)
    _, ro, rp, ri = oracle.drop_pad(idx, E, C)
    assert ro[E] < T * k
    f = g.standard_normal((T * k, d)).astype(np.float32)     # kept rows in expert order
    w = g.random((T, k)).astype(np.float32)
    ys = g.standard_normal((T, d)).astype(np.float32)
    y = torch.empty((T, d), device=DEV)
    B.combine(ds, T, dev(f), invc, dev(w), dev(ys), y)
    kept = ri >= 0
    f_tok = np.where(kept[:, None], f[np.maximum(ri, 0)], 0.0).astype(np.float32).reshape(T, k, d)
    w_kept = np.where(kept.reshape(T, k), w, 0.0).astype(np.float32)
    assert np.array_equal(np_(y), oracle.combine_f32(f_tok, w_kept, ys))


@pytest.mark.parametrize("gating", [0, 1, 2, 3])
def test_router_backward(gating):
    """mm_router_backward_f32 against the oracle's double evaluation at the
    S router shape (T = 2048, E = 60, top-4, d = 768) with dropped
    assignments and the pages' z-loss weight: dz per token and dWr within
    1e-4 of the row / matrix maximum, dx (accumulated onto a given
    gradient) within 1e-4 per row."""
    g = rng(90 + gating)
    T, E, k, d = 2048, 60, 4, 768
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = (g.standard_normal(E) * 0.1).astype(np.float32)
    idx = _skewed_ids(g, T, E, k)
    inv = g.permutation(T * k).astype(np.int32)
    inv[g.random(T * k) < 0.03] = -1
    f = g.standard_normal((T * k, d)).astype(np.float32)
    dy = g.standard_normal((T, d)).astype(np.float32)
    dx0 = g.standard_normal((T, d)).astype(np.float32)
    ds = B.desc(d, E, 384, 0, k, gating=gating)
    dz = torch.empty((T, E), device=DEV)
    dwr = torch.empty((E, d), device=DEV)
    dx = dev(dx0)
    B.router_backward_f32(ds, T, dev(x), dev(wr), dev(bias), dev(idx), dev(f), dev(inv), dev(dy), 1e-4,
                          dz, dwr, dx)
    rdz, rdwr, rdx = oracle.router_backward(x, wr, bias, idx, f, inv, dy, gating, 1e-4, dx=dx0)
    assert _row_rel(np_(dz), rdz).max() <= 1e-4
    assert np.abs(np_(dwr) - rdwr).max() <= 1e-4 * np.abs(rdwr).max()
    assert _row_rel(np_(dx), rdx).max() <= 1e-4


@pytest.mark.parametrize("gating", [0, 1, 2, 3])
def test_router_backward_zloss_only(gating):
    """The z-loss term alone: with dy = 0 the gate term vanishes, so dz, dWr
    and dx (accumulated onto zeros) are the z-loss gradient only, checked
    against the oracle at 1e-4 of the row / matrix maximum (the test above
    cannot see it: at lambda_z = 1e-4 and T = 2048 it is about 1e-8 of the
    gate term).  Under the sigmoid gates every logit's dz here, selected or
    not, is pure z-loss."""
    g = rng(190 + gating)
    T, E, k, d = 512, 60, 4, 768
    x = g.standard_normal((T, d)).astype(np.float32)
    wr = (g.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = (g.standard_normal(E) * 0.1).astype(np.float32)
    idx = _skewed_ids(g, T, E, k)
    inv = g.permutation(T * k).astype(np.int32)
    f = g.standard_normal((T * k, d)).astype(np.float32)
    dy = np.zeros((T, d), np.float32)
    dx0 = np.zeros((T, d), np.float32)
    ds = B.desc(d, E, 384, 0, k, gating=gating)
    dz = torch.empty((T, E), device=DEV)
    dwr = torch.empty((E, d), device=DEV)
    dx = dev(dx0)
    B.router_backward_f32(ds, T, dev(x), dev(wr), dev(bias), dev(idx), dev(f), dev(inv), dev(dy), 1e-4,
                          dz, dwr, dx)
    rdz, rdwr, rdx = oracle.router_backward(x, wr, bias, idx, f, inv, dy, gating, 1e-4, dx=dx0)
    assert np.all(np.abs(rdz).max(1) > 0)          # the reference is not trivially zero
    assert _row_rel(np_(dz), rdz).max() <= 1e-4
    assert np.abs(np_(dwr) - rdwr).max() <= 1e-4 * np.abs(rdwr).max()
    assert _row_rel(np_(dx), rdx).max() <= 1e-4


def test_gather_rows_bitexact():
    """mm_gather_rows: dst[r] = scale[perm[r]] * src[perm[r] // k] (FP32
    product), zero rows for -1."""
    g = rng(60)
    T, k, d = 37, 4, 768
    src = g.standard_normal((T, d)).astype(np.float32)
    w = g.random(T * k).astype(np.float32)
    perm = g.permutation(T * k).astype(np.int32)
    perm[5] = -1
    dst = torch.empty((T * k, d), device=DEV)
    B.gather_rows(T * k, d, k, dev(perm), dev(w), dev(src), dst)
    want = src[np.maximum(perm, 0) // k] * w[np.maximum(perm, 0)][:, None]
    want[5] = 0.0
    assert np.array_equal(np_(dst), want.astype(np.float32))
    B.gather_rows(T * k, d, k, dev(perm), None, dev(src), dst)
    want = src[np.maximum(perm, 0) // k].copy()
    want[5] = 0.0
    assert np.array_equal(np_(dst), want)


# ------------------------------------------------------------ expert stages
def _sorted_reference(layer, w, lw, x):
    """Oracle per-sorted-row gate/up and down results for the layer's routing."""
    perm = np_(layer.perm)
    off = np_(layer.offsets)
    xq, sx = oracle.quant_act_i8(x)
    rows = w.T * w.k
    hq = np.zeros((rows, w.h), np.int8)
    hs = np.zeros((rows,), np.float32)
    f = np.zeros((rows, w.d))
    igu = np.zeros((rows, 2 * w.h, w.d // 32), np.int32)
    idn = np.zeros((rows, w.d, w.h // 32), np.int32)
    a = np.zeros((rows, w.h), np.float32)
    for e in range(w.E):
        p = np.arange(off[e], off[e + 1])
        if len(p) == 0:
            continue
        tok = perm[p] // w.k
        gq, gs = oracle.quant_w4g32(lw.w_gu[e])
        dq, dsc = oracle.quant_w4g32(lw.w_d[e])
        hq[p], hs[p], f[p], igu[p], idn[p], a[p] = oracle.ffn_w4a8(
            xq[tok], sx[tok], gq, gs, dq, dsc, want_isum=True, want_a=True)
    return hq, hs, f, igu, idn, a


# The cases reach each kernel family: weight-streaming (up to 32 routed rows),
# matrix-core (more rows, K % 128 == 0) and row-tile (the rest: K % 128 != 0,
# or K beyond the weight-streaming limit of 2560).
STAGE_CASES = [
    ("s_prefill", 200, {}),                              # matrix-core
    ("m_prefill", 70, {}),                               # matrix-core, few rows per expert
    ("m_prefill", 8, {}),                                # weight-streaming
    ("l_prefill", 8, {}),                                # weight-streaming, skewed routing (several tiles per expert)
    ("s_prefill", 3, {}),                                # weight-streaming, decode-sized
    ("s_prefill", 150, {"d": 704, "h": 320, "hs": 640}),  # row-tile (K % 128 != 0)
    ("s_prefill", 30, {"d": 2688, "hs": 0}),              # gate/up row-tile (K > 2560)
]


@pytest.mark.parametrize("name,T,over", STAGE_CASES)
def test_expert_stages_int4(name, T, over):
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    xd = dev(x)
    layer.buffers(T)
    layer.router(xd, T)
    layer.route(T)
    layer.act_quant(xd, T)
    rows = T * w.k
    isum_gu = torch.zeros((rows, 2 * w.h, w.d // 32), dtype=torch.int32, device=DEV)
    layer.gateup(xd, T, isum=isum_gu)
    hq_ref, hs_ref, f_ref, igu_ref, idn_ref, a_ref = _sorted_reference(layer, w, lw, x)
    # exact int32 group sums of the fused gate/up product
    assert np.array_equal(np_(isum_gu), igu_ref)
    # re-quantised hidden rows and their scales
    assert np.array_equal(np_(layer.hbuf), hq_ref)
    assert np.array_equal(np_(layer.hscale), hs_ref)
    # FP32 hidden rows (h_scale NULL): the same kernel without the re-quantisation
    a_gpu = torch.empty((rows, w.h), dtype=torch.float32, device=DEV)
    layer.gateup_f32(xd, T, a_gpu)
    assert np.array_equal(np_(a_gpu), a_ref)
    # down product, stage-isolated: feed the oracle's hidden rows
    layer.hbuf.copy_(dev(hq_ref))
    layer.hscale.copy_(dev(hs_ref))
    isum_d = torch.zeros((rows, w.d, w.h // 32), dtype=torch.int32, device=DEV)
    layer.down(T, isum=isum_d)
    assert np.array_equal(np_(isum_d), idn_ref)
    assert np.array_equal(np_(layer.f), f_ref)


# Merged routed+shared products on the f16 matrix cores (the standalone merged
# entries): ragged expert tiles, empty experts (skewed L routing), a tail of
# one row, E = 1, and row counts from a single tile to many (dense problems
# in 64- and 128-row tiles).
PAIR_CASES = [("s_prefill", 200, {}), ("s_prefill", 37, {}), ("m_prefill", 300, {}),
              ("l_prefill", 130, {}), ("s_prefill", 129, {"E": 1, "k": 1}),
              ("s_prefill", 33, {"E": 64, "k": 8})]


def _shared_reference(w, lw, x):
    xq, sx = oracle.quant_act_i8(x)
    gq, gs = oracle.quant_w4g32(lw.ws_gu)
    dq, dsc = oracle.quant_w4g32(lw.ws_d)
    return oracle.ffn_w4a8(xq, sx, gq, gs, dq, dsc, want_isum=True, want_a=True)


@pytest.mark.parametrize("name,T,over", PAIR_CASES)
def test_gateup_pair_f32(name, T, over):
    """The merged routed+shared gate/up launch (mm_expert_gateup_pair_f32) from
    f16 paired x codes: the codes equal the row-major ones, the exact group
    sums equal the oracle's, and the FP32 hidden rows equal the single
    gate/up call's and the oracle's bit for bit."""
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    xd = dev(x)
    layer.buffers(T)
    layer.router(xd, T)
    layer.route(T)
    layer.act_quant(xd, T)
    xq16 = torch.empty((T, w.d), dtype=torch.int16, device=DEV)
    sx16 = torch.empty((T,), dtype=torch.float32, device=DEV)
    B.act_quant_i8_layout(T, w.d, xd, xq16, sx16, B.MM_ACT_F16_PAIRED)
    assert np.array_equal(decode_f16_paired(np_(xq16), w.d), np_(layer.xq))
    assert np.array_equal(np_(sx16), np_(layer.sx))
    rows = T * w.k
    G = w.d // 32
    h_r = torch.empty((rows, w.h), dtype=torch.float32, device=DEV)
    h_s = torch.empty((T, w.hs), dtype=torch.float32, device=DEV)
    i_r = torch.zeros((rows, 2 * w.h, G), dtype=torch.int32, device=DEV)
    i_s = torch.zeros((T, 2 * w.hs, G), dtype=torch.int32, device=DEV)
    layer.gateup_pair_f32(T, xq16, h_r, h_s, isum_r=i_r, isum_s=i_s)
    ref = _sorted_reference(layer, w, lw, x)
    assert np.array_equal(np_(i_r), ref[3])
    assert np.array_equal(np_(h_r), ref[5])
    sref = _shared_reference(w, lw, x)
    assert np.array_equal(np_(i_s), sref[3])
    assert np.array_equal(np_(h_s), sref[5])
    # the production form (no group sums written) gives the same rows
    h_r2 = torch.empty_like(h_r)
    h_s2 = torch.empty_like(h_s)
    layer.gateup_pair_f32(T, xq16, h_r2, h_s2)
    assert np.array_equal(np_(h_r2), np_(h_r))
    assert np.array_equal(np_(h_s2), np_(h_s))
    a_one = torch.empty((rows, w.h), dtype=torch.float32, device=DEV)
    layer.gateup_f32(xd, T, a_one)
    assert np.array_equal(np_(h_r), np_(a_one))


@pytest.mark.parametrize("name,T,over", PAIR_CASES)
def test_down_pair_f32(name, T, over):
    """The merged routed+shared down launch (mm_expert_down_pair_f32),
    stage-isolated: the oracle's hidden codes go in as f16 paired codes, the
    exact group sums and the FP32 outputs equal the oracle's bit for bit."""
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    xd = dev(x)
    layer.buffers(T)
    layer.router(xd, T)
    layer.route(T)
    rows = T * w.k
    hq_ref, hs_ref, f_ref, _, idn_ref, a_ref = _sorted_reference(layer, w, lw, x)
    shq, shs, sys_, _, sidn, sa = _shared_reference(w, lw, x)
    # the hidden codes through the f16 paired quantiser (codes equal the oracle's)
    hq_r = torch.empty((rows, w.h), dtype=torch.int16, device=DEV)
    hs_r = torch.empty((rows,), dtype=torch.float32, device=DEV)
    hq_s = torch.empty((T, w.hs), dtype=torch.int16, device=DEV)
    hs_s = torch.empty((T,), dtype=torch.float32, device=DEV)
    B.act_quant_i8_layout(rows, w.h, dev(a_ref), hq_r, hs_r, B.MM_ACT_F16_PAIRED)
    B.act_quant_i8_layout(T, w.hs, dev(sa), hq_s, hs_s, B.MM_ACT_F16_PAIRED)
    assert np.array_equal(decode_f16_paired(np_(hq_r), w.h), hq_ref)
    assert np.array_equal(np_(hs_r), hs_ref)
    assert np.array_equal(decode_f16_paired(np_(hq_s), w.hs), shq)
    assert np.array_equal(np_(hs_s), shs)
    f = torch.empty((rows, w.d), dtype=torch.float32, device=DEV)
    ys = torch.empty((T, w.d), dtype=torch.float32, device=DEV)
    i_r = torch.zeros((rows, w.d, w.h // 32), dtype=torch.int32, device=DEV)
    i_s = torch.zeros((T, w.d, w.hs // 32), dtype=torch.int32, device=DEV)
    layer.down_pair_f32(T, hq_r, hs_r, hq_s, hs_s, f, ys, isum_r=i_r, isum_s=i_s)
    assert np.array_equal(np_(i_r), idn_ref)
    assert np.array_equal(np_(f), f_ref.astype(np.float32))
    assert np.array_equal(np_(i_s), sidn)
    assert np.array_equal(np_(ys), sys_.astype(np.float32))


# ------------------------------------------------------------ whole layer
CASES = [
    ("tiny_f32", 128, {}),
    ("tiny_f32", 37, {}),
    ("s_prefill", 256, {}),
    ("s_prefill", 100, {"hs": 0}),
    ("s_prefill", 1, {}),
    ("m_prefill", 200, {}),
    ("l_prefill", 130, {}),
    ("l_prefill_bf16", 64, {}),
    ("l_prefill_bf16", 300, {}),                          # bf16 matrix cores, many row tiles
    ("l_decode_bf16", 1, {}),                             # bf16 weight-streaming kernels
    ("l_decode_bf16", 16, {}),                            # ... 64 routed rows, 16 shared
    ("l_decode_bf16", 17, {}),                            # ... shared expert back on the matrix cores
    ("s_prefill", 200, {"wfmt": "bf16"}),
    ("s_prefill", 64, {"E": 8, "k": 2, "d": 128, "h": 64, "hs": 64}),
    ("s_prefill", 16, {"E": 1, "k": 1, "hs": 0}),
    ("s_prefill", 8, {}),                                 # decode batch
    ("l_prefill", 1, {}),                                 # decode, largest shared expert
    ("m_prefill", 8, {}),                                 # largest weight-streaming shared batch
    ("m_prefill", 9, {}),                                 # ... and the first on the matrix cores
    ("s_prefill", 150, {"d": 704, "h": 320, "hs": 640}),  # row-tile kernels
]


@pytest.mark.parametrize("name,T,over", CASES)
def test_layer_end_to_end(name, T, over):
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    layer.forward(dev(x))
    ref = oracle_forward(w, lw, x)
    assert np.array_equal(np_(layer.idx), ref.idx)
    assert np.array_equal(np_(layer.topw), ref.w.astype(np.float32))
    y = layer_output(layer)
    tol = TOL_BF16 if w.wfmt == "bf16" else TOL_F32
    assert row_rel_err(y, ref.y) <= tol
    if w.wfmt == "int4g32":
        assert np.array_equal(y, ref.y.astype(np.float32))
    # routed outputs per slot, and the shared expert on its own (the routed
    # term is only a few percent of y)
    inv = np_(layer.inv)
    f = np_(layer.f)[inv].reshape(T, w.k, w.d)
    assert row_rel_err(f.reshape(T * w.k, w.d), ref.f.reshape(T * w.k, w.d)) <= (
        TOL_BF16 if w.wfmt == "bf16" else 5e-3)
    if w.hs:
        assert row_rel_err(np_(layer.ys), ref.ys) <= tol


def test_layer_deterministic_and_no_shared_equals_routed_only():
    w = wl.WORKLOADS["s_prefill"].with_(T=300)
    lw = wl.layer_weights(w)
    x = dev(wl.tokens(w))
    layer = make_layer(w, lw)
    y1 = np_(layer.forward(x)).copy()
    y2 = np_(layer.forward(x)).copy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # zero routed down weights: y equals the shared expert bit for bit
    lw0 = wl.LayerWeights(lw.wr, lw.bias, lw.w_gu, np.zeros_like(lw.w_d), lw.ws_gu, lw.ws_d)
    l0 = make_layer(w, lw0)
    y0 = np_(l0.forward(x))
    assert np.array_equal(y0, np_(l0.ys))


def test_token_permutation_equivariance_gpu():
    w = wl.WORKLOADS["s_prefill"].with_(T=257)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    pi = rng(3).permutation(w.T)
    layer = make_layer(w, lw)
    y = np_(layer.forward(dev(x))).copy()
    yp = np_(layer.forward(dev(x[pi]))).copy()
    assert np.array_equal(y[pi], yp)


def test_rmsnorm():
    x = rng(5).standard_normal((67, 768)).astype(np.float32)
    y = torch.empty((67, 768), dtype=torch.float32, device=DEV)
    B.rmsnorm_f32(67, 768, 1e-5, dev(x), y)
    assert row_rel_err(np_(y), oracle.rmsnorm(x, 1e-5)) < 1e-5


# ------------------------------------------------------------ full sizes
# mm_moe_forward: the one-call layer.  Cases reach its merged launches
# (weight-streaming pair, matrix-core pair), the mixed case that falls back to
# separate launches, the other weight formats and the no-shared layer.
FUSED_CASES = [
    ("s_prefill", 1, {}), ("s_prefill", 8, {}),                          # weight-streaming pair
    ("s_prefill", 9, {}), ("s_prefill", 64, {}),                         # matrix-core pair, decode batches
    ("l_prefill", 1, {}), ("m_prefill", 2, {}), ("s_prefill", 3, {}),     # one-workgroup front and past it
    ("s_prefill", 16, {"k": 2}), ("s_prefill", 5, {"E": 64, "k": 8}),    # mixed: separate launches
    ("s_prefill", 256, {}), ("s_prefill", 700, {}),                      # matrix-core pair
    ("s_prefill", 1900, {}),                                               # ... wide waves (two column pairs / four tiles)
    ("s_prefill", 120, {"hs": 0}),
    ("m_prefill", 200, {}), ("l_prefill", 130, {}),
    ("s_prefill", 150, {"d": 704, "h": 320, "hs": 640}),                  # row-tile kernels
    ("s_prefill", 5, {"d": 704, "h": 320, "hs": 640}),                    # down pair from INT8 rows (h % 128 != 0)
    ("l_prefill_bf16", 64, {}), ("tiny_f32", 37, {}), ("l_decode_bf16", 8, {}),
    ("s_prefill", 4, {}),                                                  # token rows staged before the tile lookup
    ("s_prefill", 1500, {"E": 16, "k": 2}),                                # count sort from router histograms, k = 2
    ("s_prefill", 2300, {"E": 1, "k": 1}),                                 # ... one expert, k = 1
    ("s_prefill", 700, {"E": 64, "k": 8}),                                 # ... k = 8: block limits inside a 16-byte piece
    ("s_prefill", 4099, {}), ("s_prefill", 4100, {"E": 16, "k": 8}),       # combine in the shared down's epilogue (ragged, k = 8)
    ("m_prefill", 4100, {}),                                               # two row tiles per wave, combine in the shared down (ragged)
    ("s_prefill", 4200, {"E": 1, "k": 1}), ("s_prefill", 4096, {"E": 8, "k": 2}),  # ... with k = 1 and k = 2 (unused slots)
    ("l_decode", 1, {}), ("m_decode", 1, {}),                              # one token: one-workgroup front, widths 1280 / 1024
    ("s_prefill", 1, {"E": 64, "k": 8}), ("s_prefill", 1, {"d": 256, "h": 128, "hs": 512}),
]


@pytest.mark.parametrize("name,T,over", FUSED_CASES)
def test_fused_forward(name, T, over):
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    xd = dev(x)
    layer.forward(xd)
    y_calls = layer_output(layer).copy()
    idx_calls = np_(layer.idx).copy()
    layer.y.zero_()
    layer.idx.zero_()
    layer.forward_fused(xd)
    # the same launches' arithmetic: bit-identical to the seven calls
    assert np.array_equal(np_(layer.idx), idx_calls)
    assert np.array_equal(layer_output(layer), y_calls)
    ref = oracle_forward(w, lw, x)
    assert np.array_equal(np_(layer.idx), ref.idx)
    y = layer_output(layer)
    if w.wfmt == "int4g32":
        assert np.array_equal(y, ref.y.astype(np.float32))
    else:
        assert row_rel_err(y, ref.y) <= (TOL_BF16 if w.wfmt == "bf16" else TOL_F32)


@pytest.mark.parametrize("name", ["s_prefill", "m_prefill", "l_prefill"])
def test_full_size_sampled(name):
    """The prefill workload at its full token count, in the configuration the
    benchmark times: routing checked in full, y on a sample of tokens (every
    token's output depends only on that token)."""
    w = wl.WORKLOADS[name]
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    layer.forward(dev(x))
    i_ref, w_ref, _ = oracle.router(x, lw.wr, lw.bias, k=w.k)
    assert np.array_equal(np_(layer.idx), i_ref)
    o_ref, p_ref, v_ref = oracle.route(i_ref, w.E)
    assert np.array_equal(np_(layer.offsets), o_ref)
    assert np.array_equal(np_(layer.perm), p_ref)
    xq_ref, sx_ref = oracle.quant_act_i8(x)
    assert np.array_equal(np_(layer.xq), xq_ref)
    sample = np.unique(np.concatenate([[0, w.T - 1], rng(11).choice(w.T, 62, replace=False)]))
    ref = oracle_forward(w, lw, x[sample])
    assert row_rel_err(np_(layer.y)[sample], ref.y) <= TOL_F32
    assert np.array_equal(np_(layer.y)[sample], ref.y.astype(np.float32))
    # the one-call layer at full size (the launches the benchmark times)
    y_calls = np_(layer.y).copy()
    layer.y.zero_()
    layer.forward_fused(dev(x))
    assert np.array_equal(np_(layer.y), y_calls)


def test_full_size_sampled_bf16():
    """The BF16-weight L prefill at its full token count (8192 tokens, the
    workgroup-tiled BF16 matrix-core kernels): routing checked in full, y on a
    sample of tokens within the BF16 bound; the one-call layer matches the
    seven calls bit for bit."""
    w = wl.WORKLOADS["l_prefill_bf16"]
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    layer.forward(dev(x))
    i_ref, _, _ = oracle.router(x, lw.wr, lw.bias, k=w.k)
    assert np.array_equal(np_(layer.idx), i_ref)
    sample = np.unique(np.concatenate([[0, w.T - 1], rng(12).choice(w.T, 30, replace=False)]))
    ref = oracle_forward(w, lw, x[sample])
    y = layer_output(layer)
    assert row_rel_err(y[sample], ref.y) <= TOL_BF16
    y_calls = np_(layer.y).copy()
    layer.y.zero_()
    layer.forward_fused(dev(x))
    assert np.array_equal(np_(layer.y), y_calls)


# ------------------------------------------------------------ decode stack
@pytest.mark.parametrize("B_", [1, 8, 64])
def test_decode_stack_teacher_forced(B_):
    """S-shaped stack, 3 layers, RMSNorm between layers.  Each layer is checked
    on the same input the device layer received (teacher forcing)."""
    w = wl.WORKLOADS["s_decode"].with_(T=B_)
    x = wl.tokens(w, step=0)
    cur = dev(x)
    for l in range(3):
        lw = wl.layer_weights(w, layer=l)
        layer = make_layer(w, lw)
        xin = np_(cur).copy()
        y = layer.forward(cur)
        ref = oracle_forward(w, lw, xin)
        assert np.array_equal(np_(layer.idx), ref.idx)
        assert row_rel_err(np_(y), ref.y) <= TOL_F32
        assert np.array_equal(np_(y), ref.y.astype(np.float32))
        nxt = torch.empty_like(y)
        B.rmsnorm_f32(B_, w.d, 1e-5, y, nxt)
        assert row_rel_err(np_(nxt), oracle.rmsnorm(np_(y), 1e-5)) < 1e-5
        # the one-call layer, with the next layer's input from its combine
        y_calls = np_(y).copy()
        nxt2 = torch.empty_like(y)
        layer.forward_fused(cur, y_norm=nxt2, norm_eps=1e-5)
        assert np.array_equal(np_(layer.y), y_calls)
        assert row_rel_err(np_(nxt2), oracle.rmsnorm(y_calls, 1e-5)) < 1e-5
        cur = nxt


@pytest.mark.parametrize("B_", [1, 8])
def test_decode_stack_free_running(B_):
    """The 20-layer S decode stack run free: the device layers (the one-launch
    layer for B = 1, the one-call layer for B = 8) feed each layer's
    RMS-normalised output to the next.  Every layer is checked against the
    oracle on the input the device layer received (routing and y bit-exact,
    the device RMSNorm within 1e-6 of the oracle's).  Beside it the oracle
    runs its own free trajectory; the two RMSNorms round differently (FP32 on
    the device, double then FP32 in the oracle), so the trajectories agree
    until such an ulp moves an INT8 code across a rounding boundary, and then
    part ways (the stack has no residual path, so random layers amplify any
    difference).  The test prints the routing flips and row errors of the two
    free trajectories per layer."""
    w = wl.WORKLOADS["s_decode"].with_(T=B_)
    x = wl.tokens(w, step=0)
    cur_dev = dev(x)
    cur_ref = x.copy()
    flips, errs = [], []
    for l in range(w.layers):
        lw = wl.layer_weights(w, layer=l)
        layer = make_layer(w, lw)
        xin = np_(cur_dev).copy()
        nxt = torch.empty_like(cur_dev)
        if layer.decode_supported(B_):
            layer.forward_decode(cur_dev, y_norm=nxt, norm_eps=1e-5)
        else:
            layer.forward_fused(cur_dev, y_norm=nxt, norm_eps=1e-5)
        y = np_(layer.y).copy()
        forced = oracle_forward(w, lw, xin)
        assert np.array_equal(np_(layer.idx), forced.idx), f"layer {l}"
        assert np.array_equal(y, forced.y.astype(np.float32)), f"layer {l}"
        assert row_rel_err(np_(nxt), oracle.rmsnorm(y, 1e-5)) < 1e-6, f"layer {l}"
        free = forced if l == 0 else oracle_forward(w, lw, cur_ref)
        flips.append(int((np.sort(np_(layer.idx), 1) != np.sort(free.idx, 1)).any(1).sum()))
        errs.append(row_rel_err(y, free.y))
        cur_dev = nxt
        cur_ref = oracle.rmsnorm(free.y.astype(np.float32), 1e-5).astype(np.float32)
        del layer
    print(f"B = {B_}: free trajectories, tokens with a routing flip per layer {flips}; "
          f"max row error per layer {[f'{e:.1e}' for e in errs]}")
    assert flips[0] == 0 and errs[0] == 0.0


# ------------------------------------------------------------ graph replay
def test_graph_replay_matches_eager():
    """The layer captured in a HIP graph (kernel nodes and the shared-expert
    stream fork/join only) gives the eager result on every replay, with other
    eager work and synchronisations between replays."""
    w = wl.WORKLOADS["s_prefill"].with_(T=300)
    lw = wl.layer_weights(w)
    x = dev(wl.tokens(w))
    layer = make_layer(w, lw)
    y_ref = np_(layer.forward(x)).copy()
    g = layer.capture(x)
    other = make_layer(w.with_(T=77), wl.layer_weights(w, layer=1))
    x2 = dev(wl.tokens(w, step=1, T=77))
    for i in range(3):
        layer.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_(layer.y), y_ref), f"replay {i}"
        other.forward(x2)
        torch.cuda.synchronize()
    # the graph reads x at replay time
    x.copy_(dev(wl.tokens(w, step=5)))
    g.replay()
    y5 = np_(layer.y).copy()
    ref5 = oracle_forward(w, lw, wl.tokens(w, step=5))
    assert np.array_equal(y5, ref5.y.astype(np.float32))
    # the one-call layer in a graph: every replay equals its eager result
    gf = layer.capture(x, fused=True)
    for i in range(3):
        layer.y.zero_()
        gf.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_(layer.y), y5), f"fused replay {i}"
        other.forward_fused(x2)
        torch.cuda.synchronize()


# ------------------------------------------------------------ selection-only bias
@pytest.mark.parametrize("name,T,gating", [
    ("l_prefill", 1, 2), ("l_prefill", 2, 3),    # one-workgroup front
    ("l_prefill", 37, 2),                        # one workgroup per token
    ("l_prefill", 260, 3),                       # 4-token router workgroups, matrix cores
    ("l_prefill", 2300, 2),                      # ... with the count sort from router histograms
])
def test_selection_only_bias_layer(name, T, gating):
    """The Zipf bias steering the selection only (MM_GATE_BIAS_SELECT_ONLY):
    ids, gate weights and y exact against the oracle, both entry points."""
    w = wl.WORKLOADS[name].with_(T=T)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw, gating=gating)
    layer.buffers(T)
    ref = oracle_forward(w, lw, x, gating=gating)
    for fwd in (layer.forward, layer.forward_fused):
        layer.y.zero_()
        fwd(dev(x))
        assert np.array_equal(np_(layer.idx), ref.idx)
        assert np.array_equal(np_(layer.topw), ref.w.astype(np.float32))
        assert np.array_equal(layer_output(layer), ref.y.astype(np.float32))


# ------------------------------------------------------------ other router rules
@pytest.mark.parametrize("name,T,over", [
    ("s_prefill", 300, {"E": 64, "k": 8}),    # largest expert count and top-k
    ("l_prefill", 2, {}),                     # Zipf bias, one-workgroup front
    ("l_prefill", 1, {}),                     # Zipf bias, one token
    ("l_prefill", 260, {}),                   # Zipf bias, matrix cores
])
def test_sigmoid_gating_layer(name, T, over):
    """The layer with sigmoid gating renormalised over the k selected (the
    alternative gate rule): same ids as softmax, weights and y exact."""
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw, gating=1)
    layer.buffers(T)
    ref = oracle_forward(w, lw, x, gating=1)
    for fwd in (layer.forward, layer.forward_fused):
        layer.y.zero_()
        fwd(dev(x))
        assert np.array_equal(np_(layer.idx), ref.idx)
        assert np.array_equal(np_(layer.topw), ref.w.astype(np.float32))
        assert np.array_equal(layer_output(layer), ref.y.astype(np.float32))
