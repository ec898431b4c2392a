"""GPU parity of the one-launch decode layer (mm_moe_decode) through the C ABI.

The one-launch form computes the same arithmetic in the same order as
mm_moe_forward, so its ids, gate weights and y are compared bit for bit with
both mm_moe_forward and the CPU oracle.  Every case also checks that no wait
inside the kernel gave up (the state's status word stays 0) and that the state
is left ready for the next call (calls in a row, with other T in between)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_ffn_amd import binding as B
from sparse_moe_ffn_amd import workloads as wl
from gpu_util import DEV, layer_output, make_layer, np_, oracle_forward

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_both(layer, x, T):
    """(idx, topw, y) of mm_moe_forward and of mm_moe_decode on the same x."""
    xd = dev(x)
    layer.forward_fused(xd)
    ref = (np_(layer.idx).copy(), np_(layer.topw).copy(), layer_output(layer).copy())
    layer.y.zero_()
    layer.idx.zero_()
    layer.topw.zero_()
    layer.forward_decode(xd)
    got = (np_(layer.idx).copy(), np_(layer.topw).copy(), layer_output(layer).copy())
    return ref, got


DECODE_CASES = [
    ("s_decode", 1, {}, 0), ("s_decode", 2, {}, 0), ("s_decode", 3, {}, 0), ("s_decode", 4, {}, 0),
    ("m_decode", 1, {}, 0), ("m_decode", 2, {}, 0), ("m_decode", 4, {}, 0),
    ("l_decode", 1, {}, 0), ("l_decode", 3, {}, 0), ("l_decode", 4, {}, 0),  # Zipf bias; 4: blocks looped
    ("s_decode", 2, {"hs": 0}, 0),                                           # no shared expert
    ("s_decode", 4, {"E": 64, "k": 8}, 0),                                   # 32 slots, 32 tiles
    ("s_decode", 3, {"E": 5, "k": 2}, 0),                                    # experts shared by tokens
    ("s_decode", 1, {"E": 1, "k": 1}, 0),                                    # one expert
    ("s_decode", 3, {"d": 256, "h": 128, "hs": 512}, 0),                     # narrowest width
    ("l_decode", 2, {}, 1), ("l_decode", 1, {}, 2), ("l_decode", 4, {}, 3),  # sigmoid, select-only bias
]


@pytest.mark.parametrize("name,T,over,gating", DECODE_CASES)
def test_decode_matches_forward_and_oracle(name, T, over, gating):
    w = wl.WORKLOADS[name].with_(T=T, **over)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw, gating=gating)
    assert layer.decode_supported(T)
    ref, got = run_both(layer, x, T)
    assert layer.decode_status() == 0
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    ora = oracle_forward(w, lw, x, gating=gating)
    assert np.array_equal(got[0], ora.idx)
    assert np.array_equal(got[1], ora.w.astype(np.float32))
    assert np.array_equal(got[2], ora.y.astype(np.float32))


def test_decode_calls_in_a_row():
    """One state buffer through 12 calls with T cycling 1..4 and fresh
    inputs: every call exact against the oracle, status word 0 throughout."""
    w = wl.WORKLOADS["s_decode"]
    lw = wl.layer_weights(w)
    layer = make_layer(w, lw)
    for i in range(12):
        T = 1 + i % 4
        x = wl.tokens(w, step=100 + i, T=T)
        layer.forward_decode(dev(x))
        ora = oracle_forward(w, lw, x)
        assert np.array_equal(np_(layer.idx), ora.idx), f"call {i}"
        assert np.array_equal(layer_output(layer), ora.y.astype(np.float32)), f"call {i}"
    assert layer.decode_status() == 0


def test_decode_stack_y_norm():
    """S-shaped 4-layer decode stack, batch 1, free running: each layer's
    one-launch call feeds its RMSNorm output to the next; every layer equals
    mm_moe_forward with y_norm bit for bit and the oracle on the same input."""
    w = wl.WORKLOADS["s_decode"].with_(T=1)
    cur = dev(wl.tokens(w, step=0))
    for l in range(4):
        lw = wl.layer_weights(w, layer=l)
        layer = make_layer(w, lw)
        xin = np_(cur).copy()
        n_ref = torch.empty_like(cur)
        layer.forward_fused(cur, y_norm=n_ref, norm_eps=1e-5)
        y_ref = np_(layer.y).copy()
        layer.y.zero_()
        nxt = torch.zeros_like(cur)
        layer.forward_decode(cur, y_norm=nxt, norm_eps=1e-5)
        assert layer.decode_status() == 0
        assert np.array_equal(np_(layer.y), y_ref)
        assert np.array_equal(np_(nxt), np_(n_ref))
        ora = oracle_forward(w, lw, xin)
        assert np.array_equal(np_(layer.y), ora.y.astype(np.float32))
        assert np.abs(np_(nxt) - oracle.rmsnorm(y_ref, 1e-5)).max() <= 1e-5 * np.abs(np_(nxt)).max()
        cur = nxt


def test_decode_bf16_output():
    """INT4 weights with BF16 y: the one-launch form rounds like the combine kernel."""
    w = wl.WORKLOADS["s_decode"].with_(T=3)
    lw = wl.layer_weights(w)
    x = wl.tokens(w)
    layer = make_layer(w, lw)
    layer.desc.out_dtype = B.MM_OUT_BF16
    layer._T = -1
    layer.buffers(3)
    xd = dev(x)
    layer.forward_fused(xd)
    y_ref = np_(layer.y).copy()
    layer.y.zero_()
    layer.forward_decode(xd)
    assert layer.decode_status() == 0
    assert np.array_equal(np_(layer.y), y_ref)


def test_decode_graph_replay():
    """The one-launch layer captured in a HIP graph: every replay equals the
    eager call, with other eager work and synchronisations between replays."""
    w = wl.WORKLOADS["m_decode"].with_(T=2)
    lw = wl.layer_weights(w)
    x = dev(wl.tokens(w))
    layer = make_layer(w, lw)
    y_ref = np_(layer.forward_decode(x)).copy()
    layer.buffers(2)
    warm = torch.cuda.Stream(device=DEV)
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        layer.forward_decode(x)
    torch.cuda.current_stream().wait_stream(warm)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_decode(x)
    other = make_layer(w.with_(T=1), wl.layer_weights(w, layer=1))
    x1 = dev(wl.tokens(w, step=3, T=1))
    for i in range(4):
        layer.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_(layer.y), y_ref), f"replay {i}"
        other.forward_decode(x1)
        torch.cuda.synchronize()
    assert layer.decode_status() == 0 and other.decode_status() == 0


def test_decode_rejects_unsupported():
    w = wl.WORKLOADS["s_decode"]
    lw = wl.layer_weights(w)
    layer = make_layer(w.with_(T=5), lw)
    assert not layer.decode_supported(5)
    with pytest.raises(B.MMError) as e:
        layer.forward_decode(dev(wl.tokens(w, T=5)))
    assert e.value.status == 2  # MM_ERR_SHAPE
