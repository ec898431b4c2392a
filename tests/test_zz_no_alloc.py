"""The no-allocation decode entry point (mm_moe_decode_noalloc) through the C
ABI: its outputs equal mm_moe_decode's (the workspace form) bit for bit, on
two calls in a row sharing the library's fixed device scratch, the second
with a smaller input (fewer tokens, narrower layer)."""
import numpy as np
import pytest
import torch

from sparse_moe_ffn_amd import binding as B
from sparse_moe_ffn_amd import workloads as wl
from gpu_util import DEV, make_layer, np_

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_noalloc_matches_workspace_form():
    none = B.weight(None, None)
    for name, T, norm in (("l_decode", 4, False), ("s_decode", 1, True)):
        w = wl.WORKLOADS[name].with_(T=T)
        lw = wl.layer_weights(w)
        layer = make_layer(w, lw)
        x = dev(wl.tokens(w, step=7))
        n_ref = torch.zeros((T, w.d), dtype=torch.float32, device=DEV) if norm else None
        layer.forward_decode(x, y_norm=n_ref, norm_eps=1e-5)
        ref = (np_(layer.idx).copy(), np_(layer.topw).copy(), np_(layer.y).copy())
        assert layer.decode_status() == 0
        idx = torch.full((T, w.k), -1, dtype=torch.int32, device=DEV)
        topw = torch.zeros((T, w.k), dtype=torch.float32, device=DEV)
        y = torch.zeros((T, w.d), dtype=torch.float32, device=DEV)
        n_out = torch.zeros((T, w.d), dtype=torch.float32, device=DEV) if norm else None
        B.moe_decode_noalloc(layer.desc, T, x, layer.wr, layer.bias, layer.w_gu.c(), layer.w_d.c(),
                             layer.ws_gu.c() if w.hs else none, layer.ws_d.c() if w.hs else none,
                             idx, topw, y, y_norm=n_out, norm_eps=1e-5 if norm else 0.0)
        torch.cuda.synchronize()
        assert np.array_equal(np_(idx), ref[0]), name
        assert np.array_equal(np_(topw), ref[1]), name
        assert np.array_equal(np_(y), ref[2]), name
        if norm:
            assert np.array_equal(np_(n_out), np_(n_ref)), name
