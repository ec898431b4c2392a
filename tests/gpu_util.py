"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
bring results back as numpy; decode the library's documented weight layouts
on the host; error metrics."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_moe_ffn_amd import binding as B
from sparse_moe_ffn_amd import workloads as wl
from sparse_moe_ffn_amd.layer import MoELayer

DEV = "cuda"


def np_(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def unpack_canonical(q: np.ndarray) -> np.ndarray:
    """Canonical INT4 bytes [rows, cols/2] -> int8 values [rows, cols]
    (column c in byte c/2, low nibble for even c, two's complement)."""
    q = q.astype(np.uint8)
    lo = (q & 0xF).astype(np.int16)
    hi = (q >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((q.shape[0], q.shape[1] * 2), np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def decode_prepacked(qp: np.ndarray, sp: np.ndarray, n: int, rows: int, cols: int):
    """Inverse of the prepacked layout described in csrc/common.h: 512-byte
    chunks per (32-row block, 32-column group); lane L holds row L%32, columns
    16*(L/32)+i; word w byte b = column 8w+b (low nibble) and 8w+b+4 (high);
    scales pre-divided by 16."""
    G, RB = cols // 32, rows // 32
    ch = qp.reshape(n, RB, G, 64, 2, 4).astype(np.uint8)       # [n, rb, g, lane, word, byte]
    lo = (ch & 0xF).astype(np.int16)
    hi = (ch >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    vals = np.concatenate([lo, hi], axis=-1)                  # [..., word, 8]: cols 8w+0..7
    vals = vals.reshape(n, RB, G, 2, 32, 16)                  # lane -> (half, row)
    q = vals.transpose(0, 1, 4, 2, 3, 5).reshape(n, rows, cols).astype(np.int8)
    s = sp.reshape(n, RB, G, 32).transpose(0, 1, 3, 2).reshape(n, rows, G) * np.float32(16)
    return q, s


def decode_f16_paired(q16: np.ndarray, cols: int) -> np.ndarray:
    """Inverse of the f16 paired code layout (include/mobmoe.h,
    MM_ACT_F16_PAIRED): 16-bit values [rows, cols] -> int8 codes [rows, cols].
    Slot s of each 8-column block holds column 2s (s < 4) or 2(s-4)+1, as a
    half value divided by 16 for columns 4..7 of the block."""
    v = q16.view(np.float16).astype(np.float32).reshape(-1, cols // 8, 8)
    col_of_slot = np.array([0, 2, 4, 6, 1, 3, 5, 7])
    out = np.empty_like(v)
    out[:, :, col_of_slot] = v
    out[:, :, 4:] *= 16.0
    assert np.array_equal(out, np.rint(out)), "f16 paired values are not whole codes"
    return out.reshape(-1, cols).astype(np.int8)


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_c |gpu - ref| / max_c |ref|."""
    g = gpu.astype(np.float64).reshape(gpu.shape[0], -1)
    r = ref.astype(np.float64).reshape(ref.shape[0], -1)
    den = np.abs(r).max(1)
    den[den == 0] = 1.0
    return float((np.abs(g - r).max(1) / den).max())


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_layer(w: wl.Workload, lw: wl.LayerWeights, keep_canonical=False, gating=0) -> MoELayer:
    return MoELayer(w.d, w.E, w.h, w.hs, w.k, lw.wr, lw.bias, lw.w_gu, lw.w_d, lw.ws_gu, lw.ws_d,
                    wfmt=w.wfmt, gating=gating,
                    out_dtype=B.MM_OUT_BF16 if w.wfmt == "bf16" else B.MM_OUT_F32,
                    device=DEV, keep_canonical=keep_canonical)


def oracle_forward(w: wl.Workload, lw: wl.LayerWeights, x: np.ndarray, gating=0, nthreads=8):
    return oracle.forward(x, lw.wr, lw.bias, lw.w_gu, lw.w_d, lw.ws_gu, lw.ws_d, k=w.k,
                          wfmt=w.wfmt, gating=gating, nthreads=nthreads)


def layer_output(layer: MoELayer) -> np.ndarray:
    y = np_(layer.y)
    if layer.desc.out_dtype == B.MM_OUT_BF16:
        return bf16_bits_to_f32(y.view(np.uint16))
    return y
