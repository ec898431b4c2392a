"""Workload shapes and seeded synthetic inputs for the MoE-FFN layer.

This module is shared by the tests, the benchmark, the HIP path's callers and
the oracle's callers.  It holds none of the layer's arithmetic: it only draws
seeded random FP32 arrays of the right shapes (and the per-expert bias vector
used for the skewed-routing workload).  Quantisation, routing and every other
step are done separately by the HIP library and by the oracle.

Shapes follow the MobileMoE close reading (paper-archivist.com):
  - section "MoE preliminaries and three design factors": base ratio
    d_ff = 4 d_model; granularity g = 8 splits each expert to hidden d_ff/8;
  - Finding 3 of the architecture search: 60 routed experts, top-4, one shared
    expert four times the size of a routed one (hidden 4h);
  - "Pre-training" efficiency list: the S model's experts are 768 x 384.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

import numpy as np

TENSOR_ROUTER, TENSOR_GATEUP, TENSOR_DOWN, TENSOR_SGATEUP, TENSOR_SDOWN, TENSOR_ZIPF = range(6)
TENSOR_WQ, TENSOR_WK, TENSOR_WV, TENSOR_WO, TENSOR_KV = range(6, 11)
HEAD_DIM, KV_HEADS = 64, 4


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed family
    d: int                # d_model
    E: int                # routed experts
    h: int                # routed expert hidden size
    hs: int               # shared expert hidden size (0: no shared expert)
    k: int                # experts per token
    T: int                # tokens per call (prefill) or batch (decode)
    wfmt: str = "int4g32"  # "f32" | "int4g32" | "bf16"
    bias: str = "none"    # "none" | "zipf"
    layers: int = 1       # stacked layers (decode stack)
    mode: str = "prefill"  # "prefill" | "decode"
    weight_std: float = 0.02

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def ops_per_token(self) -> int:
        """Int8 multiply-add ops per token of the expert FFNs: 2 * active MACs."""
        return 2 * (self.k * 3 * self.d * self.h + 3 * self.d * self.hs)


WORKLOADS: Dict[str, Workload] = {
    # Tiny layer, FP32 everywhere (parity workload).
    "tiny_f32": Workload("tiny_f32", 0, d=256, E=60, h=64, hs=256, k=4, T=128, wfmt="f32"),
    # MobileMoE-S-shaped layer, prefill of 2048 tokens, INT4 g32 weights, INT8 activations.
    "s_prefill": Workload("s_prefill", 1, d=768, E=60, h=384, hs=1536, k=4, T=2048),
    # S-shaped 20-layer stack, decode with batch 1/8/64, RMSNorm between layers.
    "s_decode": Workload("s_decode", 2, d=768, E=60, h=384, hs=1536, k=4, T=1, layers=20,
                         mode="decode"),
    # MobileMoE-M-shaped layer.
    "m_prefill": Workload("m_prefill", 3, d=1024, E=60, h=512, hs=2048, k=4, T=8192),
    "m_decode": Workload("m_decode", 3, d=1024, E=60, h=512, hs=2048, k=4, T=1, mode="decode"),
    # MobileMoE-L-shaped layer with a Zipf-skewed router bias; INT4 and BF16 weights.
    "l_prefill": Workload("l_prefill", 4, d=1280, E=60, h=640, hs=2560, k=4, T=8192, bias="zipf"),
    "l_decode": Workload("l_decode", 4, d=1280, E=60, h=640, hs=2560, k=4, T=1, bias="zipf",
                         mode="decode"),
    "l_prefill_bf16": Workload("l_prefill_bf16", 4, d=1280, E=60, h=640, hs=2560, k=4, T=8192,
                               bias="zipf", wfmt="bf16"),
    "l_decode_bf16": Workload("l_decode_bf16", 4, d=1280, E=60, h=640, hs=2560, k=4, T=1,
                              bias="zipf", wfmt="bf16", mode="decode"),
}


def weight_seed(w: Workload, layer: int, tensor: int) -> int:
    return 1_000_000 * (w.index + 1) + 1_000 * layer + tensor


def input_seed(w: Workload, step: int) -> int:
    return 2_000_000 * (w.index + 1) + step


def _normal(seed: int, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def zipf_bias(w: Workload, layer: int = 0, s: float = 1.2) -> np.ndarray:
    """Per-expert router bias b_e = -s * ln(rank_e), rank a seeded permutation
    of 1..E, so the prior routing weight of expert e is proportional to
    rank_e^(-s) (a Zipf-shaped load)."""
    g = np.random.Generator(np.random.PCG64(weight_seed(w, layer, TENSOR_ZIPF)))
    rank = g.permutation(w.E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


@dataclass
class LayerWeights:
    wr: np.ndarray                 # [E, d] FP32 router
    bias: Optional[np.ndarray]     # [E] or None
    w_gu: np.ndarray               # [E, 2h, d]: gate rows 0..h-1, up rows h..2h-1
    w_d: np.ndarray                # [E, d, h]
    ws_gu: Optional[np.ndarray]    # [2hs, d]
    ws_d: Optional[np.ndarray]     # [d, hs]


def layer_weights(w: Workload, layer: int = 0) -> LayerWeights:
    """FP32 weights ~ N(0, std^2) from the per-(workload, layer, tensor) seed."""
    sd = w.weight_std
    wr = _normal(weight_seed(w, layer, TENSOR_ROUTER), (w.E, w.d), sd)
    w_gu = _normal(weight_seed(w, layer, TENSOR_GATEUP), (w.E, 2 * w.h, w.d), sd)
    w_d = _normal(weight_seed(w, layer, TENSOR_DOWN), (w.E, w.d, w.h), sd)
    ws_gu = ws_d = None
    if w.hs:
        ws_gu = _normal(weight_seed(w, layer, TENSOR_SGATEUP), (2 * w.hs, w.d), sd)
        ws_d = _normal(weight_seed(w, layer, TENSOR_SDOWN), (w.d, w.hs), sd)
    bias = zipf_bias(w, layer) if w.bias == "zipf" else None
    return LayerWeights(wr, bias, w_gu, w_d, ws_gu, ws_d)


@dataclass
class AttnWeights:
    n_h: int                       # query heads (d / 64)
    n_kv: int                      # key/value heads
    wq: np.ndarray                 # [n_h * 64, d]
    wk: np.ndarray                 # [n_kv * 64, d]
    wv: np.ndarray                 # [n_kv * 64, d]
    wo: np.ndarray                 # [d, n_h * 64]


def attn_weights(w: Workload, layer: int = 0) -> AttnWeights:
    """The attention projections of the decoder block around the layer: GQA
    with KV_HEADS heads of HEAD_DIM and d / HEAD_DIM query heads
    (section "MoE preliminaries and three design factors"; "Mid-training":
    n_kv = 4, d_h = 64), FP32 ~ N(0, std^2) from per-tensor seeds."""
    n_h, sd = w.d // HEAD_DIM, w.weight_std
    qd, kd = n_h * HEAD_DIM, KV_HEADS * HEAD_DIM
    return AttnWeights(n_h, KV_HEADS,
                       _normal(weight_seed(w, layer, TENSOR_WQ), (qd, w.d), sd),
                       _normal(weight_seed(w, layer, TENSOR_WK), (kd, w.d), sd),
                       _normal(weight_seed(w, layer, TENSOR_WV), (kd, w.d), sd),
                       _normal(weight_seed(w, layer, TENSOR_WO), (w.d, qd), sd))


def kv_context(w: Workload, B: int, max_T: int, layer: int = 0):
    """Earlier context already in an INT8 KV cache: codes uniform in
    [-127, 127] and per-vector scales uniform in [0.5, 1.5] / 127, as
    (k_codes, v_codes [B, n_kv, max_T, 64] int8, k_scales, v_scales
    [B, n_kv, max_T] FP32)."""
    g = np.random.Generator(np.random.PCG64(weight_seed(w, layer, TENSOR_KV) + 7919 * B + max_T))
    shp = (B, KV_HEADS, max_T, HEAD_DIM)
    kq = g.integers(-127, 128, shp, dtype=np.int8)
    vq = g.integers(-127, 128, shp, dtype=np.int8)
    ks = (g.uniform(0.5, 1.5, shp[:3]) / 127).astype(np.float32)
    vs = (g.uniform(0.5, 1.5, shp[:3]) / 127).astype(np.float32)
    return kq, vq, ks, vs


def tokens(w: Workload, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Layer input x ~ N(0, 1), [T, d] FP32."""
    return _normal(input_seed(w, step), (T if T is not None else w.T, w.d), 1.0)


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same structure) for quick parity cases."""
    return w.with_(**kw)


def param_counts(d: int, n_layers: int, vocab: int = 128_256, E: int = 60, k: int = 4,
                 n_kv: int = 4, d_head: int = 64) -> Tuple[int, int]:
    """(active, total) parameter counts of a MobileMoE model with routed hidden
    d_ff/8 = d/2, shared hidden 4*(d/2), GQA attention with n_kv KV heads of
    width d_head, FP32 router [E, d] and a tied embedding of `vocab` rows.
    Used only to check the layer shapes against the counts the pages print."""
    h = d // 2
    hs = 4 * h
    attn = 2 * d * d + 2 * d * (n_kv * d_head)
    router = E * d
    expert = 3 * d * h
    shared = 3 * d * hs
    per_layer_total = attn + router + E * expert + shared
    per_layer_active = attn + router + k * expert + shared
    emb = vocab * d
    return n_layers * per_layer_active + emb, n_layers * per_layer_total + emb
