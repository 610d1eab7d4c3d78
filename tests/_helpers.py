"""Shared helpers for the GPU parity tests (tolerances are stated here once)."""
import numpy as np
import torch

import oracle as O
from sparse_attention_decode_qsa_amd import binding as qb
import synth

# Scores against the oracle run on the oracle's own pooled rows: max |delta| per row
# <= SCORE_REL * max |score| (fp32 accumulation plus <= 1 binary16 ulp per pooled value).
SCORE_REL = 1e-3
# Scores against the oracle run on the GPU's pooled rows: |delta_b| <= SCORE_ABS_REL *
# sum_i |q_i * P_bi|.  The kernel sums 16 pairwise dot2 steps per lane and a 6-level
# lane tree, so fp32 rounding stays below ~22 * 2^-24 of that sum.
SCORE_ABS_REL = 1e-5
# Attention outputs: max |delta| <= ATTN_REL * max |out_ref| (binary16 in, fp32 accumulate).
ATTN_REL = 2e-3
# Pooled rows: |delta| <= one binary16 ulp of the reference value + POOL_ABS (fp32 vs fp64
# rounding before the final binary16 rounding; slack for RoPE cancellation).
POOL_ABS = 4e-6


def f16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_pool_close(gpu, ref):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    d = np.abs(g - r)
    bound = f16_ulp(r) + POOL_ABS
    bad = d > bound
    assert not bad.any(), f"{bad.sum()} pooled values off by more than 1 ulp; max {d.max()}"


def assert_attn_close(gpu, ref, what="attention"):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.max(np.abs(g - r))
    assert err <= ATTN_REL * np.max(np.abs(r)), f"{what}: max err {err} vs max |ref| {np.abs(r).max()}"


def dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def cfg_of(w: synth.Workload, cap=None) -> qb.Config:
    return qb.Config(h_idx=w.h_idx, d_idx=w.d_idx, topk_blocks=w.topk, hq=w.hq, hkv=w.hkv, d=w.d,
                     dv=w.dv, cap_tokens=cap or w.cap_tokens)


def shape_of(w: synth.Workload) -> O.Shape:
    return O.Shape(w.h_idx, w.d_idx, w.topk, w.hq, w.hkv, w.d, w.dv)


class OracleLayer:
    """Host caches kept by the oracle for one layer."""

    def __init__(self, w: synth.Workload, cap: int):
        self.raw = np.zeros((cap, w.h_idx, w.d_idx), np.float16)
        self.pooled = np.zeros((cap // 4, w.h_idx, w.d_idx), np.float16)
        self.k = np.zeros((cap, w.hkv, w.d), np.float16)
        self.v = np.zeros((cap, w.hkv, w.dv), np.float16)


def setup_decode(w: synth.Workload, layer: int = 0, with_oracle: bool = True):
    """GPU layer (pooled by the library's own append) and, optionally, the oracle's."""
    L = synth.decode_layer(w, layer)
    n0 = L["n_prefix"]
    cfg = cfg_of(w)
    g = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(L["raw"]), 0, g.k_raw, g.k_pool)
    g.k_cache[:n0] = dev(L["k"])
    g.v_cache[:n0] = dev(L["v"])
    o = None
    if with_oracle:
        o = OracleLayer(w, w.cap_tokens)
        O.pool_append(L["raw"], 0, o.raw, o.pooled)
        o.k[:n0], o.v[:n0] = L["k"], L["v"]
    return L, cfg, g, o
