"""Seeded synthetic inputs for the QSA layer step.

This module only draws random numbers and lays them out; it is shared by the tests,
the benchmark and the smoke check, and imports neither the HIP binding nor the
oracle.  All raw tensors are N(0, 1) rounded to binary16 (round-to-nearest-even).

Seeds: ``seed = 1000 * config + 10 * layer + tensor`` with tensor ids
0 raw indexer keys, 1 indexer query, 2 K, 3 V, 4 attention query,
5 new-token rows, 6 planted block ids or the MLA mask.

Stream layout: an array of n values is drawn in chunks of ``CHUNK`` values; chunk i
comes from ``PCG64(SeedSequence(seed).spawn(n_chunks)[i])``.  The result does not
depend on how many threads fill it.

Beyond drawing numbers there are two pieces of arithmetic.  ``correlated_rows`` mixes
the indexer-query rows of the correlated prefill workload (a first-order
autoregression over rows).  ``_rotate`` is used for the
"planted" blocks of the 255k decode workload: the 4 raw keys of a planted block are
the indexer query rotated back by the half-split RoPE angle of the block's
position, so that after pooling, normalisation and RoPE the block lines up with the
query and scores far above the random blocks.  A mistake in it can only make the
planted blocks score low, which the planted-selection tests detect.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
BLOCK = 4

T_RAW, T_QIDX, T_K, T_V, T_Q, T_NEW, T_PLANT = range(7)


def seed_for(cid: int, layer: int, tensor: int) -> int:
    return 1000 * cid + 10 * layer + tensor


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f16(seed: int, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to float16, chunked as described above."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, np.float16)
    n_chunks = max(1, -(-n // CHUNK))
    children = np.random.SeedSequence(seed).spawn(n_chunks)

    def fill(i):
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    decode:  the caches hold ``n_tokens - 1`` tokens; one decode step appends token
             ``n_tokens - 1`` and attends with ``n_tokens`` tokens visible.
    prefill: the caches hold ``n_tokens`` tokens (the depth); a chunk of ``n_q``
             tokens at positions ``n_tokens .. n_tokens + n_q - 1`` is appended and
             each chunk row attends causally.
    mla:     ``n_tokens`` latent KV rows, a mask with ``list_len`` visible positions.
    """
    name: str
    cid: int
    kind: str
    n_tokens: int
    h_idx: int = 16
    d_idx: int = 128
    topk: int = 512
    hq: int = 32
    hkv: int = 4
    d: int = 128
    dv: int = 128
    n_layers: int = 1
    planted: int = 0
    n_q: int = 1
    list_len: int = 0
    q_corr: float = 0.0   # prefill: lag-1 correlation of consecutive indexer-query rows
    extra: dict = field(default_factory=dict)

    @property
    def cap_tokens(self) -> int:
        need = self.n_tokens + (self.n_q if self.kind == "prefill" else 0) + 64
        return (need + 3) // 4 * 4

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    "tiny_decode_4k": Workload("tiny_decode_4k", 1, "decode", 4096, h_idx=4, d_idx=64, topk=64,
                               hq=8, hkv=1, d=128, dv=128),
    "decode_61789": Workload("decode_61789", 2, "decode", 61789, n_layers=12),
    "decode_126253": Workload("decode_126253", 8, "decode", 126253, n_layers=12),
    # one rank's share of the 255,181 context split over 8 GPUs
    "decode_31898": Workload("decode_31898", 9, "decode", 31898, n_layers=12),
    "decode_255181": Workload("decode_255181", 3, "decode", 255181, n_layers=12, planted=8),
    "prefill_1024_at_126253": Workload("prefill_1024_at_126253", 4, "prefill", 126253, n_q=1024),
    # the same caches, with indexer queries that drift slowly from row to row
    "prefill_1024_at_126253_corr": Workload("prefill_1024_at_126253_corr", 4, "prefill", 126253,
                                            n_q=1024, q_corr=0.99),
    "mla_list_262144": Workload("mla_list_262144", 5, "mla", 262144, hq=16, hkv=1, d=576, dv=512,
                                list_len=2048),
}


def _rotate(v: np.ndarray, pos: float, base: float, sign: float) -> np.ndarray:
    """Half-split rotation of the last axis by sign * pos * base^(-2i/d), in fp64."""
    v = v.astype(np.float64)
    d = v.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    theta = sign * pos * base ** (-2.0 * i / d)
    c, s = np.cos(theta), np.sin(theta)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def planted_blocks(w: Workload, layer: int, nb: int) -> np.ndarray:
    if w.planted == 0:
        return np.zeros(0, np.int64)
    r = rng(seed_for(w.cid, layer, T_PLANT))
    return np.sort(r.choice(nb, size=w.planted, replace=False)).astype(np.int64)


def decode_layer(w: Workload, layer: int, base: float = 1.0e4) -> dict:
    """Host arrays for one decode layer: prefix caches (n_tokens-1 rows) and 4 new
    tokens (positions n_tokens-1 .. n_tokens+2, so a step cycle covers every tail
    length), one indexer query and one attention query."""
    assert w.kind == "decode"
    n0 = w.n_tokens - 1
    raw = normal_f16(seed_for(w.cid, layer, T_RAW), (n0, w.h_idx, w.d_idx))
    k = normal_f16(seed_for(w.cid, layer, T_K), (n0, w.hkv, w.d))
    v = normal_f16(seed_for(w.cid, layer, T_V), (n0, w.hkv, w.dv))
    q_idx = normal_f16(seed_for(w.cid, layer, T_QIDX), (w.h_idx, w.d_idx))
    q = normal_f16(seed_for(w.cid, layer, T_Q), (w.hq, w.d))
    new = normal_f16(seed_for(w.cid, layer, T_NEW),
                     (4 * (w.h_idx * w.d_idx + w.hkv * w.d + w.hkv * w.dv),))
    o1 = 4 * w.h_idx * w.d_idx
    o2 = o1 + 4 * w.hkv * w.d
    k_idx_new = new[:o1].reshape(4, w.h_idx, w.d_idx)
    k_new = new[o1:o2].reshape(4, w.hkv, w.d)
    v_new = new[o2:].reshape(4, w.hkv, w.dv)
    planted = planted_blocks(w, layer, n0 // BLOCK)
    for b in planted:
        key = _rotate(q_idx, float(BLOCK * b), base, -1.0).astype(np.float16)
        raw[BLOCK * b:BLOCK * b + BLOCK] = key[None]
    return dict(raw=raw, k=k, v=v, q_idx=q_idx, q=q, k_idx_new=k_idx_new, k_new=k_new,
                v_new=v_new, planted=planted, n_prefix=n0)


def prefill_inputs(w: Workload, layer: int = 0) -> dict:
    """Caches for depth + chunk tokens; the chunk rows are the last n_q rows."""
    assert w.kind == "prefill"
    n_all = w.n_tokens + w.n_q
    raw = normal_f16(seed_for(w.cid, layer, T_RAW), (n_all, w.h_idx, w.d_idx))
    k = normal_f16(seed_for(w.cid, layer, T_K), (n_all, w.hkv, w.d))
    v = normal_f16(seed_for(w.cid, layer, T_V), (n_all, w.hkv, w.dv))
    q_idx = normal_f16(seed_for(w.cid, layer, T_QIDX), (w.n_q, w.h_idx, w.d_idx))
    if w.q_corr:
        q_idx = correlated_rows(q_idx, w.q_corr)
    q = normal_f16(seed_for(w.cid, layer, T_Q), (w.n_q, w.hq, w.d))
    return dict(raw=raw, k=k, v=v, q_idx=q_idx, q=q, depth=w.n_tokens)


def correlated_rows(z: np.ndarray, rho: float) -> np.ndarray:
    """Rows x_0 = z_0, x_r = rho x_(r-1) + sqrt(1 - rho^2) z_r (fp64, then rounded to
    binary16): every row stays N(0, 1) and rows i apart correlate by rho^i, so that
    nearby query rows choose overlapping blocks."""
    x = np.empty(z.shape, np.float64)
    x[0] = z[0]
    c = np.sqrt(1.0 - rho * rho)
    for r in range(1, z.shape[0]):
        x[r] = rho * x[r - 1] + c * z[r].astype(np.float64)
    return x.astype(np.float16)


def mla_inputs(w: Workload, runs: bool = False, layer: int = 0) -> dict:
    """Latent KV rows [n, dkq], queries [hq, dkq] and an additive binary16 mask
    (0 visible, -inf hidden) with list_len visible positions: uniform distinct
    positions, or (runs=True) list_len/4 distinct 4-aligned runs of 4."""
    assert w.kind == "mla"
    kv = normal_f16(seed_for(w.cid, layer, T_K), (w.n_tokens, w.d))
    q = normal_f16(seed_for(w.cid, layer, T_Q), (w.hq, w.d))
    r = rng(seed_for(w.cid, layer, T_PLANT) + (1 if runs else 0))
    if runs:
        starts = r.choice(w.n_tokens // 4, size=w.list_len // 4, replace=False) * 4
        pos = (starts[:, None] + np.arange(4)[None]).ravel()
    else:
        pos = r.choice(w.n_tokens, size=w.list_len, replace=False)
    mask = np.full(w.n_tokens, -np.inf, np.float16)
    mask[pos] = 0.0
    return dict(kv=kv, q=q, mask=mask, positions=np.sort(pos))
