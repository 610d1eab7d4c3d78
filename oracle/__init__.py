"""QSA layer-step oracle: numpy wrappers over the plain C reference in qsa_oracle.c.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``sparse_attention_decode_qsa_amd``) never imports it, and it never imports the
product path.

Every wrapper takes numpy arrays (binary16 data as ``np.float16``) and returns
fp64 results where the method produces real numbers, exactly as the C code does.
See qsa_oracle.c for the sources each function follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")
BLOCK = 4


_SRC_MT = os.path.join(_HERE, "qsa_oracle_mt.c")
_LIB_MT = os.path.join(_HERE, "libqsa_oracle_mt.so")
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fPIC"]


def build() -> str:
    """Compile qsa_oracle.c with gcc (strict IEEE: no fast-math, no contraction) into
    the parity library, and, as a second library, the same source together with
    qsa_oracle_mt.c (the all-core timing form of the decode step)."""
    cmd = ["gcc", *CFLAGS, "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    cmd = ["gcc", *CFLAGS, "-pthread", "-shared", "-o", _LIB_MT + ".tmp", _SRC, _SRC_MT, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_MT + ".tmp", _LIB_MT)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        p = C.c_void_p
        i64, i32, dbl = C.c_int64, C.c_int32, C.c_double
        sig = {
            "orc_h2d": (dbl, [C.c_uint16]),
            "orc_d2h": (C.c_uint16, [dbl]),
            "orc_h2d_array": (None, [p, i64, p]),
            "orc_d2h_array": (None, [p, i64, p]),
            "orc_block_pos": (i64, [i64]),
            "orc_pool_block": (None, [C.c_int, C.c_int, p, i64, dbl, dbl, p, p]),
            "orc_pool_rebuild": (None, [C.c_int, C.c_int, p, i64, dbl, dbl, p, p]),
            "orc_pool_append": (None, [C.c_int, C.c_int, p, i64, i64, p, p, dbl, dbl, p]),
            "orc_index_score": (None, [C.c_int, C.c_int, p, p, i64, p, p]),
            "orc_topk_sort": (i64, [p, i64, i64, p]),
            "orc_topk_rank": (i64, [p, i64, i64, p]),
            "orc_cells": (i64, [p, i64, i64, p]),
            "orc_attn_cells": (None, [C.c_int] * 4 + [p, p, p, p, i64, dbl, p]),
            "orc_attn_dense_masked": (None, [C.c_int] * 4 + [p, p, p, i64, p, dbl, p]),
            "orc_decode_step": (i64, [p, p, p, p, p, i64, p, p, p, p, p, p, p, p, p, p]),
            "orc_prefill_row": (i64, [p, p, p, p, i64, p, p, p, p, p, p]),
            "orc_mask_list": (i64, [p, i64, p]),
            "orc_mla_attn": (None, [C.c_int] * 3 + [p, p, p, p, p, i64, dbl, p]),
            "orc_mla_dense": (None, [C.c_int] * 3 + [p, p, p, p, i64, dbl, p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


_lib_mt = None


def lib_mt():
    """The timing library (qsa_oracle.c + qsa_oracle_mt.c); used only to time the
    oracle over all host cores."""
    global _lib_mt
    if _lib_mt is None:
        if not os.path.exists(_LIB_MT):
            build()
        L = C.CDLL(_LIB_MT)
        p, i64 = C.c_void_p, C.c_int64
        L.orc_decode_step_mt.restype = i64
        L.orc_decode_step_mt.argtypes = [p, p, p, p, p, i64, p, p, p, p, p, p, p, p, p, p,
                                         C.c_int]
        _lib_mt = L
    return _lib_mt


class _Cfg(C.Structure):
    _fields_ = [("h_idx", C.c_int32), ("d_idx", C.c_int32), ("topk", C.c_int32),
                ("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32), ("dv", C.c_int32),
                ("rope_base", C.c_double), ("rms_eps", C.c_double), ("scale", C.c_double)]


@dataclass(frozen=True)
class Shape:
    """Shapes and constants of one QSA layer (see the C header comment)."""
    h_idx: int
    d_idx: int
    topk: int
    hq: int
    hkv: int
    d: int
    dv: int
    rope_base: float = 1.0e4
    rms_eps: float = 1.0e-6
    scale: float | None = None

    def c(self) -> _Cfg:
        sc = self.scale if self.scale is not None else 1.0 / np.sqrt(self.d)
        return _Cfg(self.h_idx, self.d_idx, self.topk, self.hq, self.hkv, self.d, self.dv,
                    self.rope_base, self.rms_eps, sc)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float16, a.dtype
    return a


# --------------------------------------------------------------------------- codec
def h2d(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h).view(np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_h2d_array(_ptr(h), h.size, _ptr(out))
    return out


def d2h(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_d2h_array(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


# --------------------------------------------------------------------------- indexer
def block_pos(b: int) -> int:
    return lib().orc_block_pos(b)


def pool_block(raw4: np.ndarray, pos: int, base=1.0e4, eps=1.0e-6, w=None) -> np.ndarray:
    raw4 = _f16(raw4)
    _, H, d = raw4.shape
    out = np.empty((H, d), np.float16)
    wv = None if w is None else np.ascontiguousarray(w, np.float32)
    lib().orc_pool_block(H, d, _ptr(raw4), pos, base, eps, _ptr(wv), _ptr(out))
    return out


def pool_rebuild(raw: np.ndarray, n_tokens: int, base=1.0e4, eps=1.0e-6, w=None) -> np.ndarray:
    raw = _f16(raw)
    H, d = raw.shape[1:]
    out = np.zeros((n_tokens // BLOCK, H, d), np.float16)
    wv = None if w is None else np.ascontiguousarray(w, np.float32)
    lib().orc_pool_rebuild(H, d, _ptr(raw), n_tokens, base, eps, _ptr(wv), _ptr(out))
    return out


def pool_append(k_new, n_before, raw, pooled, base=1.0e4, eps=1.0e-6, w=None) -> None:
    """In place on raw [cap, H, d] and pooled [cap/4, H, d] (both np.float16)."""
    k_new = _f16(k_new)
    assert raw.flags.c_contiguous and pooled.flags.c_contiguous
    H, d = raw.shape[1:]
    n_new = k_new.shape[0]
    assert n_before + n_new <= raw.shape[0]
    assert (n_before + n_new) // BLOCK <= pooled.shape[0]
    wv = None if w is None else np.ascontiguousarray(w, np.float32)
    lib().orc_pool_append(H, d, _ptr(k_new), n_new, n_before, _ptr(raw), _ptr(pooled),
                          base, eps, _ptr(wv))


def index_score(q_idx: np.ndarray, pooled: np.ndarray, nb: int):
    """Returns (fp64 scores, the same rounded to fp32)."""
    q_idx = _f16(q_idx)
    pooled = _f16(pooled)
    H, d = q_idx.shape
    assert pooled.shape[0] >= nb and pooled.shape[1:] == (H, d)
    s64 = np.empty(nb, np.float64)
    s32 = np.empty(nb, np.float32)
    lib().orc_index_score(H, d, _ptr(q_idx), _ptr(pooled), nb, _ptr(s64), _ptr(s32))
    return s64, s32


# --------------------------------------------------------------------------- selection
def topk_sort(scores: np.ndarray, k: int) -> np.ndarray:
    s = np.ascontiguousarray(scores, np.float32)
    out = np.empty(max(min(k, s.size), 0), np.int32)
    n = lib().orc_topk_sort(_ptr(s), s.size, k, _ptr(out))
    return out[:n]


def topk_rank(scores: np.ndarray, k: int) -> np.ndarray:
    s = np.ascontiguousarray(scores, np.float32)
    out = np.empty(s.size, np.int32)
    n = lib().orc_topk_rank(_ptr(s), s.size, k, _ptr(out))
    return out[:n]


def cells(blk: np.ndarray, n_tokens: int) -> np.ndarray:
    blk = np.ascontiguousarray(blk, np.int32)
    out = np.empty(BLOCK * blk.size + BLOCK, np.int64)
    n = lib().orc_cells(_ptr(blk), blk.size, n_tokens, _ptr(out))
    return out[:n]


# --------------------------------------------------------------------------- attention
def attn_cells(q, k_cache, v_cache, cell_list, scale) -> np.ndarray:
    q, k_cache, v_cache = _f16(q), _f16(k_cache), _f16(v_cache)
    hq, d = q.shape
    _, hkv, dk = k_cache.shape
    dv = v_cache.shape[2]
    assert dk == d and hq % hkv == 0
    cl = np.ascontiguousarray(cell_list, np.int64)
    out = np.empty((hq, dv), np.float64)
    lib().orc_attn_cells(hq, hkv, d, dv, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cl),
                         cl.size, scale, _ptr(out))
    return out


def attn_dense_masked(q, k_cache, v_cache, n_tokens, visible, scale) -> np.ndarray:
    q, k_cache, v_cache = _f16(q), _f16(k_cache), _f16(v_cache)
    hq, d = q.shape
    _, hkv, _ = k_cache.shape
    dv = v_cache.shape[2]
    vis = np.ascontiguousarray(visible, np.uint8)
    assert vis.size >= n_tokens
    out = np.empty((hq, dv), np.float64)
    lib().orc_attn_dense_masked(hq, hkv, d, dv, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                n_tokens, _ptr(vis), scale, _ptr(out))
    return out


# --------------------------------------------------------------------------- composed
def decode_step(shape: Shape, raw, pooled, k_cache, v_cache, n_before, q_idx, k_idx_new,
                q, k_new, v_new, rms_w=None):
    """One decode step of one layer; mutates the four caches in place.

    Returns dict(scores64, scores32, blk, out) where out is [hq, dv] fp64."""
    n = n_before + 1
    nb = n // BLOCK
    s64 = np.empty(nb, np.float64)
    s32 = np.empty(nb, np.float32)
    blk = np.empty(max(min(shape.topk, nb), 1), np.int32)
    out = np.empty((shape.hq, shape.dv), np.float64)
    wv = None if rms_w is None else np.ascontiguousarray(rms_w, np.float32)
    cfg = shape.c()
    for a in (raw, pooled, k_cache, v_cache):
        assert a.flags.c_contiguous and a.dtype == np.float16
    assert n <= raw.shape[0] and n <= k_cache.shape[0] and nb <= pooled.shape[0]
    ns = lib().orc_decode_step(C.byref(cfg), _ptr(raw), _ptr(pooled), _ptr(k_cache),
                               _ptr(v_cache), n_before, _ptr(_f16(q_idx)), _ptr(_f16(k_idx_new)),
                               _ptr(_f16(q)), _ptr(_f16(k_new)), _ptr(_f16(v_new)), _ptr(wv),
                               _ptr(s64), _ptr(s32), _ptr(blk), _ptr(out))
    return dict(scores64=s64, scores32=s32, blk=blk[:ns], out=out)


def decode_step_mt(shape: Shape, raw, pooled, k_cache, v_cache, n_before, q_idx, k_idx_new,
                   q, k_new, v_new, threads: int, rms_w=None):
    """decode_step with the block scan split over `threads` POSIX threads (timing form:
    each thread runs the same per-block fp64 sum on its own block range, so the
    results equal decode_step's)."""
    n = n_before + 1
    nb = n // BLOCK
    s64 = np.empty(max(nb, 1), np.float64)
    s32 = np.empty(max(nb, 1), np.float32)
    blk = np.empty(max(min(shape.topk, nb), 1), np.int32)
    out = np.empty((shape.hq, shape.dv), np.float64)
    wv = None if rms_w is None else np.ascontiguousarray(rms_w, np.float32)
    cfg = shape.c()
    for a in (raw, pooled, k_cache, v_cache):
        assert a.flags.c_contiguous and a.dtype == np.float16
    assert n <= raw.shape[0] and n <= k_cache.shape[0] and nb <= pooled.shape[0]
    ns = lib_mt().orc_decode_step_mt(C.byref(cfg), _ptr(raw), _ptr(pooled), _ptr(k_cache),
                                     _ptr(v_cache), n_before, _ptr(_f16(q_idx)),
                                     _ptr(_f16(k_idx_new)), _ptr(_f16(q)), _ptr(_f16(k_new)),
                                     _ptr(_f16(v_new)), _ptr(wv), _ptr(s64), _ptr(s32), _ptr(blk),
                                     _ptr(out), int(threads))
    return dict(scores64=s64[:nb], scores32=s32[:nb], blk=blk[:ns], out=out)


def prefill_row(shape: Shape, pooled, k_cache, v_cache, pos, q_idx_row, q_row):
    """One query row at position pos; caches must already hold tokens [0, pos]."""
    n = pos + 1
    nb = n // BLOCK
    s64 = np.empty(max(nb, 1), np.float64)
    s32 = np.empty(max(nb, 1), np.float32)
    blk = np.empty(max(min(shape.topk, nb), 1), np.int32)
    out = np.empty((shape.hq, shape.dv), np.float64)
    cfg = shape.c()
    assert n <= k_cache.shape[0] and nb <= pooled.shape[0]
    ns = lib().orc_prefill_row(C.byref(cfg), _ptr(_f16(pooled)), _ptr(_f16(k_cache)),
                               _ptr(_f16(v_cache)), pos, _ptr(_f16(q_idx_row)), _ptr(_f16(q_row)),
                               _ptr(s64), _ptr(s32), _ptr(blk), _ptr(out))
    return dict(scores64=s64[:nb], scores32=s32[:nb], blk=blk[:ns], out=out)


# --------------------------------------------------------------------------- MLA list path
def mask_list(mask: np.ndarray) -> np.ndarray:
    m = _f16(mask)
    out = np.empty(m.size, np.int32)
    n = lib().orc_mask_list(_ptr(m), m.size, _ptr(out))
    return out[:n]


def mla_attn(q, kv, v, mask, lst, dv, scale) -> np.ndarray:
    q, kv, mask = _f16(q), _f16(kv), _f16(mask)
    hq, dkq = q.shape
    vv = None if v is None else _f16(v)
    lst = np.ascontiguousarray(lst, np.int32)
    out = np.empty((hq, dv), np.float64)
    lib().orc_mla_attn(hq, dkq, dv, _ptr(q), _ptr(kv), _ptr(vv), _ptr(mask), _ptr(lst), lst.size,
                       scale, _ptr(out))
    return out


def mla_dense(q, kv, v, mask, dv, scale) -> np.ndarray:
    q, kv, mask = _f16(q), _f16(kv), _f16(mask)
    hq, dkq = q.shape
    vv = None if v is None else _f16(v)
    out = np.empty((hq, dv), np.float64)
    lib().orc_mla_dense(hq, dkq, dv, _ptr(q), _ptr(kv), _ptr(vv), _ptr(mask), mask.size, scale,
                        _ptr(out))
    return out
