"""ctypes binding of libqsa.so, the QSA layer-step library (C ABI in include/qsa.h).

Argument marshalling only: every function takes torch tensors that already live on
the GPU, checks dtype/shape/contiguity, and passes raw pointers, sizes and the
current HIP stream to the C entry point of the same name.  Every step of the path
runs in the library's HIP kernels; if the library is missing this module raises.
PyTorch supplies device memory and streams, nothing else.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass

import torch  # loads PyTorch's HIP runtime first; libqsa binds to that same runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK = 0
QSA_ERR_INVALID = -1
QSA_ERR_CAPACITY = -2
QSA_ERR_UNSUPPORTED = -3
QSA_ERR_HIP = -4
QSA_STEP_FUSED_GATHER = 0
QSA_STEP_COMPACT_GATHER = 1
QSA_PREFILL_PER_ROW = 0
QSA_PREFILL_GROUPED_UNION = 1
QSA_PREFILL_UNION_ALL = 2

EXPORTS = [
    "qsa_status_string", "qsa_last_error", "qsa_config_check", "qsa_workspace_size",
    "qsa_workspace_init", "qsa_pool_append", "qsa_pool_rebuild", "qsa_kv_append",
    "qsa_index_score", "qsa_topk_blocks", "qsa_gather_kv", "qsa_sparse_attn",
    "qsa_prefill_attn", "qsa_decode_step", "qsa_decode_multi", "qsa_prefill_step",
    "qsa_mla_workspace_size", "qsa_mla_sparse_attn", "qsa_mla_list_status",
    "qsa_decode_step_noalloc", "qsa_trace_scan",
]
QSA_NOALLOC_SCRATCH_BYTES = 16 << 20


class QsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class qsa_config(C.Structure):
    _fields_ = [("h_idx", C.c_int32), ("d_idx", C.c_int32), ("block", C.c_int32),
                ("topk_blocks", C.c_int32), ("hq", C.c_int32), ("hkv", C.c_int32),
                ("d", C.c_int32), ("dv", C.c_int32), ("cap_tokens", C.c_int32),
                ("rope_base", C.c_float), ("rms_eps", C.c_float), ("attn_scale", C.c_float)]


class qsa_layer_bufs(C.Structure):
    _fields_ = [("k_raw", C.c_void_p), ("k_pool", C.c_void_p), ("k_cache", C.c_void_p),
                ("v_cache", C.c_void_p), ("rms_w", C.c_void_p)]


_lib = None


def load():
    """Loads libqsa.so (built in-tree) and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
    L = C.CDLL(LIB_PATH)
    p, i32, u32, sz = C.c_void_p, C.c_int32, C.c_uint32, C.c_size_t
    cfg = C.POINTER(qsa_config)
    sig = {
        "qsa_status_string": (C.c_char_p, [C.c_int]),
        "qsa_last_error": (C.c_char_p, []),
        "qsa_config_check": (C.c_int, [cfg]),
        "qsa_workspace_size": (sz, [cfg, i32, i32]),
        "qsa_workspace_init": (C.c_int, [p, sz, p]),
        "qsa_pool_append": (C.c_int, [cfg, p, i32, i32, p, p, p, p]),
        "qsa_pool_rebuild": (C.c_int, [cfg, p, p, p, i32, i32, p]),
        "qsa_kv_append": (C.c_int, [cfg, p, p, i32, i32, p, p, p]),
        "qsa_index_score": (C.c_int, [cfg, p, i32, i32, p, p, i32, p]),
        "qsa_topk_blocks": (C.c_int, [cfg, p, i32, i32, i32, p, p, p, sz, p]),
        "qsa_gather_kv": (C.c_int, [cfg, p, i32, i32, p, p, p, p, p]),
        "qsa_sparse_attn": (C.c_int, [cfg, p, p, p, i32, p, p, sz, p]),
        "qsa_prefill_attn": (C.c_int, [cfg, p, i32, i32, p, i32, p, p, p, u32, p, sz, p]),
        "qsa_decode_step": (C.c_int, [cfg, C.POINTER(qsa_layer_bufs), i32, p, p, p, p, p, p, p,
                                      p, u32, p, sz, p]),
        "qsa_decode_multi": (C.c_int, [cfg, C.POINTER(qsa_layer_bufs), i32, i32, p, p, p, p, p,
                                       p, p, i32, p, p, sz, p]),
        "qsa_prefill_step": (C.c_int, [cfg, C.POINTER(qsa_layer_bufs), i32, i32, p, p, p, p, p,
                                       p, p, i32, p, u32, p, sz, p]),
        "qsa_mla_workspace_size": (sz, [i32, i32, i32]),
        "qsa_mla_sparse_attn": (C.c_int, [p, i32, p, p, i32, i32, p, i32, i32, C.c_float, p, p,
                                          p, p, sz, p]),
        "qsa_mla_list_status": (C.c_int, [p, i32, C.POINTER(i32), p]),
        "qsa_decode_step_noalloc": (C.c_int, [cfg, C.POINTER(qsa_layer_bufs), i32, p, p, p, p,
                                              p, p, p, p, u32, p]),
        "qsa_trace_scan": (C.c_int, [p, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != QSA_OK:
        msg = load().qsa_last_error().decode(errors="replace")
        raise QsaError(status, msg)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, numel=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return C.c_void_p(t.data_ptr())


H16 = torch.float16


@dataclass(frozen=True)
class Config:
    """Python view of qsa_config."""
    h_idx: int = 16
    d_idx: int = 128
    topk_blocks: int = 512
    hq: int = 32
    hkv: int = 4
    d: int = 128
    dv: int = 128
    cap_tokens: int = 4096
    rope_base: float = 1.0e4
    rms_eps: float = 1.0e-6
    attn_scale: float | None = None
    block: int = 4

    def c(self) -> qsa_config:
        sc = self.attn_scale if self.attn_scale is not None else 1.0 / math.sqrt(self.d)
        return qsa_config(self.h_idx, self.d_idx, self.block, self.topk_blocks, self.hq, self.hkv,
                          self.d, self.dv, self.cap_tokens, self.rope_base, self.rms_eps, sc)


class Layer:
    """Device caches of one layer (allocated with torch; owned by the caller)."""

    def __init__(self, cfg: Config, device="cuda", rms_w=None):
        cap = cfg.cap_tokens
        self.cfg = cfg
        self.k_raw = torch.zeros((cap, cfg.h_idx, cfg.d_idx), dtype=H16, device=device)
        self.k_pool = torch.zeros((cap // 4, cfg.h_idx, cfg.d_idx), dtype=H16, device=device)
        self.k_cache = torch.zeros((cap, cfg.hkv, cfg.d), dtype=H16, device=device)
        self.v_cache = torch.zeros((cap, cfg.hkv, cfg.dv), dtype=H16, device=device)
        self.rms_w = None if rms_w is None else rms_w.to(device=device, dtype=torch.float32)

    def bufs(self) -> qsa_layer_bufs:
        return qsa_layer_bufs(self.k_raw.data_ptr(), self.k_pool.data_ptr(),
                              self.k_cache.data_ptr(), self.v_cache.data_ptr(),
                              None if self.rms_w is None else self.rms_w.data_ptr())


def qsa_config_check(cfg: Config) -> None:
    c = cfg.c()
    _check(load().qsa_config_check(C.byref(c)))


def qsa_workspace_size(cfg: Config, n_q: int, n_ctx: int) -> int:
    c = cfg.c()
    n = load().qsa_workspace_size(C.byref(c), n_q, n_ctx)
    if n == 0:
        raise QsaError(QSA_ERR_INVALID, "invalid config or sizes for qsa_workspace_size")
    return n


def workspace(cfg: Config, n_q: int, n_ctx: int, device="cuda") -> torch.Tensor:
    """Allocates (with torch) and clears a workspace for calls up to (n_q, n_ctx)."""
    n = qsa_workspace_size(cfg, n_q, n_ctx)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    qsa_workspace_init(ws)
    return ws


def qsa_workspace_init(ws: torch.Tensor) -> None:
    _check(load().qsa_workspace_init(_ptr(ws, name="ws"), ws.numel() * ws.element_size(),
                                     _stream()))


def qsa_pool_append(cfg: Config, k_new, n_before: int, k_raw, k_pool, rms_w=None) -> None:
    c = cfg.c()
    n_new = k_new.shape[0]
    _check(load().qsa_pool_append(C.byref(c), _ptr(k_new, H16, name="k_new"), n_new, n_before,
                                  _ptr(k_raw, H16, name="k_raw"), _ptr(k_pool, H16, name="k_pool"),
                                  _ptr(rms_w, torch.float32, name="rms_w"), _stream()))


def qsa_pool_rebuild(cfg: Config, k_raw, k_pool, b_from: int, n_tokens: int, rms_w=None) -> None:
    c = cfg.c()
    _check(load().qsa_pool_rebuild(C.byref(c), _ptr(k_raw, H16, name="k_raw"),
                                   _ptr(k_pool, H16, name="k_pool"),
                                   _ptr(rms_w, torch.float32, name="rms_w"), b_from, n_tokens,
                                   _stream()))


def qsa_kv_append(cfg: Config, k_new, v_new, n_before: int, k_cache, v_cache) -> None:
    c = cfg.c()
    _check(load().qsa_kv_append(C.byref(c), _ptr(k_new, H16), _ptr(v_new, H16), k_new.shape[0],
                                n_before, _ptr(k_cache, H16), _ptr(v_cache, H16), _stream()))


def qsa_index_score(cfg: Config, q_idx, pos0: int, k_pool, scores, ld: int | None = None) -> None:
    c = cfg.c()
    n_q = q_idx.shape[0] if q_idx.dim() == 3 else 1
    ld = ld if ld is not None else (scores.shape[-1] if scores.dim() == 2 else scores.numel())
    _check(load().qsa_index_score(C.byref(c), _ptr(q_idx, H16, name="q_idx"), n_q, pos0,
                                  _ptr(k_pool, H16, name="k_pool"),
                                  _ptr(scores, torch.float32, name="scores"), ld, _stream()))


def qsa_topk_blocks(cfg: Config, scores, n_q: int, ld: int, pos0: int, blk, n_sel, ws) -> None:
    c = cfg.c()
    _check(load().qsa_topk_blocks(C.byref(c), _ptr(scores, torch.float32, name="scores"), n_q, ld,
                                  pos0, _ptr(blk, torch.int32, name="blk"),
                                  _ptr(n_sel, torch.int32, name="n_sel"), _ptr(ws, name="ws"),
                                  ws.numel(), _stream()))


def qsa_gather_kv(cfg: Config, blk, n_blk: int, n_tokens: int, k_cache, v_cache, k_sel,
                  v_sel) -> None:
    c = cfg.c()
    _check(load().qsa_gather_kv(C.byref(c), _ptr(blk, torch.int32, name="blk"), n_blk, n_tokens,
                                _ptr(k_cache, H16), _ptr(v_cache, H16), _ptr(k_sel, H16),
                                _ptr(v_sel, H16), _stream()))


def qsa_sparse_attn(cfg: Config, q, k_sel, v_sel, n_cells: int, out, ws) -> None:
    c = cfg.c()
    _check(load().qsa_sparse_attn(C.byref(c), _ptr(q, H16, name="q"), _ptr(k_sel, H16),
                                  _ptr(v_sel, H16), n_cells, _ptr(out, torch.float32, name="out"),
                                  _ptr(ws), ws.numel(), _stream()))


def qsa_prefill_attn(cfg: Config, q, pos0: int, blk, ldb: int, k_cache, v_cache, out, ws,
                     flags: int = QSA_PREFILL_PER_ROW) -> None:
    c = cfg.c()
    _check(load().qsa_prefill_attn(C.byref(c), _ptr(q, H16, name="q"), q.shape[0], pos0,
                                   _ptr(blk, torch.int32, name="blk"), ldb, _ptr(k_cache, H16),
                                   _ptr(v_cache, H16), _ptr(out, torch.float32, name="out"),
                                   flags, _ptr(ws), 0 if ws is None else ws.numel(), _stream()))


def qsa_decode_step(cfg: Config, layer: Layer, n_before: int, q_idx, k_idx_new, q, k_new, v_new,
                    out, ws, scores_out=None, blk_out=None, flags: int = QSA_STEP_FUSED_GATHER):
    c = cfg.c()
    b = layer.bufs()
    _check(load().qsa_decode_step(C.byref(c), C.byref(b), n_before, _ptr(q_idx, H16, name="q_idx"),
                                  _ptr(k_idx_new, H16, name="k_idx_new"), _ptr(q, H16, name="q"),
                                  _ptr(k_new, H16, name="k_new"), _ptr(v_new, H16, name="v_new"),
                                  _ptr(out, torch.float32, name="out"),
                                  _ptr(scores_out, torch.float32, name="scores_out"),
                                  _ptr(blk_out, torch.int32, name="blk_out"), flags, _ptr(ws),
                                  ws.numel(), _stream()))


def qsa_decode_multi(cfg: Config, layer: Layer, n_before: int, q_idx, k_idx_new, q, k_new, v_new,
                     out, ws, scores_out=None, ld_scores: int = 0, blk_out=None) -> None:
    c = cfg.c()
    b = layer.bufs()
    _check(load().qsa_decode_multi(C.byref(c), C.byref(b), n_before, q_idx.shape[0],
                                   _ptr(q_idx, H16, name="q_idx"),
                                   _ptr(k_idx_new, H16, name="k_idx_new"), _ptr(q, H16, name="q"),
                                   _ptr(k_new, H16, name="k_new"), _ptr(v_new, H16, name="v_new"),
                                   _ptr(out, torch.float32, name="out"),
                                   _ptr(scores_out, torch.float32, name="scores_out"), ld_scores,
                                   _ptr(blk_out, torch.int32, name="blk_out"), _ptr(ws), ws.numel(),
                                   _stream()))


def qsa_prefill_step(cfg: Config, layer: Layer, n_before: int, q_idx, k_idx_new, q, k_new, v_new,
                     out, ws, scores_out=None, ld_scores: int = 0, blk_out=None,
                     flags: int = QSA_PREFILL_PER_ROW) -> None:
    c = cfg.c()
    b = layer.bufs()
    _check(load().qsa_prefill_step(C.byref(c), C.byref(b), n_before, q_idx.shape[0],
                                   _ptr(q_idx, H16), _ptr(k_idx_new, H16), _ptr(q, H16),
                                   _ptr(k_new, H16), _ptr(v_new, H16), _ptr(out, torch.float32),
                                   _ptr(scores_out, torch.float32), ld_scores,
                                   _ptr(blk_out, torch.int32), flags, _ptr(ws), ws.numel(),
                                   _stream()))


def qsa_mla_workspace_size(hq: int, dv: int, list_cap: int) -> int:
    n = load().qsa_mla_workspace_size(hq, dv, list_cap)
    if n == 0:
        raise QsaError(QSA_ERR_INVALID, "invalid sizes for qsa_mla_workspace_size")
    return n


def qsa_mla_sparse_attn(q, kv, v, mask, list_cap: int, scale: float, n_list, out, ws,
                        list_out=None, dv: int = 512) -> None:
    hq, dkq = q.shape
    n = kv.shape[0]
    _check(load().qsa_mla_sparse_attn(_ptr(q, H16, name="q"), hq, _ptr(kv, H16, name="kv"),
                                      _ptr(v, H16, name="v"), dkq, dv,
                                      _ptr(mask, H16, name="mask"), n, list_cap, scale,
                                      _ptr(list_out, torch.int32, name="list_out"),
                                      _ptr(n_list, torch.int32, name="n_list"),
                                      _ptr(out, torch.float32, name="out"), _ptr(ws),
                                      ws.numel(), _stream()))


def qsa_mla_list_status(n_list, list_cap: int) -> int:
    """Waits for the current stream and returns the visible-position count of the
    last list call; raises QsaError(QSA_ERR_CAPACITY) if it exceeds list_cap."""
    n = C.c_int32(0)
    _check(load().qsa_mla_list_status(_ptr(n_list, torch.int32, name="n_list"), list_cap,
                                      C.byref(n), _stream()))
    return int(n.value)


def qsa_decode_step_noalloc(cfg, layer, n_before: int, q_idx, k_idx_new, q, k_new, v_new, out,
                            scores_out=None, blk_out=None,
                            flags: int = QSA_STEP_FUSED_GATHER) -> None:
    """qsa_decode_step with the library's static scratch instead of a workspace."""
    c = cfg.c()
    b = layer.bufs()
    _check(load().qsa_decode_step_noalloc(
        C.byref(c), C.byref(b), n_before, _ptr(q_idx, H16, name="q_idx"),
        _ptr(k_idx_new, H16, name="k_idx_new"), _ptr(q, H16, name="q"),
        _ptr(k_new, H16, name="k_new"), _ptr(v_new, H16, name="v_new"),
        _ptr(out, torch.float32, name="out"), _ptr(scores_out, torch.float32, name="scores_out"),
        _ptr(blk_out, torch.int32, name="blk_out"), flags, _stream()))


def qsa_trace_scan(start=None, stop=None) -> None:
    """The calling thread's next decode step records `start` and `stop`
    (torch.cuda.Event, timing enabled, each recorded once so that it exists) with
    the start and end times of its scoring kernel; None for both clears."""
    def handle(ev):
        if ev is None:
            return None
        if not ev.cuda_event:
            raise ValueError("qsa_trace_scan: record the event once before passing it")
        return C.c_void_p(ev.cuda_event)
    _check(load().qsa_trace_scan(handle(start), handle(stop)))
