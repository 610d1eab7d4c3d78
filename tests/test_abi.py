"""The C ABI without a GPU: the library loads, exports every function qsa.h declares,
and rejects bad arguments on the host before anything reaches the GPU."""
import ctypes as C
import os
import re
import subprocess

import pytest

from sparse_attention_decode_qsa_amd import binding as qb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qb.LIB_PATH):
        pytest.fail("libqsa.so is not built (run __graft_entry__.build())")
    return qb.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["qsa_pool_append", "qsa_index_score", "qsa_topk_blocks", "qsa_gather_kv",
              "qsa_sparse_attn", "qsa_decode_step", "qsa_mla_sparse_attn"]:
        assert n in names
    assert set(names) == set(qb.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", qb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None
    # the library exports the C ABI and nothing else (no helpers, no C++ names)
    assert exported == set(declared_functions())


def test_status_strings(lib):
    assert lib.qsa_status_string(0) == b"ok"
    assert lib.qsa_status_string(-3).startswith(b"unsupported")
    assert lib.qsa_status_string(42) == b"unknown status"


def cfg(**kw):
    base = dict(h_idx=16, d_idx=128, topk_blocks=512, hq=32, hkv=4, d=128, dv=128,
                cap_tokens=255244)
    base.update(kw)
    return qb.Config(**base)


def test_config_check_accepts_the_workloads(lib):
    qb.qsa_config_check(cfg())
    qb.qsa_config_check(cfg(h_idx=4, d_idx=64, topk_blocks=64, hq=8, hkv=1, cap_tokens=4160))


@pytest.mark.parametrize("kw,status", [
    (dict(block=8), qb.QSA_ERR_UNSUPPORTED),
    (dict(d_idx=100), qb.QSA_ERR_INVALID),
    (dict(h_idx=3), qb.QSA_ERR_UNSUPPORTED),
    (dict(hq=30), qb.QSA_ERR_INVALID),
    (dict(hq=12, hkv=4), qb.QSA_ERR_UNSUPPORTED),
    (dict(d=96, dv=96), qb.QSA_ERR_UNSUPPORTED),
    (dict(cap_tokens=4097), qb.QSA_ERR_UNSUPPORTED),
    (dict(cap_tokens=1 << 22), qb.QSA_ERR_UNSUPPORTED),
    (dict(topk_blocks=0), qb.QSA_ERR_UNSUPPORTED),
    (dict(rope_base=-1.0), qb.QSA_ERR_INVALID),
])
def test_config_check_rejects(lib, kw, status):
    with pytest.raises(qb.QsaError) as e:
        qb.qsa_config_check(cfg(**kw))
    assert e.value.status == status


def test_workspace_size_is_monotone_and_zero_on_bad_input(lib):
    c = cfg().c()
    a = lib.qsa_workspace_size(C.byref(c), 1, 61789)
    b = lib.qsa_workspace_size(C.byref(c), 1, 255181)
    p = lib.qsa_workspace_size(C.byref(c), 1024, 127277)
    assert 0 < a < b < p
    assert lib.qsa_workspace_size(C.byref(c), 0, 100) == 0
    assert lib.qsa_workspace_size(C.byref(c), 1, 255245) == 0  # beyond cap_tokens
    assert lib.qsa_mla_workspace_size(16, 512, 2048) > 0
    assert lib.qsa_mla_workspace_size(0, 512, 2048) == 0


FAKE = C.c_void_p(1 << 20)          # aligned, never dereferenced: checks fail first
MISALIGNED = C.c_void_p((1 << 20) + 2)


def test_entry_points_reject_bad_arguments_on_the_host(lib):
    c = cfg(cap_tokens=4096).c()
    cp = C.byref(c)
    # NULL / misaligned pointers
    assert lib.qsa_pool_append(cp, None, 4, 0, FAKE, FAKE, None, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_append(cp, MISALIGNED, 4, 0, FAKE, FAKE, None, None) == qb.QSA_ERR_INVALID
    # capacity
    assert lib.qsa_pool_append(cp, FAKE, 8, 4090, FAKE, FAKE, None, None) == qb.QSA_ERR_CAPACITY
    assert lib.qsa_kv_append(cp, FAKE, FAKE, 1, 4096, FAKE, FAKE, None) == qb.QSA_ERR_CAPACITY
    # negative sizes
    assert lib.qsa_pool_append(cp, FAKE, -1, 0, FAKE, FAKE, None, None) == qb.QSA_ERR_INVALID
    # n_new == 0 is a no-op that succeeds without touching anything
    assert lib.qsa_pool_append(cp, None, 0, 0, None, None, None, None) == qb.QSA_OK
    # rebuild: b_from outside [0, floor(n_tokens/4)], n_tokens past capacity, NULL caches;
    # an empty range is a no-op
    assert lib.qsa_pool_rebuild(cp, FAKE, FAKE, None, 26, 100, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_rebuild(cp, FAKE, FAKE, None, -1, 100, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_rebuild(cp, FAKE, FAKE, None, 0, 4097, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_rebuild(cp, None, FAKE, None, 0, 100, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_rebuild(cp, FAKE, MISALIGNED, None, 0, 100, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_pool_rebuild(cp, None, None, None, 25, 103, None) == qb.QSA_OK
    # score: ld too small
    assert lib.qsa_index_score(cp, FAKE, 1, 4000, FAKE, FAKE, 10, None) == qb.QSA_ERR_INVALID
    # top-k: workspace too small
    assert lib.qsa_topk_blocks(cp, FAKE, 1, 1024, 4000, FAKE, FAKE, FAKE, 64, None) == \
        qb.QSA_ERR_CAPACITY
    # gather: n_blk must equal min(k, nb)
    assert lib.qsa_gather_kv(cp, FAKE, 3, 100, FAKE, FAKE, FAKE, FAKE, None) == qb.QSA_ERR_INVALID
    # attention: cells out of range
    assert lib.qsa_sparse_attn(cp, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30, None) == \
        qb.QSA_ERR_INVALID
    assert lib.qsa_sparse_attn(cp, FAKE, FAKE, FAKE, 4 * 512 + 4, FAKE, FAKE, 1 << 30, None) == \
        qb.QSA_ERR_INVALID
    # decode step: NULL layer, bad flags, position past capacity
    assert lib.qsa_decode_step(cp, None, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                               FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    b = qb.qsa_layer_bufs(1 << 20, 1 << 20, 1 << 20, 1 << 20, None)
    assert lib.qsa_decode_step(cp, C.byref(b), 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               None, 0, FAKE, 1 << 30, None) == qb.QSA_ERR_CAPACITY
    assert lib.qsa_decode_step(cp, C.byref(b), 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               None, 7, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_decode_step(cp, C.byref(b), 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               None, 0, FAKE, 16, None) == qb.QSA_ERR_CAPACITY
    assert b"workspace" in lib.qsa_last_error()
    # multi-query decode: n_q outside [1, 4], rows past capacity, ld_scores too small
    assert lib.qsa_decode_multi(cp, C.byref(b), 10, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                0, None, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_decode_multi(cp, C.byref(b), 10, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                0, None, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_decode_multi(cp, C.byref(b), 4094, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None, 0, None, FAKE, 1 << 30, None) == qb.QSA_ERR_CAPACITY
    assert lib.qsa_decode_multi(cp, C.byref(b), 1000, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 200, None, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    # prefill attention / step: unknown flags, the union form's shape limits and workspace
    U = qb.QSA_PREFILL_GROUPED_UNION
    assert lib.qsa_prefill_attn(cp, FAKE, 8, 100, FAKE, 512, FAKE, FAKE, FAKE, 6, FAKE, 1 << 30,
                                None) == qb.QSA_ERR_INVALID
    assert lib.qsa_prefill_attn(cp, FAKE, 8, 100, FAKE, 512, FAKE, FAKE, FAKE, U, FAKE, 64,
                                None) == qb.QSA_ERR_CAPACITY
    assert lib.qsa_prefill_attn(cp, FAKE, 8, 100, FAKE, 512, FAKE, FAKE, FAKE, U, None, 1 << 30,
                                None) == qb.QSA_ERR_INVALID
    for kw in (dict(d=64, dv=64), dict(hq=8, hkv=4), dict(hq=32, hkv=1),
               dict(hq=16, hkv=4, topk_blocks=1024)):
        c2 = cfg(cap_tokens=4096, **kw).c()
        assert lib.qsa_prefill_attn(C.byref(c2), FAKE, 8, 100, FAKE, c2.topk_blocks, FAKE, FAKE,
                                    FAKE, U, FAKE, 1 << 30, None) == qb.QSA_ERR_UNSUPPORTED, kw
        assert lib.qsa_prefill_step(C.byref(c2), C.byref(b), 100, 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None, 0, None, U, FAKE, 1 << 30, None) == \
            qb.QSA_ERR_UNSUPPORTED, kw
    assert lib.qsa_prefill_step(cp, C.byref(b), 100, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                0, None, 4, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    # the union-for-every-group flag needs the grouped-union flag
    assert lib.qsa_prefill_step(cp, C.byref(b), 100, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                0, None, qb.QSA_PREFILL_UNION_ALL, FAKE, 1 << 30, None) == \
        qb.QSA_ERR_INVALID
    assert lib.qsa_prefill_attn(cp, FAKE, 8, 100, FAKE, 512, FAKE, FAKE, FAKE,
                                qb.QSA_PREFILL_UNION_ALL, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID


def test_mla_preconditions(lib):
    ws = 1 << 30
    args = lambda n, cap, mask=FAKE, dkq=576, dv=512, hq=16: (
        FAKE, hq, FAKE, None, dkq, dv, mask, n, cap, 0.05, None, FAKE, FAKE, FAKE, ws, None)
    assert lib.qsa_mla_sparse_attn(*args(262144, 2048, mask=None)) == qb.QSA_ERR_UNSUPPORTED
    assert lib.qsa_mla_sparse_attn(*args(2048, 512)) == qb.QSA_ERR_UNSUPPORTED      # n < 4096
    assert lib.qsa_mla_sparse_attn(*args(6000, 3001)) == qb.QSA_ERR_UNSUPPORTED     # n < 2 cap
    assert lib.qsa_mla_sparse_attn(*args(8192, 1024, dkq=512)) == qb.QSA_ERR_UNSUPPORTED
    assert lib.qsa_mla_sparse_attn(*args(8192, 1024, hq=12)) == qb.QSA_ERR_UNSUPPORTED
    # the capacity check after a list call rejects bad arguments on the host
    assert lib.qsa_mla_list_status(None, 2048, None, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_mla_list_status(FAKE, 0, None, None) == qb.QSA_ERR_INVALID


def test_trace_scan_arguments(lib):
    # both events or neither; a decode step that fails on the host clears the
    # setting, so a later step does not record stale events
    assert lib.qsa_trace_scan(FAKE, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_trace_scan(None, FAKE) == qb.QSA_ERR_INVALID
    assert lib.qsa_trace_scan(None, None) == qb.QSA_OK
    assert lib.qsa_trace_scan(FAKE, FAKE) == qb.QSA_OK
    c = cfg(cap_tokens=4096).c()
    assert lib.qsa_decode_step(C.byref(c), None, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               None, 0, FAKE, 1 << 30, None) == qb.QSA_ERR_INVALID
    assert lib.qsa_trace_scan(None, None) == qb.QSA_OK
