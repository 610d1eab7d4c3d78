"""GPU parity of the MLA-style list attention (mask -> 64-bit ballot list ->
attention over the listed rows of one shared latent KV head)."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_qsa_amd import binding as qb
import synth
from _helpers import assert_attn_close, dev, host

pytestmark = pytest.mark.gpu


def run_mla(q, kv, mask, list_cap, scale, v=None):
    hq = q.shape[0]
    ws = torch.zeros(qb.qsa_mla_workspace_size(hq, 512, list_cap), dtype=torch.uint8,
                     device="cuda")
    qb.qsa_workspace_init(ws)
    out = torch.empty((hq, 512), device="cuda")
    lst = torch.full((list_cap,), -1, dtype=torch.int32, device="cuda")
    n_list = torch.zeros(1, dtype=torch.int32, device="cuda")
    qb.qsa_mla_sparse_attn(dev(q), dev(kv), None if v is None else dev(v), dev(mask), list_cap,
                           scale, n_list, out, ws, list_out=lst)
    return host(out), host(lst), int(host(n_list)[0]), ws


@pytest.mark.parametrize("runs", [False, True])
def test_mla_full_workload(gpu, runs):
    w = synth.WORKLOADS["mla_list_262144"]
    I = synth.mla_inputs(w, runs=runs)
    scale = 1.0 / np.sqrt(576)
    out, lst, nl, ws = run_mla(I["q"], I["kv"], I["mask"], w.list_len, scale)
    ref_list = np.flatnonzero(I["mask"] != -np.inf)
    n_list = torch.tensor([nl], dtype=torch.int32, device="cuda")
    assert qb.qsa_mla_list_status(n_list, w.list_len) == w.list_len
    assert nl == ref_list.size == w.list_len
    assert np.array_equal(lst[:nl], ref_list)
    assert np.array_equal(lst[:nl], O.mask_list(I["mask"]))
    ref = O.mla_attn(I["q"], I["kv"], None, I["mask"], ref_list, 512, scale)
    assert_attn_close(out, ref)


@pytest.mark.parametrize("hq", [1, 2, 4, 8, 16])
def test_mla_head_counts_and_separate_v(gpu, hq):
    n = 8192
    r = np.random.default_rng(hq)
    kv = synth.normal_f16(70 + hq, (n, 576))
    q = synth.normal_f16(80 + hq, (hq, 576))
    v = synth.normal_f16(90 + hq, (n, 512))
    mask = np.full(n, -np.inf, np.float16)
    pos = np.sort(r.choice(n, 700, replace=False))
    mask[pos] = r.choice([0.0, -1.0, 0.5], pos.size).astype(np.float16)
    for vv in (None, v):
        out, lst, nl, _ = run_mla(q, kv, mask, 1024, 0.04, v=vv)
        assert nl == 700 and np.array_equal(lst[:nl], pos)
        ref = O.mla_attn(q, kv, vv, mask, pos, 512, 0.04)
        assert_attn_close(out, ref)


def test_mla_edges(gpu):
    n = 4096
    kv = synth.normal_f16(71, (n, 576))
    q = synth.normal_f16(72, (16, 576))
    # first and last positions, a full 64-lane word, lanes 32..63 of a word
    mask = np.full(n, -np.inf, np.float16)
    pos = np.array([0, *range(128, 192), *range(288, 320), n - 1])
    mask[pos] = 0.0
    out, lst, nl, _ = run_mla(q, kv, mask, 2048, 0.05)
    assert nl == pos.size and np.array_equal(lst[:nl], pos)
    assert_attn_close(out, O.mla_attn(q, kv, None, mask, pos, 512, 0.05))
    # a single visible position returns its latent value row
    mask1 = np.full(n, -np.inf, np.float16)
    mask1[1234] = 0.0
    out1, _, nl1, _ = run_mla(q, kv, mask1, 64, 0.05)
    assert nl1 == 1
    assert np.allclose(out1, kv[1234, :512].astype(np.float32)[None], rtol=0, atol=1e-6)


def test_mla_list_overflow_reports_count_and_nan(gpu):
    n = 8192
    kv = synth.normal_f16(73, (n, 576))
    q = synth.normal_f16(74, (4, 576))
    mask = np.zeros(n, np.float16)  # everything visible
    mask[::3] = -np.inf
    visible = int(np.sum(mask != -np.inf))
    out, lst, nl, _ = run_mla(q, kv, mask, 1024, 0.05)
    assert nl == visible > 1024
    assert np.isnan(out).all()
    # the first list_cap entries are still the first visible positions
    assert np.array_equal(lst, np.flatnonzero(mask != -np.inf)[:1024])
    # the host-side status call reports the overflow as a capacity error
    n_list = torch.tensor([nl], dtype=torch.int32, device="cuda")
    with pytest.raises(qb.QsaError) as e:
        qb.qsa_mla_list_status(n_list, 1024)
    assert e.value.status == qb.QSA_ERR_CAPACITY
    assert qb.qsa_mla_list_status(n_list, visible) == visible


def test_mla_nothing_visible(gpu):
    n = 4096
    kv = synth.normal_f16(75, (n, 576))
    q = synth.normal_f16(76, (2, 576))
    mask = np.full(n, -np.inf, np.float16)
    out, _, nl, _ = run_mla(q, kv, mask, 128, 0.05)
    assert nl == 0
    # softmax over an empty set: the oracle's 0/0 is NaN, and so is the kernel's
    ref = O.mla_attn(q, kv, None, mask, np.zeros(0, np.int32), 512, 0.05)
    assert np.isnan(ref).all() and np.isnan(out).all()


@pytest.mark.parametrize("list_cap", [64, 4096, 4160, 8192])
def test_mla_list_forms(gpu, list_cap):
    # list capacities of one and of several 64-slot chunks per attention work group,
    # with the caller's list or without it: the same list, count and attention
    n = 2 * list_cap if list_cap >= 4096 else 8192
    r = np.random.default_rng(list_cap)
    kv = synth.normal_f16(200 + list_cap % 97, (n, 576))
    q = synth.normal_f16(300 + list_cap % 89, (16, 576))
    mask = np.full(n, -np.inf, np.float16)
    # clustered and scattered positions: runs over several 1,024-position segments,
    # whole empty segments, single positions
    vis = min(list_cap, 3000)
    pos = np.sort(np.unique(np.concatenate([
        np.arange(100, 100 + vis // 2),
        r.choice(np.arange(5000, n), vis - vis // 2, replace=False)])))[:vis]
    mask[pos] = 0.0
    scale = 1.0 / np.sqrt(576)
    out, lst, nl, _ = run_mla(q, kv, mask, list_cap, scale)
    assert nl == pos.size and np.array_equal(lst[:nl], pos)
    ref = O.mla_attn(q, kv, None, mask, pos, 512, scale)
    assert_attn_close(out, ref)
    # no list output requested: the same count and attention
    ws = torch.zeros(qb.qsa_mla_workspace_size(16, 512, list_cap), dtype=torch.uint8,
                     device="cuda")
    qb.qsa_workspace_init(ws)
    out2 = torch.empty((16, 512), device="cuda")
    n_list = torch.zeros(1, dtype=torch.int32, device="cuda")
    qb.qsa_mla_sparse_attn(dev(q), dev(kv), None, dev(mask), list_cap, scale, n_list, out2, ws)
    assert int(host(n_list)[0]) == pos.size
    assert np.array_equal(host(out2), out)
