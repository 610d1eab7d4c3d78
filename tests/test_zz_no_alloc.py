"""The decode step that allocates nothing (qsa_decode_step_noalloc, static scratch in
the library) against the decode step with a caller workspace, through the C ABI."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_qsa_amd import binding as qb
import synth
from _helpers import dev, host

pytestmark = pytest.mark.gpu


def small(n_tokens, **kw):
    base = dict(h_idx=16, d_idx=128, topk=512, hq=32, hkv=4, d=128, dv=128)
    base.update(kw)
    return synth.Workload(f"noalloc_{n_tokens}", 11, "decode", n_tokens, **base)


def two_layers(w):
    """Two identical GPU layer states (each entry point appends to its own)."""
    L = synth.decode_layer(w, 0)
    n0 = L["n_prefix"]
    cfg = qb.Config(h_idx=w.h_idx, d_idx=w.d_idx, topk_blocks=w.topk, hq=w.hq, hkv=w.hkv,
                    d=w.d, dv=w.dv, cap_tokens=w.cap_tokens)
    layers = []
    for _ in range(2):
        g = qb.Layer(cfg)
        qb.qsa_pool_append(cfg, dev(L["raw"]), 0, g.k_raw, g.k_pool)
        g.k_cache[:n0] = dev(L["k"])
        g.v_cache[:n0] = dev(L["v"])
        layers.append(g)
    return L, cfg, layers


def step_both(w, L, cfg, layers, step):
    """The same step through both entry points; outputs, scores and chosen ids."""
    n0 = L["n_prefix"]
    nb = (n0 + step + 1) // 4
    res = []
    for i, g in enumerate(layers):
        out = torch.full((w.hq, w.dv), 9.0, device="cuda")
        scores = torch.full((max(nb, 1),), 9.0, device="cuda")
        blk = torch.full((w.topk,), -1, dtype=torch.int32, device="cuda")
        args = (cfg, g, n0 + step, dev(L["q_idx"]), dev(L["k_idx_new"][step]), dev(L["q"]),
                dev(L["k_new"][step]), dev(L["v_new"][step]), out)
        if i == 0:
            ws = qb.workspace(cfg, 1, w.cap_tokens)
            qb.qsa_decode_step(*args, ws, scores_out=scores, blk_out=blk)
        else:
            qb.qsa_decode_step_noalloc(*args, scores_out=scores, blk_out=blk)
        torch.cuda.synchronize()
        res.append((host(out), host(scores)[:nb], host(blk)[:min(w.topk, nb)]))
    return res


def test_noalloc_step_equals_workspace_step_twice_shrinking(gpu):
    # two calls in a row on the shared static scratch, the second on a smaller
    # context (fewer blocks, fewer cells); then the first shape again: the same
    # kernels on the same inputs give the same bits as the workspace form
    for n_tokens, k, steps in [(4 * 20000 + 1, 512, 4), (4 * 1500 + 3, 64, 2),
                               (4 * 20000 + 1, 512, 1)]:
        w = small(n_tokens, topk=k)
        L, cfg, layers = two_layers(w)
        for step in range(steps):
            (o0, s0, b0), (o1, s1, b1) = step_both(w, L, cfg, layers, step)
            assert np.array_equal(b0, b1), (n_tokens, step)
            assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), (n_tokens, step)
            assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), (n_tokens, step)


def test_noalloc_compact_gather_and_rejections(gpu):
    w = small(4 * 3000 + 2)
    L, cfg, layers = two_layers(w)
    n0 = L["n_prefix"]
    outs = []
    for g in layers:
        out = torch.empty((w.hq, w.dv), device="cuda")
        qb.qsa_decode_step_noalloc(cfg, g, n0, dev(L["q_idx"]), dev(L["k_idx_new"][0]),
                                   dev(L["q"]), dev(L["k_new"][0]), dev(L["v_new"][0]), out,
                                   flags=qb.QSA_STEP_COMPACT_GATHER)
        outs.append(host(out))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    # a shape whose scratch exceeds the static array is refused before any work
    big = qb.Config(h_idx=16, d_idx=128, topk_blocks=1024, hq=1024, hkv=64, d=128, dv=128,
                    cap_tokens=1 << 21)
    assert qb.qsa_workspace_size(big, 1, 1 << 20) > qb.QSA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(qb.QsaError) as e:
        qb.qsa_decode_step_noalloc(big, layers[0], (1 << 20) - 1, dev(L["q_idx"]),
                                   dev(L["k_idx_new"][0]), dev(L["q"]), dev(L["k_new"][0]),
                                   dev(L["v_new"][0]), torch.empty((1024, 128), device="cuda"))
    assert e.value.status == qb.QSA_ERR_CAPACITY
