"""GPU parity of the decode path against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_qsa_amd import binding as qb
import synth
from _helpers import (SCORE_ABS_REL, SCORE_REL, assert_attn_close, assert_pool_close, cfg_of,
                      dev, host, setup_decode, shape_of)

pytestmark = pytest.mark.gpu


def small(n_tokens, **kw):
    base = dict(h_idx=16, d_idx=128, topk=512, hq=32, hkv=4, d=128, dv=128)
    base.update(kw)
    return synth.Workload(f"small_{n_tokens}", 7, "decode", n_tokens, **base)


# ------------------------------------------------------------------ a1 pool append
@pytest.mark.parametrize("H,d,n", [(16, 128, 4 * 700 + 3), (4, 64, 4 * 1000 + 1), (1, 128, 77),
                                   (32, 64, 130), (8, 256, 41)])
def test_pool_append_matches_oracle(gpu, H, d, n):
    cfg = qb.Config(h_idx=H, d_idx=d, topk_blocks=8, hq=8, hkv=1, d=128, dv=128,
                    cap_tokens=((n + 8) // 4) * 4)
    raw = synth.normal_f16(11, (n, H, d))
    w = torch.linspace(0.5, 1.5, d, dtype=torch.float32)
    for rms in (None, w):
        g = qb.Layer(cfg, rms_w=rms)
        qb.qsa_pool_append(cfg, dev(raw), 0, g.k_raw, g.k_pool, g.rms_w)
        ref = O.pool_rebuild(raw, n, w=None if rms is None else rms.numpy())
        got = host(g.k_pool[:n // 4])
        assert_pool_close(got, ref)
        assert np.array_equal(host(g.k_raw[:n]).view(np.uint16), raw.view(np.uint16))
        assert not host(g.k_pool[n // 4:]).any()  # incomplete block untouched


def test_incremental_append_is_bitwise_chunk_append(gpu):
    H, d, n = 16, 128, 4 * 300 + 2
    cfg = qb.Config(h_idx=H, d_idx=d, cap_tokens=1216)
    raw = synth.normal_f16(12, (n, H, d))
    a = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(raw), 0, a.k_raw, a.k_pool)
    b = qb.Layer(cfg)
    for t in range(n):
        qb.qsa_pool_append(cfg, dev(raw[t:t + 1]), t, b.k_raw, b.k_pool)
    c = qb.Layer(cfg)
    r = np.random.default_rng(3)
    t = 0
    while t < n:
        k = int(min(n - t, r.integers(1, 23)))
        qb.qsa_pool_append(cfg, dev(raw[t:t + k]), t, c.k_raw, c.k_pool)
        t += k
    pa = host(a.k_pool).view(np.uint16)
    assert np.array_equal(pa, host(b.k_pool).view(np.uint16))
    assert np.array_equal(pa, host(c.k_pool).view(np.uint16))


@pytest.mark.parametrize("hkv,d,dv,n_before,n_new", [(4, 128, 128, 0, 1), (4, 128, 128, 1003, 37),
                                                     (1, 64, 64, 4000, 96), (2, 64, 64, 17, 1)])
def test_kv_append_is_an_exact_copy(gpu, hkv, d, dv, n_before, n_new):
    # byte work: the new rows land bit for bit at [n_before, n_before + n_new); every
    # other row keeps its contents
    cap = 4160
    cfg = qb.Config(hq=hkv * 8, hkv=hkv, d=d, dv=dv, cap_tokens=cap)
    k_new = synth.normal_f16(120 + n_new, (n_new, hkv, d))
    v_new = synth.normal_f16(121 + n_new, (n_new, hkv, dv))
    kc0 = synth.normal_f16(122, (cap, hkv, d))
    vc0 = synth.normal_f16(123, (cap, hkv, dv))
    kc, vc = dev(kc0), dev(vc0)
    qb.qsa_kv_append(cfg, dev(k_new), dev(v_new), n_before, kc, vc)
    ek, ev = kc0.copy(), vc0.copy()
    ek[n_before:n_before + n_new] = k_new
    ev[n_before:n_before + n_new] = v_new
    assert np.array_equal(host(kc).view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(host(vc).view(np.uint16), ev.view(np.uint16))


# ------------------------------------------------------------------ cache lifecycle
def test_pool_rebuild_after_state_load_and_edit(gpu):
    # a state load (only the raw keys restored) and a sequence edit from token t on:
    # rebuilding from block 0 / from block t // 4 gives the bits of a fresh append
    H, d, n = 16, 128, 4 * 900 + 3
    cfg = qb.Config(h_idx=H, d_idx=d, cap_tokens=4 * 904)
    raw = synth.normal_f16(13, (n, H, d))
    ref = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(raw), 0, ref.k_raw, ref.k_pool)
    loaded = qb.Layer(cfg)
    loaded.k_raw[:n] = dev(raw)
    loaded.k_pool.fill_(7.0)  # stale content from before the load
    qb.qsa_pool_rebuild(cfg, loaded.k_raw, loaded.k_pool, 0, n)
    nb = n // 4
    assert np.array_equal(host(loaded.k_pool[:nb]).view(np.uint16),
                          host(ref.k_pool[:nb]).view(np.uint16))
    assert np.all(host(loaded.k_pool[nb:]) == 7.0)  # the incomplete block is not touched
    # edit tokens [t, n) and rebuild from the block holding t
    t = 4 * 517 + 2
    edited = raw.copy()
    edited[t:] = synth.normal_f16(14, (n - t, H, d))
    loaded.k_raw[t:n] = dev(edited[t:])
    qb.qsa_pool_rebuild(cfg, loaded.k_raw, loaded.k_pool, t // 4, n)
    fresh = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(edited), 0, fresh.k_raw, fresh.k_pool)
    assert np.array_equal(host(loaded.k_pool[:nb]).view(np.uint16),
                          host(fresh.k_pool[:nb]).view(np.uint16))
    assert_pool_close(host(loaded.k_pool[:nb]), O.pool_rebuild(edited, n))


def test_speculative_rollback_needs_no_rebuild(gpu):
    # decode steps append 4 draft tokens that complete a block, the drafts are
    # rejected (the count rolls back), other tokens are decoded in their place: the
    # caches and every step's output equal those of a run that never saw the drafts
    w = small(4 * 2000 + 1)
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]                        # 8000 tokens: block 1999 is complete
    drafts = synth.normal_f16(70, (4, 16, 128))
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    out = torch.empty((w.hq, w.dv), device="cuda")
    for j in range(4):  # positions n0 .. n0 + 3; the last one completes block 2000
        qb.qsa_decode_step(cfg, g, n0 + j, dev(L["q_idx"]), dev(drafts[j]), dev(L["q"]),
                           dev(L["k_new"][j]), dev(L["v_new"][j]), out, ws)
    assert host(g.k_pool[2000]).any()
    # rejected: decode the accepted tokens from position n0 again
    for step in range(4):
        check_step(w, L, cfg, g, o, n0 + step, step, qb.QSA_STEP_FUSED_GATHER)
    clean = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(L["raw"]), 0, clean.k_raw, clean.k_pool)
    qb.qsa_pool_append(cfg, dev(L["k_idx_new"]), n0, clean.k_raw, clean.k_pool)
    nb = (n0 + 4) // 4
    assert np.array_equal(host(g.k_pool[:nb]).view(np.uint16),
                          host(clean.k_pool[:nb]).view(np.uint16))


def test_trace_scan_events_leave_the_step_unchanged(gpu):
    # events handed to the scoring launch of a step: the step's results are bit for
    # bit those of an untraced step at the same position, the events carry a
    # positive kernel time within the whole step's, and the next step is untraced
    w = small(4 * 20000 + 3)
    L, cfg, g, _ = setup_decode(w, with_oracle=False)
    n0 = L["n_prefix"]
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    nb = (n0 + 1) // 4
    res = []
    for traced in (True, False, True):
        out = torch.empty((w.hq, w.dv), device="cuda")
        scores = torch.empty(nb, device="cuda")
        blk = torch.full((512,), -1, dtype=torch.int32, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record()  # creates the events
        if traced:
            qb.qsa_trace_scan(ev[0], ev[1])
        ev[2].record()
        qb.qsa_decode_step(cfg, g, n0, dev(L["q_idx"]), dev(L["k_idx_new"][0]), dev(L["q"]),
                           dev(L["k_new"][0]), dev(L["v_new"][0]), out, ws, scores_out=scores,
                           blk_out=blk)
        ev[3].record()
        torch.cuda.synchronize()
        step_ms = ev[2].elapsed_time(ev[3])
        if traced:
            scan_ms = ev[0].elapsed_time(ev[1])
            assert 0.0 < scan_ms < step_ms, (scan_ms, step_ms)
        res.append((host(out), host(scores), host(blk)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for a, b in zip(res[0], res[2]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    b = host(blk)
    assert np.array_equal(b, O.topk_sort(res[0][1], 512))


# ------------------------------------------------------------------ a2 scores
@pytest.mark.parametrize("H,d,nb", [(16, 128, 3001), (4, 64, 1024), (16, 128, 1), (2, 64, 333),
                                    (8, 128, 2047), (32, 128, 100)])
def test_index_score_decode(gpu, H, d, nb):
    cfg = qb.Config(h_idx=H, d_idx=d, cap_tokens=4 * nb + 64)
    P = synth.normal_f16(20, (nb, H, d))
    q = synth.normal_f16(21, (H, d))
    pool = torch.zeros((cfg.cap_tokens // 4, H, d), dtype=torch.float16, device="cuda")
    pool[:nb] = dev(P)
    s = torch.full((nb + 7,), 12345.0, device="cuda")
    qb.qsa_index_score(cfg, dev(q), 4 * nb + 2, pool, s, ld=nb + 7)
    got = host(s)
    s64, _ = O.index_score(q, P, nb)
    bound = SCORE_ABS_REL * (np.abs(P.astype(np.float64).reshape(nb, -1)) @
                             np.abs(q.astype(np.float64).ravel()))
    assert np.all(np.abs(got[:nb] - s64) <= bound)
    assert np.all(got[nb:] == 12345.0)  # nothing written past the complete blocks


# ------------------------------------------------------------------ a3 top-k (decode form)
def run_topk_decode(scores, k):
    nb = scores.size
    cfg = qb.Config(topk_blocks=k, cap_tokens=4 * nb + 64)
    ws = qb.workspace(cfg, 1, 4 * nb + 3)
    blk = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the row at position 4*nb + 2 sees exactly nb complete blocks
    qb.qsa_topk_blocks(cfg, dev(scores.astype(np.float32)), 1, nb, 4 * nb + 2, blk, nsel, ws)
    n = int(host(nsel)[0])
    return host(blk)[:n], n, ws


def crafted(nb, kind, r):
    if kind == "normal":
        return r.standard_normal(nb).astype(np.float32) * 45
    if kind == "all_equal":
        return np.full(nb, 3.25, np.float32)
    if kind == "few_values":
        return r.integers(-3, 4, nb).astype(np.float32)
    if kind == "zeros_signed":
        s = np.zeros(nb, np.float32)
        s[r.random(nb) < 0.5] = -0.0
        s[r.random(nb) < 0.01] = 1.0
        return s
    if kind == "nan_inf":
        s = r.standard_normal(nb).astype(np.float32)
        s[r.random(nb) < 0.05] = np.nan
        s[r.random(nb) < 0.01] = np.inf
        s[r.random(nb) < 0.01] = -np.inf
        return s
    if kind == "tie_at_cut":
        s = r.standard_normal(nb).astype(np.float32)
        order = np.argsort(-s)
        s[order[500:530]] = s[order[505]]
        return s
    if kind == "narrow":   # everything in one 12-bit bin: candidate path overflows LDS
        return (1.0 + r.random(nb).astype(np.float32) * 1e-3).astype(np.float32)
    if kind == "ascending":  # every candidate in the last regions of the row
        return np.sort(r.standard_normal(nb).astype(np.float32) * 45)
    if kind == "sample_misleads":  # the sampled scores alone sit far above the rest
        s = r.standard_normal(nb).astype(np.float32)
        stride = max(64, -(-nb // 1024))
        s[:40 * stride:stride] = 1000.0
        return s
    if kind == "crowded_bin":  # the threshold bin holds more than 1024 keys
        s = r.standard_normal(nb).astype(np.float32) * 45
        idx = r.choice(nb, min(1500, nb // 2), replace=False)
        s[idx] = (1000.0 + r.random(idx.size) * 0.1).astype(np.float32)
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "all_equal", "few_values", "zeros_signed", "nan_inf",
                                  "tie_at_cut", "narrow", "ascending", "sample_misleads",
                                  "crowded_bin"])
@pytest.mark.parametrize("nb", [513, 5000, 20000, 40000, 63795, 65536, 70001])
def test_topk_decode_bit_exact(gpu, kind, nb):
    r = np.random.default_rng(nb + len(kind))
    s = crafted(nb, kind, r)
    got, n, ws = run_topk_decode(s, 512)
    assert n == 512
    assert np.array_equal(got, O.topk_sort(s, 512))


@pytest.mark.parametrize("nb,k", [(1, 512), (512, 512), (511, 512), (0, 4), (100, 99), (100, 1)])
def test_topk_decode_small_and_edges(gpu, nb, k):
    r = np.random.default_rng(nb * 7 + k)
    s = r.standard_normal(max(nb, 1)).astype(np.float32)[:nb]
    if nb == 0:
        cfg = qb.Config(topk_blocks=k, cap_tokens=64)
        ws = qb.workspace(cfg, 1, 3)
        blk = torch.full((k,), -7, dtype=torch.int32, device="cuda")
        nsel = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        qb.qsa_topk_blocks(cfg, torch.zeros(4, device="cuda"), 1, 4, 2, blk, nsel, ws)
        assert int(host(nsel)[0]) == 0
        return
    got, n, _ = run_topk_decode(s, k)
    assert n == min(k, nb)
    assert np.array_equal(got, O.topk_sort(s, k))


def test_topk_decode_repeated_calls_share_workspace(gpu):
    r = np.random.default_rng(5)
    nb = 20000
    cfg = qb.Config(topk_blocks=512, cap_tokens=4 * nb + 64)
    ws = qb.workspace(cfg, 1, 4 * nb + 3)
    blk = torch.zeros(512, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(6):
        s = crafted(nb, ["normal", "few_values", "narrow"][i % 3], r)
        qb.qsa_topk_blocks(cfg, dev(s), 1, nb, 4 * nb + 2, blk, nsel, ws)
        assert np.array_equal(host(blk), O.topk_sort(s, 512))


# ------------------------------------------------------------------ a4 gather + a5 attention
@pytest.mark.parametrize("n_tokens", [4 * 3000 + 1, 4 * 3000 + 3, 4 * 3000, 4 * 100 + 2, 3])
def test_gather_and_sparse_attn(gpu, n_tokens):
    w = small(n_tokens)
    cfg = cfg_of(w)
    r = np.random.default_rng(n_tokens)
    K = synth.normal_f16(30, (n_tokens, 4, 128))
    V = synth.normal_f16(31, (n_tokens, 4, 128))
    q = synth.normal_f16(32, (32, 128))
    nb = n_tokens // 4
    nsel = min(512, nb)
    blk = np.sort(r.choice(nb, nsel, replace=False)).astype(np.int32) if nb else \
        np.zeros(0, np.int32)
    cells = O.cells(blk, n_tokens)
    kc, vc = dev(K), dev(V)
    ks = torch.zeros((2051, 4, 128), dtype=torch.float16, device="cuda")
    vs = torch.zeros_like(ks)
    qb.qsa_gather_kv(cfg, dev(blk) if nsel else torch.zeros(1, dtype=torch.int32, device="cuda"),
                     nsel, n_tokens, kc, vc, ks, vs)
    nc = cells.size
    assert np.array_equal(host(ks[:nc]).view(np.uint16), K[cells].view(np.uint16))
    assert np.array_equal(host(vs[:nc]).view(np.uint16), V[cells].view(np.uint16))
    ws = qb.workspace(cfg, 1, n_tokens)
    out = torch.empty((32, 128), device="cuda")
    qb.qsa_sparse_attn(cfg, dev(q), ks, vs, nc, out, ws)
    ref = O.attn_cells(q, K, V, cells, w.scale)
    assert_attn_close(host(out), ref)


@pytest.mark.parametrize("hq,hkv,d", [(8, 1, 128), (16, 16, 64), (16, 1, 64), (4, 2, 128),
                                      (32, 2, 128)])
def test_sparse_attn_head_layouts(gpu, hq, hkv, d):
    cfg = qb.Config(h_idx=16, d_idx=128, topk_blocks=64, hq=hq, hkv=hkv, d=d, dv=d,
                    cap_tokens=1024)
    nc = 4 * 64 + 3
    K = synth.normal_f16(40, (nc, hkv, d))
    V = synth.normal_f16(41, (nc, hkv, d))
    q = synth.normal_f16(42, (hq, d))
    ws = qb.workspace(cfg, 1, 1000)
    out = torch.empty((hq, d), device="cuda")
    qb.qsa_sparse_attn(cfg, dev(q), dev(K), dev(V), nc, out, ws)
    ref = O.attn_cells(q, K, V, np.arange(nc), 1 / np.sqrt(d))
    assert_attn_close(host(out), ref)


# ------------------------------------------------------------------ a6 decode step
def check_step(w, L, cfg, g, o, n_before, step, flags):
    nb = (n_before + 1) // 4
    out = torch.empty((w.hq, w.dv), device="cuda")
    scores = torch.empty(max(nb, 1), device="cuda")
    blk = torch.full((w.topk,), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    qb.qsa_decode_step(cfg, g, n_before, dev(L["q_idx"]), dev(L["k_idx_new"][step]), dev(L["q"]),
                       dev(L["k_new"][step]), dev(L["v_new"][step]), out, ws, scores_out=scores,
                       blk_out=blk, flags=flags)
    ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, n_before, L["q_idx"],
                        L["k_idx_new"][step], L["q"], L["k_new"][step], L["v_new"][step])
    s_gpu = host(scores)[:nb]
    if nb:
        assert np.max(np.abs(s_gpu - ref["scores64"])) <= SCORE_REL * np.max(np.abs(ref["scores64"]))
    nsel = min(w.topk, nb)
    b_gpu = host(blk)[:nsel]
    assert np.array_equal(b_gpu, O.topk_sort(s_gpu, w.topk))
    # end to end: blocks that differ from the oracle's own choice sit at the cut
    diff = set(b_gpu.tolist()) ^ set(ref["blk"].tolist())
    if diff and nb > w.topk:
        kth = np.sort(ref["scores64"])[::-1][w.topk - 1]
        for b in diff:
            assert abs(ref["scores64"][b] - kth) <= SCORE_REL * np.max(np.abs(ref["scores64"]))
    cells = O.cells(b_gpu, n_before + 1)
    ref_out = O.attn_cells(L["q"], o.k, o.v, cells, w.scale)
    assert_attn_close(host(out), ref_out)
    return b_gpu


@pytest.mark.parametrize("flags", [qb.QSA_STEP_FUSED_GATHER, qb.QSA_STEP_COMPACT_GATHER])
def test_decode_step_tiny_workload(gpu, flags):
    w = synth.WORKLOADS["tiny_decode_4k"]
    L, cfg, g, o = setup_decode(w)
    check_step(w, L, cfg, g, o, L["n_prefix"], 0, flags)
    # the step completed block 1023: the GPU's new pooled row matches the oracle's
    assert_pool_close(host(g.k_pool[1023]), o.pooled[1023])


@pytest.mark.parametrize("name,flags", [("decode_61789", qb.QSA_STEP_FUSED_GATHER),
                                        ("decode_61789", qb.QSA_STEP_COMPACT_GATHER),
                                        ("decode_126253", qb.QSA_STEP_FUSED_GATHER)])
def test_decode_step_cycle(gpu, name, flags):
    # the 64k and 128k workloads, 4 consecutive steps: the tail lengths of the cycle
    # and a completed block
    w = synth.WORKLOADS[name]
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    for step in range(4):
        check_step(w, L, cfg, g, o, n0 + step, step, flags)
    nb = (n0 + 4) // 4
    assert_pool_close(host(g.k_pool[nb - 1]), o.pooled[nb - 1])
    assert np.array_equal(host(g.k_raw[n0:n0 + 4]).view(np.uint16),
                          L["k_idx_new"].view(np.uint16))


def random_decode_config(seed):
    """A seeded draw over the configurations the step supports: indexer rows of
    16..512 sixteen-byte pieces, 1..16 query heads per KV head, head dims 64 or 128,
    k from 1 to 1,024, contexts from 2 to 24,000 tokens, either gather form."""
    rng = np.random.default_rng(9000 + seed)
    d_idx = int(rng.choice([16, 32, 64, 128, 256]))
    rowc = int(rng.choice([r for r in (16, 32, 64, 128, 256, 512) if r * 8 >= d_idx]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h * G <= 64]))
    d = int(rng.choice([64, 128]))
    topk = int(rng.choice([1, 3, 64, 200, 512, 1024]))
    n_tokens = int(rng.integers(2, 24000))
    flags = qb.QSA_STEP_FUSED_GATHER if seed % 3 else qb.QSA_STEP_COMPACT_GATHER
    w = synth.Workload(f"random_{seed}", 500 + seed, "decode", n_tokens, h_idx=rowc * 8 // d_idx,
                       d_idx=d_idx, topk=topk, hq=hkv * G, hkv=hkv, d=d, dv=d)
    return w, flags


@pytest.mark.parametrize("seed", range(24))
def test_decode_step_random_configs(gpu, seed):
    # two consecutive steps of a drawn configuration (the second one completes a
    # block in a quarter of the draws), each against the oracle
    w, flags = random_decode_config(seed)
    print(f"config {w}", flush=True)
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    for step in range(2):
        check_step(w, L, cfg, g, o, n0 + step, step, flags)


def test_decode_step_small_contexts(gpu):
    # nb <= k (full attention), N < 4 (no complete block), k = nb - 1
    for n_tokens, k in [(1, 512), (3, 512), (4, 512), (2049, 512), (2053, 512), (401, 99)]:
        w = small(n_tokens, topk=k)
        L, cfg, g, o = setup_decode(w)
        check_step(w, L, cfg, g, o, L["n_prefix"], 0, qb.QSA_STEP_FUSED_GATHER)


def test_decode_step_k1024_one_kv_head_cycle(gpu):
    # k = 1024 with one KV head: up to 4 * 1024 + 3 = 4099 cells, 65 chunks of 64,
    # more than the 64 splits one work group per chunk would need; every position
    # of the 4-step cycle (tails 1, 2, 3 and a completed block)
    w = small(4 * 3000 + 1, topk=1024, hq=8, hkv=1)
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    for step in range(4):
        check_step(w, L, cfg, g, o, n0 + step, step, qb.QSA_STEP_FUSED_GATHER)


@pytest.mark.parametrize("n_tokens", [4 * 3000 + 2, 4 * 3000 + 3])
def test_decode_multi_k1024_two_kv_heads(gpu, n_tokens):
    # two verification rows with k = 1024 and two KV heads: rows of 4097 .. 4099 cells
    w = small(n_tokens, topk=1024, hq=8, hkv=2)
    L, cfg, g, o = setup_decode(w)
    n0, n_q = L["n_prefix"], 2
    q_idx = synth.normal_f16(85, (n_q, 16, 128))
    q = synth.normal_f16(86, (n_q, 8, 128))
    out = torch.empty((n_q, 8, 128), device="cuda")
    ld = (n0 + n_q) // 4 + 3
    scores = torch.empty((n_q, ld), device="cuda")
    blk = torch.full((n_q, 1024), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, w.cap_tokens)
    qb.qsa_decode_multi(cfg, g, n0, dev(q_idx), dev(L["k_idx_new"][:n_q]), dev(q),
                        dev(L["k_new"][:n_q]), dev(L["v_new"][:n_q]), out, ws,
                        scores_out=scores, ld_scores=ld, blk_out=blk)
    for row in range(n_q):
        ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, n0 + row, q_idx[row],
                            L["k_idx_new"][row], q[row], L["k_new"][row], L["v_new"][row])
        nb = (n0 + row + 1) // 4
        s_gpu = host(scores[row])[:nb]
        assert np.max(np.abs(s_gpu - ref["scores64"])) <= SCORE_REL * np.max(np.abs(ref["scores64"]))
        b_gpu = host(blk[row])[:min(1024, nb)]
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, 1024)), row
        ref_out = O.attn_cells(q[row], o.k, o.v, O.cells(b_gpu, n0 + row + 1), w.scale)
        assert_attn_close(host(out[row]), ref_out, f"row {row}")


@pytest.mark.parametrize("layer", [0, 7])
def test_decode_step_255181_planted(gpu, layer):
    # the 256k workload, layer 0 and one other seeded layer: planted blocks are
    # chosen, full parity.  Layer 0 runs the whole cycle the benchmark times
    # (positions N-1 .. N+2: tails 1, 2, 3, then the step that completes a block)
    w = synth.WORKLOADS["decode_255181"]
    L, cfg, g, o = setup_decode(w, layer)
    n0 = L["n_prefix"]
    # pooled cache built by the library vs the oracle, on 2000 sampled rows
    rows = np.sort(np.random.default_rng(1).choice(n0 // 4, 2000, replace=False))
    assert_pool_close(host(g.k_pool[torch.from_numpy(rows).cuda()]), o.pooled[rows])
    for step in range(4 if layer == 0 else 1):
        b = check_step(w, L, cfg, g, o, n0 + step, step, qb.QSA_STEP_FUSED_GATHER)
        assert set(L["planted"].tolist()) <= set(b.tolist())
    if layer == 0:
        nb = (n0 + 4) // 4  # the block completed by the last step, pooled on the GPU
        assert_pool_close(host(g.k_pool[nb - 1]), o.pooled[nb - 1])


# ------------------------------------------------------------------ decode top-k on clustered scores
def clustered_values(pattern, nb, r):
    """Per-block values v_b; a pooled row of all v_b against an all-ones query scores
    exactly 2048 * v_b, on the GPU and in the oracle."""
    v = (np.round(r.standard_normal(nb) * 6.4) / 64).astype(np.float16)  # no subnormals
    if pattern == "one_scan_group":
        # the blocks b with b mod 3068 in [20, 24) on top: the decode scan's 767 scan
        # work groups read runs of 4 neighbouring rows (row b in work group
        # (b mod 3068) / 4), so these all belong to one work group, whose 8-entry
        # candidate list cannot hold them (full-row fallback)
        sel = (np.arange(nb) % 3068 >= 20) & (np.arange(nb) % 3068 < 24)
        v[sel] = (4.0 + np.arange(sel.sum()) / 64).astype(np.float16)
    elif pattern == "recent_window":
        v[-700:] = np.linspace(1.0, 2.0, 700).astype(np.float16)
    elif pattern == "ascending":
        v = np.sort(v)
    elif pattern == "all_equal":
        v[:] = 1.0
    elif pattern == "few_values":
        v = r.integers(-2, 3, nb).astype(np.float16)
    return v


@pytest.mark.parametrize("pattern", ["one_scan_group", "recent_window", "ascending", "all_equal",
                                     "few_values"])
def test_decode_step_clustered_scores(gpu, pattern):
    nb0, H, d = 20000, 16, 128
    n_before = 4 * nb0 + 3        # the step completes block nb0 (scored by the append)
    w = small(n_before + 1)
    cfg = cfg_of(w)
    r = np.random.default_rng(len(pattern))
    v = clustered_values(pattern, nb0, r)
    pooled = np.zeros((w.cap_tokens // 4, H, d), np.float16)
    pooled[:nb0] = v[:, None, None]
    raw = np.zeros((w.cap_tokens, H, d), np.float16)
    raw[4 * nb0:n_before] = synth.normal_f16(60, (3, H, d))
    K = synth.normal_f16(61, (w.cap_tokens, 4, 128))
    V = synth.normal_f16(62, (w.cap_tokens, 4, 128))
    K[n_before:] = 0
    V[n_before:] = 0
    q_idx = np.ones((H, d), np.float16)
    q = synth.normal_f16(63, (32, 128))
    k_idx_new = synth.normal_f16(64, (H, d))
    k_new, v_new = synth.normal_f16(65, (4, 128)), synth.normal_f16(66, (4, 128))

    g = qb.Layer(cfg)
    g.k_pool.copy_(dev(pooled))
    g.k_raw.copy_(dev(raw))
    g.k_cache.copy_(dev(K))
    g.v_cache.copy_(dev(V))
    out = torch.empty((32, 128), device="cuda")
    scores = torch.empty(nb0 + 1, device="cuda")
    blk = torch.full((512,), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    qb.qsa_decode_step(cfg, g, n_before, dev(q_idx), dev(k_idx_new), dev(q), dev(k_new),
                       dev(v_new), out, ws, scores_out=scores, blk_out=blk)
    ref = O.decode_step(shape_of(w), raw, pooled, K, V, n_before, q_idx, k_idx_new, q, k_new,
                        v_new)
    s_gpu = host(scores)
    # complete blocks score exactly; the appended one within the score bound
    assert np.array_equal(s_gpu[:nb0], 2048.0 * v.astype(np.float32))
    assert abs(s_gpu[nb0] - ref["scores64"][nb0]) <= SCORE_REL * np.max(np.abs(ref["scores64"]))
    b_gpu = host(blk)
    assert np.array_equal(b_gpu, O.topk_sort(s_gpu, 512))
    assert np.array_equal(b_gpu, ref["blk"])
    ref_out = O.attn_cells(q, K, V, O.cells(b_gpu, n_before + 1), w.scale)
    assert_attn_close(host(out), ref_out)


def scan_share_rows(b, nb, nwg, rpw):
    """Rows of the decode scan's work group b (of nwg): runs of 4 row groups of rpw
    rows at stride 4 nwg groups, in scan order."""
    g = np.arange((nb + rpw - 1) // rpw)
    rows = np.concatenate([np.arange(x * rpw, (x + 1) * rpw) for x in g if (x % (4 * nwg)) // 4 == b])
    return rows[rows < nb]


@pytest.mark.parametrize("H,d,nb0,n_groups,per_group,edges", [
    (16, 128, 20000, 1, 28, False),    # one work group's 26 rows all on top: widened
    (16, 128, 20000, 40, 12, False),   # 40 lists widened at once (160 spare threads)
    (4, 64, 20000, 3, 20, False),      # row groups of 2 rows (a 4 x 64 indexer)
    (2, 64, 20000, 5, 30, False),      # row groups of 4 rows (a 2 x 64 indexer)
    (2, 64, 20001, 4, 30, True),       # the first and last work groups; a partial last group
    (32, 128, 20000, 3, 24, False),    # rows of 512 16-byte pieces (a 32 x 128 indexer)
    (4, 64, 200000, 20, 20, False),    # 20 work groups of 264 rows do not fit: whole-row selection
])
def test_decode_step_hidden_rows(gpu, H, d, nb0, n_groups, per_group, edges):
    # the top of the score row crowds the shares of n_groups scan work groups (more
    # than 8 chosen rows each), so their 8-entry lists hide chosen rows: the tail
    # replaces those lists by all their rows, or selects from the whole score row
    # when the rows do not fit; the chosen ids equal the top-k of the GPU's scores.
    # edges: the chosen work groups include the first and the last two (whose
    # second run ends in the partial last row group when nb0 is not a multiple of
    # the group size)
    n_before = 4 * nb0 + 3  # the step completes block nb0
    w = small(n_before + 1, h_idx=H, d_idx=d, hq=8, hkv=1, d=64, dv=64)
    cfg = cfg_of(w)
    r = np.random.default_rng(nb0 + n_groups)
    v = (np.round(r.standard_normal(nb0) * 6.4) / 64).astype(np.float16)
    # the scan's layout: row groups of rpw rows (one wave-wide load per group), one
    # work group per 8 row groups, at most 767
    rpw = 64 // min(64, H * d // 8)
    nwg = min(767, -(-(-(-nb0 // rpw)) // 8))
    hi = []
    if edges:
        groups = [0, nwg - 1, nwg - 2] + r.choice(np.arange(1, nwg - 2), n_groups - 3,
                                                  replace=False).tolist()
        assert nb0 - 1 in scan_share_rows(nwg - 2, nb0, nwg, rpw)  # the partial group
    else:
        groups = r.choice(nwg, n_groups, replace=False).tolist()
    for b in groups:
        rows = scan_share_rows(int(b), nb0, nwg, rpw)
        assert rows.size > 8
        hi.extend(rows[:per_group].tolist())
    hi = np.array(hi)
    v[hi] = (4.0 + np.arange(hi.size) / 64).astype(np.float16)
    pooled = np.zeros((w.cap_tokens // 4, H, d), np.float16)
    pooled[:nb0] = v[:, None, None]
    raw = np.zeros((w.cap_tokens, H, d), np.float16)
    raw[4 * nb0:n_before] = synth.normal_f16(80, (3, H, d))
    K = synth.normal_f16(81, (w.cap_tokens, 1, 64))
    V = synth.normal_f16(82, (w.cap_tokens, 1, 64))
    K[n_before:] = 0
    V[n_before:] = 0
    q_idx = np.ones((H, d), np.float16)
    q = synth.normal_f16(83, (8, 64))
    k_idx_new = synth.normal_f16(84, (H, d))
    k_new, v_new = synth.normal_f16(85, (1, 64)), synth.normal_f16(86, (1, 64))

    g = qb.Layer(cfg)
    g.k_pool.copy_(dev(pooled))
    g.k_raw.copy_(dev(raw))
    g.k_cache.copy_(dev(K))
    g.v_cache.copy_(dev(V))
    out = torch.empty((8, 64), device="cuda")
    scores = torch.empty(nb0 + 1, device="cuda")
    blk = torch.full((512,), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    for flags in (qb.QSA_STEP_FUSED_GATHER, qb.QSA_STEP_COMPACT_GATHER):
        qb.qsa_decode_step(cfg, g, n_before, dev(q_idx), dev(k_idx_new), dev(q), dev(k_new),
                           dev(v_new), out, ws, scores_out=scores, blk_out=blk, flags=flags)
        s_gpu = host(scores)
        assert np.array_equal(s_gpu[:nb0], float(H * d) * v.astype(np.float32))
        b_gpu = host(blk)
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, 512)), flags
        assert set(hi.tolist()) <= set(b_gpu.tolist())
        ref_out = O.attn_cells(q, K, V, O.cells(b_gpu, n_before + 1), w.scale)
        assert_attn_close(host(out), ref_out, f"flags {flags}")


@pytest.mark.parametrize("pattern", ["one_scan_group", "recent_window", "all_equal",
                                     "few_values"])
def test_decode_multi_clustered_scores(gpu, pattern):
    # three rows with their own score orders over the same clustered blocks (query
    # all ones, all minus ones, half the features): each row's candidate lists come
    # from the same scan, and a row whose chosen blocks crowd one work group falls
    # back alone; row 2 completes block nb0, which only it sees
    nb0, H, d, n_q = 20000, 16, 128, 3
    n_before = 4 * nb0 + 1
    w = small(n_before + n_q)
    cfg = cfg_of(w)
    r = np.random.default_rng(100 + len(pattern))
    v = clustered_values(pattern, nb0, r)
    pooled = np.zeros((w.cap_tokens // 4, H, d), np.float16)
    pooled[:nb0] = v[:, None, None]
    raw = np.zeros((w.cap_tokens, H, d), np.float16)
    raw[4 * nb0:n_before] = synth.normal_f16(70, (n_before - 4 * nb0, H, d))
    K = synth.normal_f16(71, (w.cap_tokens, 4, 128))
    V = synth.normal_f16(72, (w.cap_tokens, 4, 128))
    K[n_before:] = 0
    V[n_before:] = 0
    half = np.ones((H, d), np.float16)
    half[:, d // 2:] = 0
    q_idx = np.stack([np.ones((H, d)), -np.ones((H, d)), half]).astype(np.float16)
    mult = [2048.0, -2048.0, 1024.0]  # complete blocks score exactly mult * v
    q = synth.normal_f16(73, (n_q, 32, 128))
    k_idx_new = synth.normal_f16(74, (n_q, H, d))
    k_new = synth.normal_f16(75, (n_q, 4, 128))
    v_new = synth.normal_f16(76, (n_q, 4, 128))

    g = qb.Layer(cfg)
    g.k_pool.copy_(dev(pooled))
    g.k_raw.copy_(dev(raw))
    g.k_cache.copy_(dev(K))
    g.v_cache.copy_(dev(V))
    ld = nb0 + 8
    out = torch.empty((n_q, 32, 128), device="cuda")
    scores = torch.full((n_q, ld), 321.0, device="cuda")
    blk = torch.full((n_q, 512), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, w.cap_tokens)
    qb.qsa_decode_multi(cfg, g, n_before, dev(q_idx), dev(k_idx_new), dev(q), dev(k_new),
                        dev(v_new), out, ws, scores_out=scores, ld_scores=ld, blk_out=blk)
    s_all, b_all, o_all = host(scores), host(blk), host(out)
    for row in range(n_q):
        ref = O.decode_step(shape_of(w), raw, pooled, K, V, n_before + row, q_idx[row],
                            k_idx_new[row], q[row], k_new[row], v_new[row])
        nb = (n_before + row + 1) // 4
        s_gpu = s_all[row][:nb]
        assert np.array_equal(s_gpu[:nb0], mult[row] * v.astype(np.float32)), row
        if nb > nb0:
            assert abs(s_gpu[nb0] - ref["scores64"][nb0]) <= \
                SCORE_REL * np.max(np.abs(ref["scores64"]))
        b_gpu = b_all[row][:min(512, nb)]
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, 512)), row
        assert np.array_equal(b_gpu, ref["blk"]), row
        ref_out = O.attn_cells(q[row], K, V, O.cells(b_gpu, n_before + row + 1), w.scale)
        assert_attn_close(o_all[row], ref_out, f"row {row}")


# ------------------------------------------------------------------ f3 multi-query decode
@pytest.mark.parametrize("n_tokens,n_q", [(4 * 3000 + 1, 3), (4 * 3000 + 3, 3), (4 * 3000, 2),
                                          (4 * 3000 + 2, 4), (2049, 3), (6, 4)])
def test_decode_multi_equals_sequential_steps(gpu, n_tokens, n_q):
    # n_q rows appended and attended in one call; row r against the oracle's decode
    # step at position n_before + r (n_q oracle steps in order on the same caches)
    w = small(n_tokens)
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    r = np.random.default_rng(n_tokens * 10 + n_q)
    q_idx = synth.normal_f16(80, (n_q, 16, 128))
    q = synth.normal_f16(81, (n_q, 32, 128))
    k_idx_new = synth.normal_f16(82, (n_q, 16, 128))
    k_new = synth.normal_f16(83, (n_q, 4, 128))
    v_new = synth.normal_f16(84, (n_q, 4, 128))
    nb_last = (n0 + n_q) // 4
    ld = nb_last + 5
    out = torch.empty((n_q, 32, 128), device="cuda")
    scores = torch.full((n_q, ld), 123.0, device="cuda")
    blk = torch.full((n_q, w.topk), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, w.cap_tokens)
    qb.qsa_decode_multi(cfg, g, n0, dev(q_idx), dev(k_idx_new), dev(q), dev(k_new), dev(v_new),
                        out, ws, scores_out=scores, ld_scores=ld, blk_out=blk)
    s_all, b_all, o_all = host(scores), host(blk), host(out)
    for row in range(n_q):
        ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, n0 + row, q_idx[row],
                            k_idx_new[row], q[row], k_new[row], v_new[row])
        nb = (n0 + row + 1) // 4
        s_gpu = s_all[row][:nb]
        if nb:
            assert np.max(np.abs(s_gpu - ref["scores64"])) <= \
                SCORE_REL * np.max(np.abs(ref["scores64"]))
        nsel = min(w.topk, nb)
        b_gpu = b_all[row][:nsel]
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, w.topk))
        ref_out = O.attn_cells(q[row], o.k, o.v, O.cells(b_gpu, n0 + row + 1), w.scale)
        assert_attn_close(o_all[row], ref_out)
    # the caches hold all n_q new tokens, pooled rows included
    nb = (n0 + n_q) // 4
    assert_pool_close(host(g.k_pool[:nb]), o.pooled[:nb])
    assert np.array_equal(host(g.k_raw[n0:n0 + n_q]).view(np.uint16), k_idx_new.view(np.uint16))


@pytest.mark.parametrize("seed", range(12))
def test_decode_multi_random_configs(gpu, seed):
    # 2-4 verification rows of a drawn configuration (as for the single step), each
    # row against the oracle's decode step at its position, in order
    w, _ = random_decode_config(100 + seed)
    n_q = 2 + seed % 3
    print(f"config {w} rows {n_q}", flush=True)
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    q_idx = synth.normal_f16(90 + seed, (n_q, w.h_idx, w.d_idx))
    q = synth.normal_f16(120 + seed, (n_q, w.hq, w.d))
    k_idx_new = synth.normal_f16(150 + seed, (n_q, w.h_idx, w.d_idx))
    k_new = synth.normal_f16(180 + seed, (n_q, w.hkv, w.d))
    v_new = synth.normal_f16(210 + seed, (n_q, w.hkv, w.dv))
    ld = (n0 + n_q) // 4 + 3
    out = torch.empty((n_q, w.hq, w.dv), device="cuda")
    scores = torch.full((n_q, ld), 123.0, device="cuda")
    blk = torch.full((n_q, w.topk), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, w.cap_tokens)
    qb.qsa_decode_multi(cfg, g, n0, dev(q_idx), dev(k_idx_new), dev(q), dev(k_new), dev(v_new),
                        out, ws, scores_out=scores, ld_scores=ld, blk_out=blk)
    s_all, b_all, o_all = host(scores), host(blk), host(out)
    for row in range(n_q):
        ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, n0 + row, q_idx[row],
                            k_idx_new[row], q[row], k_new[row], v_new[row])
        nb = (n0 + row + 1) // 4
        s_gpu = s_all[row][:nb]
        if nb:
            assert np.max(np.abs(s_gpu - ref["scores64"])) <= \
                SCORE_REL * np.max(np.abs(ref["scores64"])), row
        b_gpu = b_all[row][:min(w.topk, nb)]
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, w.topk)), row
        ref_out = O.attn_cells(q[row], o.k, o.v, O.cells(b_gpu, n0 + row + 1), w.scale)
        assert_attn_close(o_all[row], ref_out, f"row {row}")
    nb = (n0 + n_q) // 4
    assert_pool_close(host(g.k_pool[:nb]), o.pooled[:nb])


def test_decode_multi_255181_planted(gpu):
    # the 256k workload with three rows: every row finds the planted blocks
    w = synth.WORKLOADS["decode_255181"]
    L, cfg, g, o = setup_decode(w)
    n0 = L["n_prefix"]
    n_q = 3
    q_idx = np.stack([L["q_idx"]] * n_q)
    q = np.stack([L["q"]] * n_q)
    out = torch.empty((n_q, 32, 128), device="cuda")
    blk = torch.full((n_q, w.topk), -1, dtype=torch.int32, device="cuda")
    ld = (n0 + n_q) // 4 + 1
    scores = torch.empty((n_q, ld), device="cuda")
    ws = qb.workspace(cfg, n_q, w.cap_tokens)
    qb.qsa_decode_multi(cfg, g, n0, dev(q_idx), dev(L["k_idx_new"][:n_q]), dev(q),
                        dev(L["k_new"][:n_q]), dev(L["v_new"][:n_q]), out, ws, scores_out=scores,
                        ld_scores=ld, blk_out=blk)
    for row in range(n_q):
        ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, n0 + row, q_idx[row],
                            L["k_idx_new"][row], q[row], L["k_new"][row], L["v_new"][row])
        nb = (n0 + row + 1) // 4
        s_gpu = host(scores[row])[:nb]
        b_gpu = host(blk[row])
        assert np.array_equal(b_gpu, O.topk_sort(s_gpu, w.topk))
        assert set(L["planted"].tolist()) <= set(b_gpu.tolist())
        ref_out = O.attn_cells(q[row], o.k, o.v, O.cells(b_gpu, n0 + row + 1), w.scale)
        assert_attn_close(host(out[row]), ref_out)


def test_decode_step_at_maximum_capacity(gpu):
    # the largest context the library takes (cap_tokens <= 2^21): 524,270 complete
    # blocks and a tail of 3; sampled pooled rows, every score, the top-k and the
    # output against the oracle
    n_tokens = 4 * 524270 + 3
    w = small(n_tokens)
    assert w.cap_tokens <= 1 << 21
    cfg = cfg_of(w)
    n0 = n_tokens - 1
    raw = synth.normal_f16(90, (n0, 16, 128))
    K = synth.normal_f16(91, (n_tokens, 4, 128))
    V = synth.normal_f16(92, (n_tokens, 4, 128))
    q_idx = synth.normal_f16(93, (16, 128))
    q = synth.normal_f16(94, (32, 128))
    k_idx_new = synth.normal_f16(95, (16, 128))
    g = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(raw), 0, g.k_raw, g.k_pool)
    g.k_cache[:n0] = dev(K[:n0])
    g.v_cache[:n0] = dev(V[:n0])
    nb = n_tokens // 4
    out = torch.empty((32, 128), device="cuda")
    scores = torch.empty(nb, device="cuda")
    blk = torch.full((512,), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, 1, w.cap_tokens)
    qb.qsa_decode_step(cfg, g, n0, dev(q_idx), dev(k_idx_new), dev(q), dev(K[n0]), dev(V[n0]),
                       out, ws, scores_out=scores, blk_out=blk)
    # pooled rows: the last blocks and a seeded sample, against the oracle's pooling
    rows = np.unique(np.concatenate([np.arange(nb - 4, nb),
                                     np.random.default_rng(9).choice(nb, 300, replace=False)]))
    got = host(g.k_pool[torch.from_numpy(rows).cuda()])
    ref = np.stack([O.pool_block(raw[4 * b:4 * b + 4], O.block_pos(b)) for b in rows])
    assert_pool_close(got, ref)
    # scores against the oracle's scan of the GPU's own pooled rows
    P = host(g.k_pool[:nb])
    s64, _ = O.index_score(q_idx, P, nb)
    bound = SCORE_ABS_REL * (np.abs(P.astype(np.float64).reshape(nb, -1)) @
                             np.abs(q_idx.astype(np.float64).ravel()))
    s_gpu = host(scores)
    assert np.all(np.abs(s_gpu - s64) <= bound)
    b_gpu = host(blk)
    assert np.array_equal(b_gpu, O.topk_sort(s_gpu, 512))
    ref_out = O.attn_cells(q, K, V, O.cells(b_gpu, n_tokens), w.scale)
    assert_attn_close(host(out), ref_out)
