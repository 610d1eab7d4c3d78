"""GPU parity of the prefill-chunk path (MFMA scoring, per-row top-k, per-row
attention, the fused prefill step) against the CPU oracle, through the C ABI."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_qsa_amd import binding as qb
import synth
from _helpers import (SCORE_ABS_REL, SCORE_REL, OracleLayer, assert_attn_close, cfg_of, dev, host,
                      shape_of)

pytestmark = pytest.mark.gpu


def sample_rows(n_q, seed, n=64):
    """The first row, the last row and n - 2 other distinct rows drawn from seed."""
    r = np.random.default_rng(seed)
    rest = r.choice(np.arange(1, n_q - 1), size=min(n - 2, max(n_q - 2, 0)), replace=False)
    return sorted({0, n_q - 1, *rest.tolist()})


def each_row(rows, fn):
    """fn(row) for every row on a thread pool (the oracle's C calls release the
    interpreter lock); the first failing row's assertion is raised."""
    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        for f in [ex.submit(fn, r) for r in rows]:
            f.result()


def abs_rows(P):
    """|P| as [rows, features] fp32, computed once per test for score_bound."""
    return np.abs(P.reshape(P.shape[0], -1).astype(np.float32))


def score_bound(q_row, absP, nb):
    """SCORE_ABS_REL * sum_i |q_i P_bi| for b < nb (fp32 is ample for a bound)."""
    return SCORE_ABS_REL * (absP[:nb] @ np.abs(q_row.astype(np.float32).ravel())).astype(
        np.float64)


def run_prefill_scores(H, d, n_q, pos0, seed, rows_to_check):
    cap = pos0 + n_q + 64
    cap -= cap % 4
    cfg = qb.Config(h_idx=H, d_idx=d, cap_tokens=cap)
    nb_max = (pos0 + n_q) // 4
    P = synth.normal_f16(seed, (nb_max, H, d))
    Q = synth.normal_f16(seed + 1, (n_q, H, d))
    pool = torch.zeros((cap // 4, H, d), dtype=torch.float16, device="cuda")
    pool[:nb_max] = dev(P)
    ld = ((nb_max + 63) // 64) * 64
    S = torch.full((n_q, ld), 777.0, device="cuda")
    qb.qsa_index_score(cfg, dev(Q), pos0, pool, S, ld=ld)
    got = host(S)
    absP = abs_rows(P)

    def check(r):
        nb = (pos0 + r + 1) // 4
        s64, _ = O.index_score(Q[r], P, nb)
        assert np.all(np.abs(got[r, :nb] - s64) <= score_bound(Q[r], absP, nb)), r

    each_row(rows_to_check, check)
    assert np.all(got[:, nb_max:] == 777.0)


@pytest.mark.parametrize("H,d,n_q,pos0", [(16, 128, 300, 1000), (16, 128, 257, 3), (4, 64, 100, 999),
                                          (8, 128, 1, 5000), (16, 128, 1024, 7),
                                          # 128 features (two 64-feature steps), 1,024, 4,096
                                          (2, 64, 70, 500), (1, 128, 130, 300), (8, 128, 2, 5000),
                                          (32, 128, 64, 2000)])
def test_index_score_prefill_mfma(gpu, H, d, n_q, pos0):
    if n_q == 1:
        pytest.skip("n_q == 1 is the decode kernel")
    run_prefill_scores(H, d, n_q, pos0, 50, range(n_q))


def test_index_score_prefill_mfma_full_size(gpu):
    w = synth.WORKLOADS["prefill_1024_at_126253"]
    run_prefill_scores(w.h_idx, w.d_idx, w.n_q, w.n_tokens, 60, sample_rows(w.n_q, 4))


def crafted_row(nb, kind, r):
    if kind == "normal":
        return r.standard_normal(nb).astype(np.float32) * 45
    if kind == "few_values":
        return r.integers(-2, 3, nb).astype(np.float32)
    if kind == "narrow":
        return (1.0 + r.random(nb).astype(np.float32) * 1e-3).astype(np.float32)
    if kind == "all_equal":
        return np.full(nb, -2.5, np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "few_values", "narrow", "all_equal"])
def test_topk_rows_bit_exact(gpu, kind):
    # rows see growing causal prefixes; first rows have nb <= k
    n_q, pos0, k = 64, 2030, 512
    cfg = qb.Config(topk_blocks=k, cap_tokens=4096)
    nb_max = (pos0 + n_q) // 4
    ld = nb_max + 3
    r = np.random.default_rng(len(kind))
    S = np.stack([np.concatenate([crafted_row(nb_max, kind, r), np.zeros(3, np.float32)])
                  for _ in range(n_q)])
    blk = torch.full((n_q, k), -5, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, pos0 + n_q)
    qb.qsa_topk_blocks(cfg, dev(S), n_q, ld, pos0, blk, nsel, ws)
    b, ns = host(blk), host(nsel)
    for i in range(n_q):
        nb = (pos0 + i + 1) // 4
        assert ns[i] == min(k, nb)
        assert np.array_equal(b[i, :ns[i]], O.topk_sort(S[i, :nb], k)), i


@pytest.mark.parametrize("n_q,pos0", [(24, 127253), (8, 200000), (4, 262140), (6, 262150),
                                     (5, 300001)])
def test_topk_rows_large_rows(gpu, n_q, pos0):
    # rows of the 128k prefill size (~31.8k blocks each), of 50,000 blocks and up to
    # exactly 65,536 (the register-resident form's largest rows, 64 keys a thread),
    # and rows past that limit
    k = 512
    cfg = qb.Config(topk_blocks=k, cap_tokens=(pos0 + n_q + 64) // 4 * 4)
    nb_max = (pos0 + n_q) // 4
    r = np.random.default_rng(9)
    S = (r.standard_normal((n_q, nb_max)) * 45).astype(np.float32)
    S[3] = np.round(S[3])           # many ties
    S[min(5, n_q - 1)] = 7.0         # all equal
    blk = torch.full((n_q, k), -5, dtype=torch.int32, device="cuda")
    nsel = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, pos0 + n_q)
    qb.qsa_topk_blocks(cfg, dev(S), n_q, nb_max, pos0, blk, nsel, ws)
    b = host(blk)
    for i in range(n_q):
        nb = (pos0 + i + 1) // 4
        assert np.array_equal(b[i], O.topk_sort(S[i, :nb], k)), i


def prefill_case(w, layer=0, flags=qb.QSA_PREFILL_PER_ROW):
    I = synth.prefill_inputs(w, layer)
    depth, n_q = I["depth"], w.n_q
    cfg = cfg_of(w)
    g = qb.Layer(cfg)
    qb.qsa_pool_append(cfg, dev(I["raw"][:depth]), 0, g.k_raw, g.k_pool)
    g.k_cache[:depth] = dev(I["k"][:depth])
    g.v_cache[:depth] = dev(I["v"][:depth])
    out = torch.empty((n_q, w.hq, w.dv), device="cuda")
    nb_end = (depth + n_q) // 4
    ld = ((nb_end + 1 + 63) // 64) * 64
    scores = torch.empty((n_q, ld), device="cuda")
    blk = torch.full((n_q, w.topk), -1, dtype=torch.int32, device="cuda")
    ws = qb.workspace(cfg, n_q, depth + n_q)
    qb.qsa_prefill_step(cfg, g, depth, dev(I["q_idx"]), dev(I["raw"][depth:]), dev(I["q"]),
                        dev(I["k"][depth:]), dev(I["v"][depth:]), out, ws, scores_out=scores,
                        ld_scores=ld, blk_out=blk, flags=flags)
    return I, cfg, g, host(out), host(scores), host(blk)


def check_prefill_rows(w, I, g, out, scores, blk, rows, oracle_pooled=None):
    depth = I["depth"]
    n_all = depth + w.n_q
    pooled_gpu = host(g.k_pool[:n_all // 4])
    absP = abs_rows(pooled_gpu)

    def check(r):
        pos = depth + r
        nb = (pos + 1) // 4
        nsel = min(w.topk, nb)
        s_gpu = scores[r, :nb]
        # scores against the oracle on the GPU's pooled rows (tight)
        s64, _ = O.index_score(I["q_idx"][r], pooled_gpu, nb)
        assert np.all(np.abs(s_gpu - s64) <= score_bound(I["q_idx"][r], absP, nb)), r
        if oracle_pooled is not None:
            s_or, _ = O.index_score(I["q_idx"][r], oracle_pooled, nb)
            assert np.max(np.abs(s_gpu - s_or)) <= SCORE_REL * np.max(np.abs(s_or)), r
        b = blk[r, :nsel]
        assert np.array_equal(b, O.topk_sort(s_gpu, w.topk)), r
        cells = O.cells(b, pos + 1)
        ref = O.attn_cells(I["q"][r], I["k"], I["v"], cells, w.scale)
        assert_attn_close(out[r], ref, f"row {r}")

    each_row(rows, check)


def test_prefill_step_small(gpu):
    w = synth.Workload("prefill_small", 6, "prefill", 4 * 700 + 1, n_q=300)
    I, cfg, g, out, scores, blk = prefill_case(w)
    depth = I["depth"]
    n_all = depth + w.n_q
    oracle_pooled = O.pool_rebuild(I["raw"], n_all)
    check_prefill_rows(w, I, g, out, scores, blk, range(w.n_q), oracle_pooled)
    # the chunk's raw/K/V rows landed in the caches
    assert np.array_equal(host(g.k_raw[depth:n_all]).view(np.uint16),
                          I["raw"][depth:].view(np.uint16))
    assert np.array_equal(host(g.v_cache[depth:n_all]).view(np.uint16),
                          I["v"][depth:].view(np.uint16))


def random_prefill_config(seed):
    """A seeded draw over the configurations a prefill chunk supports: indexer rows
    of 16..512 sixteen-byte pieces, 1..16 query heads per KV head, head dims 64 or
    128, k from 1 to 1,024, depths up to 12,000 tokens, chunks of 2..400 rows, and the
    per-row, grouped-union and union-for-every-group forms."""
    rng = np.random.default_rng(7000 + seed)
    d_idx = int(rng.choice([16, 32, 64, 128, 256]))
    rowc = int(rng.choice([r for r in (16, 32, 64, 128, 256, 512) if r * 8 >= d_idx]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h * G <= 64]))
    d = int(rng.choice([64, 128]))
    topk = int(rng.choice([1, 3, 64, 200, 512, 1024]))
    depth = int(rng.integers(1, 12000))
    n_q = int(rng.integers(2, 400))
    flags = (qb.QSA_PREFILL_PER_ROW, UNION, UNION_ALL)[seed % 3]
    w = synth.Workload(f"random_prefill_{seed}", 600 + seed, "prefill", depth,
                       h_idx=rowc * 8 // d_idx, d_idx=d_idx, topk=topk, hq=hkv * G, hkv=hkv,
                       d=d, dv=d, n_q=n_q, q_corr=float(rng.choice([0.0, 0.9])))
    return w, flags


@pytest.mark.parametrize("seed", range(18))
def test_prefill_step_random_configs(gpu, seed):
    # a drawn configuration: 24 sampled rows (first, last and 22 seeded) against the
    # oracle, on the GPU's own pooled rows and the oracle's
    w, flags = random_prefill_config(seed)
    print(f"config {w} flags {flags}", flush=True)
    G = w.hq // w.hkv
    if flags != qb.QSA_PREFILL_PER_ROW and not (G in (4, 8, 16) and w.d == 128
                                                 and (128 // G) * w.topk <= 16384):
        # outside the grouped-union form's shapes the call refuses (status UNSUPPORTED)
        with pytest.raises(qb.QsaError, match="grouped union"):
            prefill_case(w, flags=flags)
        flags = qb.QSA_PREFILL_PER_ROW
    I, cfg, g, out, scores, blk = prefill_case(w, flags=flags)
    oracle_pooled = O.pool_rebuild(I["raw"], I["depth"] + w.n_q)
    check_prefill_rows(w, I, g, out, scores, blk, sample_rows(w.n_q, seed, 24), oracle_pooled)


def test_prefill_step_is_decode_per_row(gpu):
    # a chunk row equals a decode step at that length (small chunk, every row)
    w = synth.Workload("prefill_vs_decode", 6, "prefill", 4 * 600 + 2, n_q=9, topk=64)
    I, cfg, g, out, scores, blk = prefill_case(w)
    depth = I["depth"]
    for r in range(w.n_q):
        o = OracleLayer(w, w.cap_tokens)
        O.pool_append(I["raw"][:depth + r], 0, o.raw, o.pooled)
        o.k[:depth + r], o.v[:depth + r] = I["k"][:depth + r], I["v"][:depth + r]
        ref = O.decode_step(shape_of(w), o.raw, o.pooled, o.k, o.v, depth + r, I["q_idx"][r],
                            I["raw"][depth + r], I["q"][r], I["k"][depth + r], I["v"][depth + r])
        nb = (depth + r + 1) // 4
        diff = set(blk[r, :min(w.topk, nb)].tolist()) ^ set(ref["blk"].tolist())
        kth = np.sort(ref["scores64"])[::-1][w.topk - 1]
        for b in diff:
            assert abs(ref["scores64"][b] - kth) <= SCORE_REL * np.max(np.abs(ref["scores64"]))
        if not diff:
            assert_attn_close(out[r], ref["out"], f"row {r}")


def test_prefill_step_full_size_sampled(gpu):
    # 64 rows (first, last, 62 seeded); scores also against the oracle's own pooling
    w = synth.WORKLOADS["prefill_1024_at_126253"]
    I, cfg, g, out, scores, blk = prefill_case(w)
    oracle_pooled = O.pool_rebuild(I["raw"], I["depth"] + w.n_q)
    check_prefill_rows(w, I, g, out, scores, blk, sample_rows(w.n_q, 8), oracle_pooled)


# ---------------------------------------------------------------- grouped-union form
UNION = qb.QSA_PREFILL_GROUPED_UNION
UNION_ALL = qb.QSA_PREFILL_GROUPED_UNION | qb.QSA_PREFILL_UNION_ALL  # no per-row groups


@pytest.mark.parametrize("q_corr", [0.0, 0.99])
def test_prefill_step_union_small(gpu, q_corr):
    # every row of a 300-row chunk (18 groups of 16 rows and a ragged group of 12)
    w = synth.Workload("prefill_small", 6, "prefill", 4 * 700 + 1, n_q=300, q_corr=q_corr)
    I, cfg, g, out, scores, blk = prefill_case(w, flags=UNION)
    check_prefill_rows(w, I, g, out, scores, blk, range(w.n_q))


def union_direct(hq, hkv, k, pos0, n_q, seed, shared=0.5, ldb_pad=0, flags=None, d=128):
    """qsa_prefill_attn on chosen-block lists drawn here (a share of the blocks common
    to each run of 8 rows; `shared` may also be a function of the row), against the
    oracle for every row: with `flags`, else the grouped-union form both with its
    per-group choice and with the union for every group."""
    dv = d
    share = shared if callable(shared) else (lambda i: shared)
    n_all = pos0 + n_q
    cap = (n_all + 64) // 4 * 4
    cfg = qb.Config(topk_blocks=k, hq=hq, hkv=hkv, d=d, dv=dv, cap_tokens=cap)
    K = synth.normal_f16(seed, (n_all, hkv, d))
    V = synth.normal_f16(seed + 1, (n_all, hkv, dv))
    Q = synth.normal_f16(seed + 2, (n_q, hq, d))
    r = np.random.default_rng(seed)
    ldb = k + ldb_pad
    B = np.full((n_q, ldb), -7, np.int32)  # past n_sel: never read
    common = None
    for i in range(n_q):
        nb = (pos0 + i + 1) // 4
        ns = min(k, nb)
        if ns == nb:
            ids = np.arange(nb)
        else:
            if common is None or i % 8 == 0:
                common = r.choice(nb, size=int(ns * share(i)), replace=False)
            rest = np.setdiff1d(np.arange(nb), common)
            ids = np.concatenate([common, r.choice(rest, size=ns - common.size, replace=False)])
        B[i, :ns] = np.sort(ids)
    kc = torch.zeros((cap, hkv, d), dtype=torch.float16, device="cuda")
    vc = torch.zeros((cap, hkv, dv), dtype=torch.float16, device="cuda")
    kc[:n_all], vc[:n_all] = dev(K), dev(V)
    ws = qb.workspace(cfg, n_q, n_all)
    scale = 1.0 / np.sqrt(d)
    refs = []
    for i in range(n_q):
        nb = (pos0 + i + 1) // 4
        refs.append(O.attn_cells(Q[i], K, V, O.cells(B[i, :min(k, nb)], pos0 + i + 1), scale))
    for f in ([UNION, UNION_ALL] if flags is None else [flags]):
        out = torch.full((n_q, hq, dv), 5.0, device="cuda")
        qb.qsa_prefill_attn(cfg, dev(Q), pos0, dev(B), ldb, kc, vc, out, ws, flags=f)
        got = host(out)
        for i in range(n_q):
            assert_attn_close(got[i], refs[i], f"flags {f} row {i}")
    return B


@pytest.mark.parametrize("hq,hkv,k,pos0,n_q", [
    (32, 4, 64, 3, 70),      # first rows see every block (nb <= k), empty and full tails
    (32, 4, 64, 257, 33),    # two full groups and a 1-row group
    (16, 4, 64, 1001, 45),   # 4 query heads per KV head: groups of 32 rows
    (32, 2, 64, 2002, 20),   # 16 query heads per KV head: groups of 8 rows
    (8, 1, 512, 9000, 17),   # k = 512, one KV head
    (32, 4, 512, 5000, 1),   # a single row
])
def test_prefill_attn_union_shapes(gpu, hq, hkv, k, pos0, n_q):
    union_direct(hq, hkv, k, pos0, n_q, 70 + n_q, ldb_pad=3)


@pytest.mark.parametrize("hq,hkv,k,pos0,n_q,d", [
    (32, 4, 64, 3, 70, 128),      # first rows see every block (nb <= k), empty and full tails
    (32, 4, 64, 257, 33, 128),    # 8 query heads per KV head
    (16, 4, 64, 1001, 45, 128),   # 4 query heads per KV head
    (32, 2, 64, 2002, 20, 128),   # 16 query heads per KV head
    (8, 1, 512, 9000, 17, 128),   # k = 512, one KV head
    (32, 4, 1024, 5000, 5, 128),  # k = 1024: 4,099 cells, a ragged last tile
    (32, 4, 512, 5000, 1, 128),   # a single row
    (32, 4, 64, 1001, 9, 64),     # d = 64: the vector-unit per-row kernel
    (8, 4, 64, 1001, 9, 128),     # 2 query heads per KV head: the vector-unit kernel
])
def test_prefill_attn_per_row_shapes(gpu, hq, hkv, k, pos0, n_q, d):
    union_direct(hq, hkv, k, pos0, n_q, 170 + n_q, shared=0.0, ldb_pad=5,
                 flags=qb.QSA_PREFILL_PER_ROW, d=d)


def test_prefill_attn_union_past_one_bitmap_window(gpu):
    # block ids on both sides of 2^18 (the union build's bitmap window)
    union_direct(8, 1, 512, 4 * ((1 << 18) + (1 << 16)) + 1001, 18, 90, shared=0.25)


def test_prefill_attn_broken_ids_are_dropped(gpu):
    # ids outside a row's [0, nb_r) (only a broken selection has them) are dropped by
    # both forms, so no row reaches past its own prefix: both equal the oracle on
    # the valid ids
    hq, hkv, k, pos0, n_q, d = 32, 4, 64, 4001, 20, 128
    n_all = pos0 + n_q
    cap = (n_all + 64) // 4 * 4
    cfg = qb.Config(topk_blocks=k, hq=hq, hkv=hkv, d=d, dv=d, cap_tokens=cap)
    K = synth.normal_f16(95, (n_all, hkv, d))
    V = synth.normal_f16(96, (n_all, hkv, d))
    Q = synth.normal_f16(97, (n_q, hq, d))
    r = np.random.default_rng(95)
    B = np.zeros((n_q, k), np.int32)
    valid = []
    for i in range(n_q):
        nb = (pos0 + i + 1) // 4
        ids = np.sort(r.choice(nb, size=k, replace=False)).astype(np.int32)
        ids[-1] = nb + 2 if i % 2 == 0 else -3   # past the prefix / negative
        ids[-2] = nb                              # the first block the row cannot see
        B[i] = ids
        valid.append(ids[(ids >= 0) & (ids < nb)])
    kc = torch.zeros((cap, hkv, d), dtype=torch.float16, device="cuda")
    vc = torch.zeros((cap, hkv, d), dtype=torch.float16, device="cuda")
    kc[:n_all], vc[:n_all] = dev(K), dev(V)
    ws = qb.workspace(cfg, n_q, n_all)
    scale = 1.0 / np.sqrt(d)
    for flags in (qb.QSA_PREFILL_PER_ROW, UNION):
        out = torch.full((n_q, hq, d), 5.0, device="cuda")
        qb.qsa_prefill_attn(cfg, dev(Q), pos0, dev(B), k, kc, vc, out, ws, flags=flags)
        got = host(out)
        for i in range(n_q):
            ref = O.attn_cells(Q[i], K, V, O.cells(np.sort(valid[i]), pos0 + i + 1), scale)
            assert_attn_close(got[i], ref, f"flags {flags} row {i}")


def test_prefill_attn_union_no_overlap(gpu):
    # rows with disjoint choices: the union holds rows x k blocks (per row, unless
    # every group is made to take the union)
    union_direct(32, 4, 64, 40000, 16, 91, shared=0.0)


def test_prefill_attn_union_mixed_groups(gpu):
    # 6 groups of 16 rows, sharing 90% of their blocks in even groups (unions of
    # about 3.4 k: the union kernel) and nothing in odd ones (16 k: per row), so one
    # call runs both kernels, each on its own groups; a ragged last group
    union_direct(32, 4, 128, 30000, 90, 92, shared=lambda i: 0.9 if (i // 16) % 2 == 0 else 0.0)


@pytest.mark.parametrize("name", ["prefill_1024_at_126253", "prefill_1024_at_126253_corr"])
def test_prefill_step_union_full_size_sampled(gpu, name):
    w = synth.WORKLOADS[name]
    I, cfg, g, out, scores, blk = prefill_case(w, flags=UNION)
    # 64 rows against the oracle: first, last, 62 seeded (group edges 15 / 16 included)
    rows = sorted({15, 16, *sample_rows(w.n_q, 18)})
    check_prefill_rows(w, I, g, out, scores, blk, rows)
    # every row against the per-row form on the same chosen blocks
    ref = torch.empty_like(dev(out))
    qb.qsa_prefill_attn(cfg, dev(I["q"]), I["depth"], dev(blk), w.topk, g.k_cache, g.v_cache, ref,
                        None)
    ref = host(ref)
    err = np.max(np.abs(out - ref), axis=(1, 2))
    assert np.all(err <= 2e-3 * np.max(np.abs(ref), axis=(1, 2))), int(np.argmax(err))
    # and the union for every group, on the same chosen blocks
    alls = torch.empty_like(dev(out))
    ws = qb.workspace(cfg, w.n_q, I["depth"] + w.n_q)
    qb.qsa_prefill_attn(cfg, dev(I["q"]), I["depth"], dev(blk), w.topk, g.k_cache, g.v_cache,
                        alls, ws, flags=UNION_ALL)
    err = np.max(np.abs(host(alls) - ref), axis=(1, 2))
    assert np.all(err <= 2e-3 * np.max(np.abs(ref), axis=(1, 2))), int(np.argmax(err))
