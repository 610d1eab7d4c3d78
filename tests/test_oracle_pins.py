"""Pins for the CPU oracle: closed forms, invariants, brute force and library routines.

None of these re-types the oracle's own formula: each one checks the oracle against
something that fixes the answer independently (numpy/scipy routines, algebraic
invariants, brute force on tiny inputs, the numbers the pages print).
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16)


def rnd(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float16)


# ------------------------------------------------------------------ binary16 codec
def test_f16_decode_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.h2d(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_f16_encode_matches_numpy_rne():
    r = np.random.default_rng(1)
    mags = 2.0 ** r.uniform(-30, 17, 200000)
    x = mags * r.choice([-1.0, 1.0], mags.size)
    # exact midpoints between neighbouring binary16 values (ties-to-even cases)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = (lo + hi) / 2
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                     2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0,
                     np.inf, -np.inf])
    x = np.concatenate([x, mids, -mids, edge])
    ours = O.d2h(x).view(np.uint16)
    with np.errstate(over="ignore"):  # the overflow edges are the point
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.isnan(O.d2h(np.array([np.nan])).astype(np.float64)[0])


# ------------------------------------------------------------------ pooled summary
def _unit_rms(v):
    return np.sqrt(np.mean(np.asarray(v, np.float64) ** 2, axis=-1))


def test_pool_equal_keys_at_position_zero_is_normalised_key():
    # 4 equal keys: the mean is the key; position 0: RoPE is the identity.
    x = rnd(2, (3, 64))
    out = O.pool_block(np.stack([x] * 4), 0)
    xd = x.astype(np.float64)
    for h in range(3):
        o = out[h].astype(np.float64)
        cos = o @ xd[h] / np.linalg.norm(o) / np.linalg.norm(xd[h])
        assert cos > 1 - 1e-6
    assert np.allclose(_unit_rms(out), 1.0, atol=2e-3)


def test_pool_uses_every_token_equally():
    # The pooled summary depends on the 4 keys only through their mean: each of
    # the four single-token placements gives the same row, and so does a
    # permutation; a dropped or double-counted token breaks this.
    x = rnd(3, (2, 32))
    z = np.zeros_like(x)
    rows = []
    for t in range(4):
        keys = [z] * 4
        keys[t] = x
        rows.append(O.pool_block(np.stack(keys), 12))
    for r in rows[1:]:
        assert np.array_equal(r, rows[0])
    a, b, c, d = (rnd(10 + i, (2, 32)) for i in range(4))
    p1 = O.pool_block(np.stack([a, b, c, d]), 8)
    p2 = O.pool_block(np.stack([d, c, b, a]), 8)
    # the mean direction: position 0 pooled row is parallel to a+b+c+d
    p0 = O.pool_block(np.stack([a, b, c, d]), 0).astype(np.float64)
    s = a.astype(np.float64) + b + c + d
    for h in range(2):
        assert p0[h] @ s[h] / np.linalg.norm(p0[h]) / np.linalg.norm(s[h]) > 1 - 1e-6
    assert np.max(np.abs(p1.astype(np.float64) - p2.astype(np.float64))) <= 2e-3


def test_rms_norm_gives_unit_rms_per_head_at_any_position():
    raw = rnd(4, (4 * 50, 4, 64))
    pooled = O.pool_rebuild(raw, raw.shape[0])
    assert np.allclose(_unit_rms(pooled), 1.0, atol=3e-3)


def test_rms_weight_scales_each_dimension():
    x = rnd(5, (4, 2, 64))
    base = O.pool_block(x, 0).astype(np.float64)
    w = np.linspace(0.5, 2.0, 64).astype(np.float32)
    wt = O.pool_block(x, 0, w=w).astype(np.float64)
    assert np.allclose(wt, base * w, rtol=2e-3, atol=2e-3)
    twice = O.pool_block(x, 40, w=np.full(64, 2.0, np.float32)).astype(np.float64)
    assert np.array_equal(twice, 2 * O.pool_block(x, 40).astype(np.float64))


def test_eps_inside_the_root():
    # a zero block stays zero; a tiny block is damped by eps (rms < 1)
    z = np.zeros((4, 1, 64), np.float16)
    assert not np.any(O.pool_block(z, 4).astype(np.float64))
    tiny = np.full((4, 1, 64), 1e-4, np.float16)
    out = O.pool_block(tiny, 0, eps=1e-6).astype(np.float64)
    ms = float(np.float16(1e-4)) ** 2
    assert np.allclose(out, np.float16(1e-4) / np.sqrt(ms + 1e-6), rtol=2e-3)


@pytest.mark.parametrize("b", [1, 7, 1000, 63795])
def test_rope_is_the_complex_rotation(b):
    # half-split RoPE = multiplying z = x[:d/2] + i x[d/2:] by exp(i * p * base^(-2j/d))
    x = rnd(6, (4, 3, 128))
    p = O.block_pos(b)
    assert p == 4 * b
    n0 = O.pool_block(x, 0).astype(np.float64)  # position 0: normalised mean, no rotation
    got = O.pool_block(x, p).astype(np.float64)
    j = np.arange(64)
    z = (n0[:, :64] + 1j * n0[:, 64:]) * np.exp(1j * p * 1.0e4 ** (-2.0 * j / 128))
    want = np.concatenate([z.real, z.imag], axis=1)
    assert np.max(np.abs(got - want)) < 4e-3


def test_rope_depends_on_relative_position_only():
    x = rnd(7, (4, 2, 64))
    y = rnd(8, (4, 2, 64))
    def dot(bx, by):
        px = O.pool_block(x, O.block_pos(bx)).astype(np.float64)
        py = O.pool_block(y, O.block_pos(by)).astype(np.float64)
        return np.sum(px * py, axis=1)
    ref = dot(5, 2)
    for off in (0, 17, 1000, 60000):
        assert np.allclose(dot(5 + off, 2 + off), ref, atol=0.05)
    # and it does depend on the offset
    assert not np.allclose(dot(5, 3), ref, atol=0.05)


def test_incremental_cache_equals_rebuild_bitwise():
    H, d, n = 2, 32, 203
    raw_all = rnd(9, (n, H, d))
    ref = O.pool_rebuild(raw_all, n)
    # one token per call
    raw = np.zeros((n + 8, H, d), np.float16)
    pooled = np.zeros(((n + 8) // 4, H, d), np.float16)
    for t in range(n):
        O.pool_append(raw_all[t:t + 1], t, raw, pooled)
    assert np.array_equal(pooled[:n // 4].view(np.uint16), ref.view(np.uint16))
    # random chunk sizes
    raw2 = np.zeros_like(raw)
    pooled2 = np.zeros_like(pooled)
    r = np.random.default_rng(0)
    t = 0
    while t < n:
        c = int(min(n - t, r.integers(1, 19)))
        O.pool_append(raw_all[t:t + c], t, raw2, pooled2)
        t += c
    assert np.array_equal(pooled2.view(np.uint16), pooled.view(np.uint16))


# ------------------------------------------------------------------ scores
def test_score_matches_numpy_matmul():
    P = rnd(11, (300, 4, 64))
    q = rnd(12, (4, 64))
    s64, s32 = O.index_score(q, P, 300)
    ref = P.astype(np.float64).reshape(300, -1) @ q.astype(np.float64).ravel()
    assert np.allclose(s64, ref, rtol=1e-13, atol=1e-11)
    assert np.array_equal(s32, ref.astype(np.float32)) or \
        np.max(np.abs(s32.astype(np.float64) - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_score_of_a_pooled_row_with_itself_is_h_times_d():
    raw = rnd(13, (4 * 20, 16, 128))
    P = O.pool_rebuild(raw, raw.shape[0])
    s64, _ = O.index_score(P[7], P, 20)
    assert abs(s64[7] - 16 * 128) < 16 * 128 * 5e-3
    assert np.argmax(s64) == 7


# ------------------------------------------------------------------ selection
def _lexsort_topk(s, k):
    s = np.asarray(s, np.float32).astype(np.float64)
    key = np.where(np.isnan(s), -np.inf, s)
    nanrank = np.isnan(s).astype(np.int64)  # NaN after everything
    order = np.lexsort((np.arange(s.size), -key, nanrank))
    return np.sort(order[:min(k, s.size)]).astype(np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_topk_sort_rank_and_lexsort_agree(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 60))
    k = int(r.integers(1, 70))
    s = r.integers(-4, 5, n).astype(np.float32) * 0.5
    s[r.random(n) < 0.2] = -0.0
    a = O.topk_sort(s, k)
    b = O.topk_rank(s, k)
    c = _lexsort_topk(s, k)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert a.size == min(k, n) and np.all(np.diff(a) > 0)


def test_topk_crafted_cases():
    assert np.array_equal(O.topk_sort(np.ones(10, np.float32), 3), [0, 1, 2])
    assert np.array_equal(O.topk_sort(np.arange(5, dtype=np.float32), 9), np.arange(5))
    s = np.array([3, 1, 2, 5, 4], np.float32)
    assert np.array_equal(O.topk_sort(s, 4), [0, 2, 3, 4])            # k = n - 1
    s = np.array([0.0, -0.0, -0.0, 0.0, 1.0], np.float32)
    assert np.array_equal(O.topk_sort(s, 3), [0, 1, 4])                # -0 ties +0
    s = np.array([np.nan, -1e30, np.nan, 2.0], np.float32)
    assert np.array_equal(O.topk_sort(s, 2), [1, 3])                   # NaN lowest
    s = np.array([1, 2, 2, 2, 2, 0], np.float32)
    assert np.array_equal(O.topk_sort(s, 3), [1, 2, 3])                # ties at the cut
    assert O.topk_sort(np.zeros(0, np.float32), 4).size == 0


@pytest.mark.parametrize("seed", range(6))
def test_block_topk_equals_cell_topk(seed):
    # block-domain selection = cell-level selection of block scores spread to every
    # cell (ties by lowest cell), as the COMMON-006 section describes
    r = np.random.default_rng(100 + seed)
    nb = int(r.integers(5, 400))
    k = int(r.integers(1, 80))
    s = np.round(r.standard_normal(nb) * 3).astype(np.float32)
    cell_scores = np.repeat(s, 4)
    cell_sel = _lexsort_topk(cell_scores, 4 * k)
    blocks_from_cells = np.unique(cell_sel // 4).astype(np.int32)
    assert np.array_equal(O.topk_sort(s, k), blocks_from_cells)


def test_cells_closed_form_and_pages_maximum():
    g = json.load(open(GOLDEN))
    B = g["block_tokens"]["value"]
    k = g["indexer_top_k_tokens"]["value"] // B
    assert k == 512
    r = np.random.default_rng(5)
    for n in [0, 1, 3, 4, 5, 2047, 2048, 2051, 4096, 61789, 255181, 255183]:
        nb = n // B
        blk = np.sort(r.choice(max(nb, 1), size=min(k, nb), replace=False)).astype(np.int32)
        c = O.cells(blk, n)
        assert c.size == B * min(k, nb) + n % B
        assert np.all(c < n) and np.unique(c).size == c.size
        if n % B == 3 and nb >= k:
            assert c.size == g["max_cells"]["value"]
    assert O.cells(np.arange(512, dtype=np.int32), 255183).size == g["max_cells"]["value"]


# ------------------------------------------------------------------ attention
def _np_attn(q, K, V, cells, scale):
    hq, d = q.shape
    hkv = K.shape[1]
    G = hq // hkv
    out = np.empty((hq, V.shape[2]))
    for h in range(hq):
        k = K[cells, h // G].astype(np.float64)
        v = V[cells, h // G].astype(np.float64)
        p = softmax(scale * (k @ q[h].astype(np.float64)))
        out[h] = p @ v
    return out


def test_attention_matches_scipy_softmax_gqa():
    q, K, V = rnd(20, (8, 32)), rnd(21, (50, 2, 32)), rnd(22, (50, 2, 16))
    cells = np.array([3, 4, 5, 6, 20, 21, 22, 23, 48, 49])
    got = O.attn_cells(q, K, V, cells, 0.2)
    assert np.allclose(got, _np_attn(q, K, V, cells, 0.2), rtol=1e-12, atol=1e-12)


def test_gathered_equals_dense_masked():
    q, K, V = rnd(23, (4, 64)), rnd(24, (103, 1, 64)), rnd(25, (103, 1, 64))
    blk = np.array([2, 9, 17], np.int32)
    c = O.cells(blk, 103)
    vis = np.zeros(103, np.uint8)
    vis[c] = 1
    a = O.attn_cells(q, K, V, c, 0.125)
    b = O.attn_dense_masked(q, K, V, 103, vis, 0.125)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_full_selection_is_causal_attention():
    # nb <= k: every block is picked, so the step is plain softmax attention over
    # all N tokens
    sh = O.Shape(h_idx=2, d_idx=32, topk=64, hq=4, hkv=2, d=32, dv=32)
    n0 = 4 * 30 + 2
    raw = np.zeros((n0 + 8, 2, 32), np.float16)
    pooled = np.zeros(((n0 + 8) // 4, 2, 32), np.float16)
    Kc = np.zeros((n0 + 8, 2, 32), np.float16)
    Vc = np.zeros((n0 + 8, 2, 32), np.float16)
    O.pool_append(rnd(30, (n0, 2, 32)), 0, raw, pooled)
    Kc[:n0], Vc[:n0] = rnd(31, (n0, 2, 32)), rnd(32, (n0, 2, 32))
    q = rnd(33, (4, 32))
    res = O.decode_step(sh, raw, pooled, Kc, Vc, n0, rnd(34, (2, 32)), rnd(35, (2, 32)), q,
                        rnd(36, (2, 32)), rnd(37, (2, 32)))
    n = n0 + 1
    assert np.array_equal(res["blk"], np.arange(n // 4))
    ref = _np_attn(q, Kc, Vc, np.arange(n), 1 / np.sqrt(32))
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_zero_query_averages_selected_values():
    q = np.zeros((2, 16), np.float16)
    K, V = rnd(40, (40, 1, 16)), rnd(41, (40, 1, 16))
    c = np.array([1, 5, 9, 30])
    out = O.attn_cells(q, K, V, c, 1.0)
    assert np.allclose(out, V[c, 0].astype(np.float64).mean(0)[None], rtol=1e-13, atol=1e-14)


def test_single_cell_returns_its_value_row():
    q, K, V = rnd(42, (4, 16)), rnd(43, (10, 2, 16)), rnd(44, (10, 2, 8))
    out = O.attn_cells(q, K, V, np.array([6]), 0.3)
    assert np.array_equal(out[:2], V[[6, 6], 0].astype(np.float64))
    assert np.array_equal(out[2:], V[[6, 6], 1].astype(np.float64))


def test_mha_when_each_head_has_its_own_kv():
    q, K, V = rnd(45, (3, 16)), rnd(46, (12, 3, 16)), rnd(47, (12, 3, 16))
    c = np.arange(12)
    out = O.attn_cells(q, K, V, c, 0.25)
    for h in range(3):
        p = softmax(0.25 * K[:, h].astype(np.float64) @ q[h].astype(np.float64))
        assert np.allclose(out[h], p @ V[:, h].astype(np.float64), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ composed steps
def test_decode_step_selects_planted_blocks():
    w = synth.Workload("planted_small", 9, "decode", 4 * 2000 + 1, h_idx=4, d_idx=64, topk=32,
                       hq=4, hkv=1, d=32, dv=32, planted=8)
    L = synth.decode_layer(w, 0)
    n0 = L["n_prefix"]
    sh = O.Shape(4, 64, 32, 4, 1, 32, 32)
    cap = n0 + 8
    raw = np.zeros((cap, 4, 64), np.float16)
    pooled = np.zeros((cap // 4, 4, 64), np.float16)
    Kc = np.zeros((cap, 1, 32), np.float16)
    Vc = np.zeros((cap, 1, 32), np.float16)
    O.pool_append(L["raw"], 0, raw, pooled)
    Kc[:n0], Vc[:n0] = L["k"], L["v"]
    res = O.decode_step(sh, raw, pooled, Kc, Vc, n0, L["q_idx"], L["k_idx_new"][0], L["q"],
                        L["k_new"][0], L["v_new"][0])
    assert set(L["planted"].tolist()) <= set(res["blk"].tolist())
    s = res["scores64"]
    top8 = np.argsort(-s)[:8]
    assert set(top8.tolist()) == set(L["planted"].tolist())
    assert s[L["planted"]].min() > 0.9 * 4 * 64


def test_all_core_timing_form_equals_decode_step():
    # the benchmark's all-core oracle timing splits only the block scan over threads;
    # every result is the single-threaded decode step's, bit for bit
    w = synth.Workload("mt_small", 9, "decode", 4 * 3000 + 2, h_idx=4, d_idx=64, topk=32,
                       hq=4, hkv=1, d=32, dv=32)
    L = synth.decode_layer(w, 0)
    n0 = L["n_prefix"]
    sh = O.Shape(4, 64, 32, 4, 1, 32, 32)
    cap = n0 + 8

    def caches():
        raw = np.zeros((cap, 4, 64), np.float16)
        pooled = np.zeros((cap // 4, 4, 64), np.float16)
        Kc = np.zeros((cap, 1, 32), np.float16)
        Vc = np.zeros((cap, 1, 32), np.float16)
        O.pool_append(L["raw"], 0, raw, pooled)
        Kc[:n0], Vc[:n0] = L["k"], L["v"]
        return raw, pooled, Kc, Vc

    args = (n0, L["q_idx"], L["k_idx_new"][0], L["q"], L["k_new"][0], L["v_new"][0])
    ref = O.decode_step(sh, *caches(), *args)
    for threads in (1, 3, 8, 64):
        got = O.decode_step_mt(sh, *caches(), *args, threads=threads)
        assert np.array_equal(got["scores64"], ref["scores64"])
        assert np.array_equal(got["blk"], ref["blk"])
        assert np.array_equal(got["out"], ref["out"])


def test_prefill_row_equals_decode_at_that_length():
    sh = O.Shape(2, 32, 8, 4, 2, 32, 32)
    n_all = 4 * 40 + 3
    raw_all, K, V = rnd(50, (n_all, 2, 32)), rnd(51, (n_all, 2, 32)), rnd(52, (n_all, 2, 32))
    pooled = O.pool_rebuild(raw_all, n_all)
    qi, q = rnd(53, (2, 32)), rnd(54, (4, 32))
    for pos in (n_all - 1, n_all - 2, 100, 37):
        row = O.prefill_row(sh, pooled, K, V, pos, qi, q)
        raw = np.zeros((n_all + 4, 2, 32), np.float16)
        pl = np.zeros(((n_all + 4) // 4, 2, 32), np.float16)
        Kc = np.zeros((n_all + 4, 2, 32), np.float16)
        Vc = np.zeros((n_all + 4, 2, 32), np.float16)
        O.pool_append(raw_all[:pos], 0, raw, pl)
        Kc[:pos], Vc[:pos] = K[:pos], V[:pos]
        dec = O.decode_step(sh, raw, pl, Kc, Vc, pos, qi, raw_all[pos], q, K[pos], V[pos])
        assert np.array_equal(row["blk"], dec["blk"])
        assert np.array_equal(row["out"], dec["out"])


# ------------------------------------------------------------------ MLA list path
def test_mask_list_is_flatnonzero():
    g = json.load(open(GOLDEN))
    w = synth.Workload("mla_small", 8, "mla", 8192, hq=4, hkv=1, d=576, dv=512, list_len=1024)
    assert w.n_tokens >= g["mla_min_key_len"]["value"]
    assert w.n_tokens >= g["mla_key_len_over_list_cap"]["value"] * w.list_len
    for runs in (False, True):
        m = synth.mla_inputs(w, runs=runs)
        lst = O.mask_list(m["mask"])
        assert np.array_equal(lst, np.flatnonzero(m["mask"] != -np.inf))
        assert np.array_equal(lst, m["positions"])


def test_mla_list_equals_dense_and_scipy():
    n, hq, dkq, dv = 700, 3, 576, 512
    kv, q = rnd(60, (n, dkq)), rnd(61, (hq, dkq))
    mask = np.full(n, -np.inf, np.float16)
    pos = np.sort(np.random.default_rng(62).choice(n, 90, replace=False))
    mask[pos] = 0
    lst = O.mask_list(mask)
    sc = 1 / np.sqrt(dkq)
    a = O.mla_attn(q, kv, None, mask, lst, dv, sc)
    b = O.mla_dense(q, kv, None, mask, dv, sc)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    k64 = kv.astype(np.float64)
    for h in range(hq):
        p = softmax(sc * k64[pos] @ q[h].astype(np.float64))
        assert np.allclose(a[h], p @ k64[pos, :dv], rtol=1e-12, atol=1e-13)
    # a separate V array is used when given
    V = rnd(63, (n, dv))
    c = O.mla_attn(q, kv, V, mask, lst, dv, sc)
    p = softmax(sc * k64[pos] @ q[0].astype(np.float64))
    assert np.allclose(c[0], p @ V[pos].astype(np.float64), rtol=1e-12, atol=1e-13)


def test_mask_list_edges_and_finite_bias():
    # first and last positions visible; a finite non-zero mask value is visible and
    # is added to the logit
    n = 4096
    mask = np.full(n, -np.inf, np.float16)
    mask[[0, 1, 63, 64, 4095]] = [0.0, -1.5, 0.0, 2.0, 0.0]
    lst = O.mask_list(mask)
    assert np.array_equal(lst, [0, 1, 63, 64, 4095])
    kv, q = rnd(70, (n, 576)), rnd(71, (2, 576))
    sc = 0.05
    out = O.mla_attn(q, kv, None, mask, lst, 512, sc)
    k64 = kv.astype(np.float64)
    for h in range(2):
        p = softmax(sc * k64[lst] @ q[h].astype(np.float64) + mask[lst].astype(np.float64))
        assert np.allclose(out[h], p @ k64[lst, :512], rtol=1e-12, atol=1e-13)
