"""QSA layer-step benchmark on one MI355X.

Default workload: decode at N = 255,181 tokens, indexer 16 x 128, top-k 512 blocks,
attention 32/4 x 128, 12 independent layer states stepped serially per token (a
real model chains its layers), 8 planted blocks per layer.  One bench step is one
token: the 12 layers one after another.  The token position cycles through
N-1, N, N+1, N+2 (tails 1, 2, 3 and a completed block), then rewinds.

Reported:
  value        layer decode steps/s (= 12 * tokens / s)
  roofline     the decode step's scoring kernel (appends + pooled-key scan +
               candidate lists): algorithmic bytes per launch / its average
               duration, from the kernel's own start/end events (qsa_trace_scan) on
               the stream it runs on, against 8 TB/s; plus HBM traffic per launch
               from rocprofv3 counters when they were taken on the current kernel
               source; "standalone" gives the same for qsa_index_score's scan
  step_hbm     algorithmic bytes of a whole layer step / measured step time
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Other workloads (one JSON line each, same keys): prefill_1024_at_126253 (prefill
chunk tokens/s; roofline = MFMA scoring against the f16 dense peak, timed alone
over three pooled-cache copies in turn so that none is left in cache, plus the
attention's K/V GB/s for the per-row form and the bytes / MFMA rate of the
grouped-union form; --per-row makes the step use the per-row form),
prefill_1024_at_126253_corr (the same caches with indexer queries correlated from
row to row, so that nearby rows choose overlapping blocks) and mla_list_262144
(list-attention calls/s, latency-bound).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA layer decode steps/s at 256k ctx + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_decode_qsa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, source: str, workload: str):
    """Counter-measured HBM bytes per launch, only if taken on this workload and on
    the current source."""
    try:
        t = json.load(open(TRAFFIC_FILE))[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != src_hash(source):
        return None
    return t.get("bytes_per_launch")


def hold_cycles(stream, ms: float) -> int:
    """Spin cycles of torch.cuda._sleep that hold `stream` for about `ms`."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 20
    with torch.cuda.stream(stream):
        a.record(stream)
        torch.cuda._sleep(n)
        b.record(stream)
    b.synchronize()
    return int(n * ms / max(a.elapsed_time(b), 1e-3))


def decode_bytes(w, nb, cells):
    """Algorithmic bytes of one decode layer step (see the design notes)."""
    row = w.h_idx * w.d_idx * 2
    scan = nb * row
    kv = cells * w.hkv * (w.d + w.dv) * 2
    small = (row                      # indexer query
             + w.hq * w.d * 2         # attention query
             + w.hq * w.dv * 4        # fp32 output
             + row                    # raw indexer key written
             + w.hkv * (w.d + w.dv) * 2)  # new K/V row written
    return scan, kv, small


def host_threads() -> int:
    """Host cores this process may use (its affinity mask), at most 16: the CPU share
    of one GPU on the boxes this runs on."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run_cpu_baseline(w, L, budget_s):
    """The oracle's decode step on layer 0 of the same workload, timed two ways:
    (i) the parity oracle on one thread; (ii) the same step with its block scan split
    over every usable host core (oracle/qsa_oracle_mt.c; identical results)."""
    import oracle as O
    n0 = L["n_prefix"]
    cap = w.cap_tokens
    raw = np.zeros((cap, w.h_idx, w.d_idx), np.float16)
    pooled = np.zeros((cap // 4, w.h_idx, w.d_idx), np.float16)
    kc = np.zeros((cap, w.hkv, w.d), np.float16)
    vc = np.zeros((cap, w.hkv, w.dv), np.float16)
    t0 = time.time()
    O.pool_append(L["raw"], 0, raw, pooled)
    kc[:n0], vc[:n0] = L["k"], L["v"]
    log(f"[cpu] oracle cache build {time.time() - t0:.1f}s")
    sh = O.Shape(w.h_idx, w.d_idx, w.topk, w.hq, w.hkv, w.d, w.dv)

    def timed(step, budget):
        steps = 0
        t0 = time.perf_counter()
        while True:
            j = steps % 4
            step(n0 + j, L["k_idx_new"][j], L["k_new"][j], L["v_new"][j])
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget or steps >= 64:
                return steps, el

    one = lambda n, ki, kn, vn: O.decode_step(sh, raw, pooled, kc, vc, n, L["q_idx"], ki,
                                               L["q"], kn, vn)
    s1, e1 = timed(one, budget_s * 2 / 3)
    threads = host_threads()
    many = lambda n, ki, kn, vn: O.decode_step_mt(sh, raw, pooled, kc, vc, n, L["q_idx"], ki,
                                                   L["q"], kn, vn, threads=threads)
    s2, e2 = timed(many, budget_s / 3)
    log(f"[cpu] oracle: 1 thread {s1 / e1:.2f}, {threads} threads {s2 / e2:.2f} layer-steps/s")
    return dict(value=s1 / e1, unit="layer-steps/s", cores=1, kind="oracle",
                sample=f"{s1} oracle decode steps on layer 0 at N={w.n_tokens} "
                       f"(positions cycling N-1..N+2), single thread, {e1:.1f} s",
                all_cores=dict(value=s2 / e2, unit="layer-steps/s", cores=threads,
                               sample=f"{s2} oracle decode steps, same positions, block scan "
                                      f"split over {threads} threads, {e2:.1f} s"))


def bench_decode(args):
    import torch
    from sparse_attention_decode_qsa_amd import binding as qb
    import synth

    w = synth.WORKLOADS[args.workload]
    n_layers = args.layers or w.n_layers
    dev = torch.device("cuda:0")
    qb.load()
    cfg = qb.Config(h_idx=w.h_idx, d_idx=w.d_idx, topk_blocks=w.topk, hq=w.hq, hkv=w.hkv, d=w.d,
                    dv=w.dv, cap_tokens=w.cap_tokens)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    layers, host0 = [], None
    t0 = time.time()
    for li in range(n_layers):
        L = synth.decode_layer(w, li)
        g = qb.Layer(cfg, dev)
        qb.qsa_pool_append(cfg, t(L["raw"]), 0, g.k_raw, g.k_pool)
        g.k_cache[:L["n_prefix"]] = t(L["k"])
        g.v_cache[:L["n_prefix"]] = t(L["v"])
        st = dict(layer=g, q_idx=t(L["q_idx"]), q=t(L["q"]), k_idx_new=t(L["k_idx_new"]),
                  k_new=t(L["k_new"]), v_new=t(L["v_new"]),
                  out=torch.empty((w.hq, w.dv), dtype=torch.float32, device=dev))
        layers.append(st)
        if li == 0:
            host0 = L
        torch.cuda.synchronize()
        log(f"[setup] layer {li} ready ({time.time() - t0:.1f}s)")
    n0 = host0["n_prefix"]
    rows = args.rows
    ws = qb.workspace(cfg, rows, w.cap_tokens, dev)
    flags = qb.QSA_STEP_COMPACT_GATHER if args.compact_gather else qb.QSA_STEP_FUSED_GATHER
    # positions cycle over the 4 new tokens of each layer (rows > 1: verification
    # steps over tokens j .. j + rows - 1, every row with the layer's queries)
    n_pos = 4 - rows + 1
    if rows > 1:
        for st in layers:
            st["q_idx_r"] = st["q_idx"].unsqueeze(0).repeat(rows, 1, 1).contiguous()
            st["q_r"] = st["q"].unsqueeze(0).repeat(rows, 1, 1).contiguous()
            st["out_r"] = torch.empty((rows, w.hq, w.dv), dtype=torch.float32, device=dev)

    def layer_step(st, j):
        if rows == 1:
            qb.qsa_decode_step(cfg, st["layer"], n0 + j, st["q_idx"], st["k_idx_new"][j],
                               st["q"], st["k_new"][j], st["v_new"][j], st["out"], ws,
                               flags=flags)
        else:
            qb.qsa_decode_multi(cfg, st["layer"], n0 + j, st["q_idx_r"],
                                st["k_idx_new"][j:j + rows], st["q_r"],
                                st["k_new"][j:j + rows], st["v_new"][j:j + rows],
                                st["out_r"], ws)

    def token(j):
        for st in layers:
            layer_step(st, j)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for j in range(n_pos):
            token(j)          # eager: also sets kernel attributes before any capture
    stream.synchronize()

    graphs = []
    if not args.eager:
        for j in range(n_pos):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                token(j)
            graphs.append(gr)
        stream.synchronize()

    def run_tokens(i0, n):
        with torch.cuda.stream(stream):
            for i in range(i0, i0 + n):
                if graphs:
                    graphs[i % n_pos].replay()
                else:
                    token(i % n_pos)

    run_tokens(0, args.warmup)
    stream.synchronize()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run_tokens(args.warmup, args.steps)
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    tok_s = args.steps / (ms / 1e3)
    layer_steps_s = tok_s * n_layers
    log(f"[time] {args.steps} tokens x {n_layers} layers in {ms:.2f} ms")

    # dominant kernel: the decode step's scan (appends, block scores, candidate
    # lists), the kernel's own start and end times taken through qsa_trace_scan on
    # eager steps in the timed region's order (layers, then positions), on its stream
    per_cycle = n_layers * n_pos
    reps = per_cycle * max(1, args.kernel_reps // per_cycle)
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    with torch.cuda.stream(stream):
        for e in tev:
            e.record(stream)  # creates the events
        # hold the stream until the host has queued every step, so that the steps run
        # back to back as in the graphs, not one by one behind the host
        torch.cuda._sleep(hold_cycles(stream, args.trace_hold_ms))
        for r in range(reps):
            qb.qsa_trace_scan(tev[2 * r], tev[2 * r + 1])
            layer_step(layers[r % n_layers], (r // n_layers) % n_pos)
    stream.synchronize()
    scan_us = sum(tev[2 * r].elapsed_time(tev[2 * r + 1]) for r in range(reps)) * 1e3 / reps
    # scan bytes of the step: the rows complete before the call (the position cycle's
    # mean), the appended block's row read back from LDS, not from HBM
    row = w.h_idx * w.d_idx * 2
    scan_bytes = float(np.mean([((w.n_tokens - 1 + j) // 4) * row for j in range(n_pos)]))
    achieved = scan_bytes / (scan_us * 1e-6) / 1e9
    rowc = w.h_idx * w.d_idx // 8
    step_kernel = f"score_decode_kernel<{rowc},{2 if rowc >= 128 else 4},512,{rows},true,true>"

    # the stand-alone scan (qsa_index_score), back to back over the layers' caches,
    # each launch's own start and end times
    nb = w.n_tokens // 4
    scores = torch.empty(nb + 64, dtype=torch.float32, device=dev)
    sreps = 12 * max(1, args.kernel_reps // 12)
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * sreps)]
    with torch.cuda.stream(stream):
        for e in sev:
            e.record(stream)
        for r in range(12):
            st = layers[r % n_layers]
            qb.qsa_index_score(cfg, st["q_idx"], w.n_tokens - 1, st["layer"].k_pool, scores)
        torch.cuda._sleep(hold_cycles(stream, args.trace_hold_ms))
        for r in range(sreps):
            st = layers[r % n_layers]
            qb.qsa_trace_scan(sev[2 * r], sev[2 * r + 1])
            qb.qsa_index_score(cfg, st["q_idx"], w.n_tokens - 1, st["layer"].k_pool, scores)
    stream.synchronize()
    alone_us = sum(sev[2 * r].elapsed_time(sev[2 * r + 1]) for r in range(sreps)) * 1e3 / sreps
    alone_bytes = nb * row
    alone_gbps = alone_bytes / (alone_us * 1e-6) / 1e9

    # whole-step algorithmic bandwidth, averaged over the 4-step position cycle
    per = []
    for j in range(n_pos):
        b = []
        for r in range(rows):
            N = w.n_tokens + j + r
            nbj = N // 4
            cells = 4 * min(w.topk, nbj) + N % 4
            b.append(decode_bytes(w, nbj, cells))
        # the pooled cache is streamed once per step, whatever the number of rows
        per.append(b[-1][0] + sum(sum(x[1:]) for x in b))
    step_bytes = float(np.mean(per))
    step_s = (ms / 1e3) / (args.steps * n_layers)
    step_gbps = step_bytes / step_s / 1e9

    res = {
        "metric": METRIC if w.n_tokens == 255181 else
        METRIC.replace("at 256k ctx", f"at {w.n_tokens:,}-token ctx"),
        "value": round(layer_steps_s, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "n_tokens": w.n_tokens, "layers_per_token": n_layers,
            "indexer": f"{w.h_idx}x{w.d_idx}", "topk_blocks": w.topk,
            "attention": f"{w.hq}/{w.hkv}x{w.d}", "planted_blocks": w.planted,
            "step": "one token = all layers, serially; position cycles N-1..N+2",
            "launch": "eager" if args.eager else "hip graph per token",
            "gather": "compact" if args.compact_gather else "fused",
            "token_steps_per_s": round(tok_s, 2),
        },
        "roofline": {
            "bound": "hbm", "kernel": step_kernel,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_for("score_decode_step_kernel", "k_score.hip", w.name),
            "algorithmic_bytes_per_launch": int(scan_bytes),
            "avg_launch_us": round(scan_us, 3),
            "timing": f"kernel start/end events of {reps} eager decode steps (qsa_trace_scan)",
            "standalone": {
                "kernel": f"score_decode_kernel<{rowc},{2 if rowc >= 128 else 4},512,1,false,false>",
                "achieved": round(alone_gbps, 1), "frac": round(alone_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for("score_decode_kernel", "k_score.hip", w.name),
                "algorithmic_bytes_per_launch": alone_bytes,
                "avg_launch_us": round(alone_us, 3),
                "timing": f"kernel start/end events of {sreps} back-to-back qsa_index_score "
                          f"launches (qsa_trace_scan)",
            },
        },
        "step_hbm": {
            "algorithmic_bytes_per_layer_step": int(step_bytes),
            "achieved": round(step_gbps, 1), "unit": "GB/s",
            "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
            "us_per_layer_step": round(step_s * 1e6, 3),
        },
    }
    if rows > 1:
        res["metric"] = (f"QSA layer verification steps/s ({rows} query rows) at "
                         + ("256k ctx" if w.n_tokens == 255181 else f"{w.n_tokens:,}-token ctx"))
        res["unit"] = "layer-verify-steps/s"
        res["config"]["rows"] = rows
        res["config"]["step"] = (f"one verification step = all layers, serially, each appending "
                                 f"and attending {rows} query rows (qsa_decode_multi)")
        res["config"]["query_rows_per_s"] = round(layer_steps_s * rows, 2)
    if not args.no_cpu_baseline:
        cb = run_cpu_baseline(w, host0, args.cpu_budget)
        if rows > 1:  # the oracle checks rows one decode step at a time
            cb["value"] /= rows
            cb["unit"] = "layer-verify-steps/s"
            cb["sample"] += f"; a verification step is {rows} of them"
        res["cpu_baseline"] = cb
    return res


def _timed(stream, fn, reps):
    """Average µs of fn() over reps launches on stream (HIP events on that stream)."""
    import torch
    with torch.cuda.stream(stream):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _contract(metric, value, unit, steps, warmup, ms, dtype, config, roofline, hib=True):
    return {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": hib, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config, "roofline": roofline}


def bench_prefill(args):
    """One prefill chunk: 1024 query rows at depth 126,253, each row with its own
    causal prefix (append, MFMA scores, per-row top-k, per-row sparse attention)."""
    import torch
    from sparse_attention_decode_qsa_amd import binding as qb
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    qb.load()
    cfg = qb.Config(h_idx=w.h_idx, d_idx=w.d_idx, topk_blocks=w.topk, hq=w.hq, hkv=w.hkv, d=w.d,
                    dv=w.dv, cap_tokens=w.cap_tokens)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    t0 = time.time()
    I = synth.prefill_inputs(w, 0)
    depth, n_q = I["depth"], w.n_q
    g = qb.Layer(cfg, dev)
    qb.qsa_pool_append(cfg, t(I["raw"][:depth]), 0, g.k_raw, g.k_pool)
    g.k_cache[:depth] = t(I["k"][:depth])
    g.v_cache[:depth] = t(I["v"][:depth])
    q_idx, q = t(I["q_idx"]), t(I["q"])
    raw_new, k_new, v_new = t(I["raw"][depth:]), t(I["k"][depth:]), t(I["v"][depth:])
    torch.cuda.synchronize()
    log(f"[setup] prefill caches ready ({time.time() - t0:.1f}s)")
    nb_end = (depth + n_q) // 4
    ld = (nb_end + 1 + 63) // 64 * 64
    out = torch.empty((n_q, w.hq, w.dv), dtype=torch.float32, device=dev)
    scores = torch.empty((n_q, ld), dtype=torch.float32, device=dev)
    blk = torch.empty((n_q, w.topk), dtype=torch.int32, device=dev)
    nsel = torch.empty(n_q, dtype=torch.int32, device=dev)
    ws = qb.workspace(cfg, n_q, depth + n_q, dev)
    stream = torch.cuda.Stream()

    flags = qb.QSA_PREFILL_PER_ROW if args.per_row else qb.QSA_PREFILL_GROUPED_UNION

    def step():
        qb.qsa_prefill_step(cfg, g, depth, q_idx, raw_new, q, k_new, v_new, out, ws,
                            scores_out=scores, ld_scores=ld, blk_out=blk, flags=flags)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    stream.synchronize()
    step_us = _timed(stream, step, args.steps)
    # the stages alone, on the caches the step leaves behind.  The scoring kernel
    # rotates over three copies of the pooled cache (3 x 130 MB, more than the
    # 256 MB last-level cache), so no launch finds its operand left in cache by the
    # previous one, as inside a step
    pools = [g.k_pool] + [g.k_pool.clone() for _ in range(2)]
    turn = [0]

    def score_once():
        qb.qsa_index_score(cfg, q_idx, depth, pools[turn[0] % len(pools)], scores, ld=ld)
        turn[0] += 1

    # plain launches back to back (a scoring launch takes ~150 us, the gaps ~1%): with
    # start/stop events on the launch this kernel itself runs ~7% slower
    score_us = _timed(stream, score_once, args.steps)
    topk_us = _timed(stream, lambda: qb.qsa_topk_blocks(cfg, scores, n_q, ld, depth, blk, nsel,
                                                        ws), args.steps)
    attn_row_us = _timed(stream, lambda: qb.qsa_prefill_attn(
        cfg, q, depth, blk, w.topk, g.k_cache, g.v_cache, out, ws), args.steps)
    attn_union_us = _timed(stream, lambda: qb.qsa_prefill_attn(
        cfg, q, depth, blk, w.topk, g.k_cache, g.v_cache, out, ws,
        flags=qb.QSA_PREFILL_GROUPED_UNION), args.steps)
    attn_union_all_us = _timed(stream, lambda: qb.qsa_prefill_attn(
        cfg, q, depth, blk, w.topk, g.k_cache, g.v_cache, out, ws,
        flags=qb.QSA_PREFILL_GROUPED_UNION | qb.QSA_PREFILL_UNION_ALL), args.steps)
    attn_us = attn_row_us if args.per_row else attn_union_us
    nbs = [(depth + r + 1) // 4 for r in range(n_q)]
    flop = 2.0 * w.h_idx * w.d_idx * float(sum(nbs))
    cells = [4 * min(w.topk, nb) + (depth + r + 1) % 4 for r, nb in enumerate(nbs)]
    kv_bytes = float(sum(cells)) * w.hkv * (w.d + w.dv) * 2
    tflops = flop / (score_us * 1e-6) / 1e12
    # the union form: blocks per group of 128 / (hq / hkv) rows, K/V bytes it streams
    # (each union block and the tail span once per group) and the MFMA work it does
    # (128 queries x every streamed cell, QK^T and PV, per KV head)
    G = 128 // (w.hq // w.hkv)
    b_host = blk.cpu().numpy()
    ublocks, ucells = [], 0
    u_limit = (G * w.topk * 3) // 8  # groups past it are attended per row
    for r0 in range(0, n_q, G):
        r1 = min(n_q, r0 + G)
        ids = np.unique(np.concatenate([b_host[r, :min(w.topk, nbs[r])] for r in range(r0, r1)]))
        t0c = 4 * nbs[r0]
        t1c = depth + r1
        tail_blocks = (t1c - 1) // 4 - t0c // 4 + 1 if t1c > t0c else 0
        ublocks.append(ids.size)
        ucells += 4 * (ids.size + tail_blocks)
    u_bytes = float(ucells) * w.hkv * (w.d + w.dv) * 2
    u_flop = 2.0 * 2.0 * 128 * float(ucells) * w.d * w.hkv
    res = _contract(
        "QSA prefill chunk tokens/s (1024 queries at depth 126,253)", n_q / (step_us * 1e-6),
        "tokens/s", args.steps, args.warmup, step_us / 1e3, "f16",
        {"workload": w.name, "depth": depth, "n_q": n_q, "indexer": f"{w.h_idx}x{w.d_idx}",
         "topk_blocks": w.topk, "attention": f"{w.hq}/{w.hkv}x{w.d}", "launch": "eager",
         "indexer_query_rows": (f"AR(1) over rows, rho {w.q_corr}" if w.q_corr
                                else "independent"),
         "attention_form": "per-row" if args.per_row else "grouped union"},
        {"bound": "mfma", "kernel": "score_prefill_kernel", "achieved": round(tflops, 2),
         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
         "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
         "traffic": traffic_for("score_prefill_kernel", "k_score_mfma.hip", w.name),
         "algorithmic_flop_per_launch": flop, "avg_launch_us": round(score_us, 2)})
    res["stages_us"] = {"step": round(step_us, 2), "score": round(score_us, 2),
                        "topk": round(topk_us, 2), "attn": round(attn_us, 2),
                        "attn_per_row": round(attn_row_us, 2),
                        "attn_grouped_union": round(attn_union_us, 2),
                        "attn_union_every_group": round(attn_union_all_us, 2)}
    # per-row form: K/V bytes the rows request (a row's cells, every KV head); most
    # are served by the last-level cache, so the rate is a gather rate, and the HBM
    # bytes come from the counters when taken on the current kernel source
    res["attention_per_row"] = {
        "form": "per-row (rows_attn_kernel)", "kv_bytes_requested": kv_bytes,
        "gather_gbps": round(kv_bytes / (attn_row_us * 1e-6) / 1e9, 1),
        "hbm_traffic_bytes": traffic_for("rows_attn_kernel", "k_rows.hip", w.name),
        "avg_launch_us": round(attn_row_us, 2)}
    res["attention_union"] = {
        "form": "grouped union, every group (QSA_PREFILL_UNION_ALL)", "rows_per_group": G,
        "union_blocks_per_group": round(float(np.mean(ublocks)), 1),
        "union_over_k": round(float(np.mean(ublocks)) / w.topk, 3),
        "groups_per_row_by_default": int(sum(1 for u in ublocks if u > u_limit)),
        "groups": len(ublocks),
        "kv_bytes_streamed": u_bytes,
        "kv_achieved_gbps": round(u_bytes / (attn_union_all_us * 1e-6) / 1e9, 1),
        "counter_traffic_bytes": traffic_for("union_attn_kernel", "k_union.hip", w.name),
        "mfma_flop": u_flop,
        "mfma_achieved_tflops": round(u_flop / (attn_union_all_us * 1e-6) / 1e12, 2),
        "mfma_frac": round(u_flop / (attn_union_all_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                           4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w, I, args.cpu_budget)
    return res


def cpu_baseline_prefill(w, I, budget_s):
    """Oracle prefill rows (each a decode-equivalent row): (i) one thread, (ii) rows
    spread over every usable host core (the oracle releases the interpreter lock)."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    depth = I["depth"]
    n_all = depth + w.n_q
    t0 = time.time()
    pooled = O.pool_rebuild(I["raw"], n_all)
    log(f"[cpu] oracle pooled rebuild {time.time() - t0:.1f}s")
    sh = O.Shape(w.h_idx, w.d_idx, w.topk, w.hq, w.hkv, w.d, w.dv)

    def row(i):
        r = (i * 97) % w.n_q
        O.prefill_row(sh, pooled, I["k"], I["v"], depth + r, I["q_idx"][r], I["q"][r])

    rows = 0
    t0 = time.perf_counter()
    while True:
        row(rows)
        rows += 1
        el = time.perf_counter() - t0
        if el >= budget_s * 2 / 3 or rows >= 64:
            break
    threads = host_threads()
    n_mt = min(64, 4 * threads)
    t1 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(row, range(n_mt)))
    el_mt = time.perf_counter() - t1
    log(f"[cpu] oracle prefill rows: 1 thread {rows / el:.2f}/s, {threads} threads "
        f"{n_mt / el_mt:.2f}/s")
    return dict(value=rows / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{rows} oracle prefill rows of the chunk (positions depth+r), single "
                       f"thread, {el:.1f} s",
                measured_rows=rows,
                extrapolated_chunk_s=round(w.n_q * el / rows, 1),
                all_cores=dict(value=n_mt / el_mt, unit="tokens/s", cores=threads,
                               sample=f"{n_mt} oracle prefill rows on {threads} threads, "
                                      f"{el_mt:.1f} s",
                               extrapolated_chunk_s=round(w.n_q * el_mt / n_mt, 1)))


def bench_mla(args):
    """MLA-style list attention at N = 262,144 with 2,048 visible positions: one call per
    layer state (its own latent rows, mask and queries), the states taken in turn."""
    import torch
    from sparse_attention_decode_qsa_amd import binding as qb
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    qb.load()
    n_layers = args.layers or 8
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    states = []
    I = None
    for layer in range(n_layers):
        Il = synth.mla_inputs(w, layer=layer)
        if layer == 0:
            I = Il
        states.append((t(Il["q"]), t(Il["kv"]), t(Il["mask"])))
    ws = torch.zeros(qb.qsa_mla_workspace_size(w.hq, w.dv, w.list_len), dtype=torch.uint8,
                     device=dev)
    qb.qsa_workspace_init(ws)
    out = torch.empty((w.hq, w.dv), dtype=torch.float32, device=dev)
    n_list = torch.zeros(1, dtype=torch.int32, device=dev)
    scale = 1.0 / float(np.sqrt(w.d))
    stream = torch.cuda.Stream()

    def call(i):
        q, kv, mask = states[i % n_layers]
        qb.qsa_mla_sparse_attn(q, kv, None, mask, w.list_len, scale, n_list, out, ws)

    def all_layers():
        for i in range(n_layers):
            call(i)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            call(i)
    stream.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        all_layers()
    stream.synchronize()
    reps = max(1, args.steps // n_layers)
    eager_us = _timed(stream, all_layers, reps) / n_layers
    graph_us = _timed(stream, gr.replay, reps) / n_layers
    nbytes = w.n_tokens * 2 + w.list_len * w.d * 2 + w.hq * w.d * 2 + w.hq * w.dv * 4
    res = _contract(
        "QSA MLA list attention calls/s (N = 262,144, 2,048 visible)", 1e6 / graph_us, "calls/s",
        reps * n_layers, args.warmup, graph_us / 1e3, "f16",
        {"workload": w.name, "n": w.n_tokens, "list": w.list_len, "hq": w.hq,
         "dkq": w.d, "dv": w.dv, "layer_states": n_layers,
         "launch": f"hip graph of {n_layers} calls, one per layer state"},
        {"bound": "latency", "kernel": "mla path (mask list + attention + combine)",
         "achieved": round(nbytes / (graph_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
         "unit": "GB/s", "frac": round(nbytes / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
         "traffic": None, "algorithmic_bytes_per_launch": nbytes,
         "avg_launch_us": round(graph_us, 2)})
    res["eager_us"] = round(eager_us, 2)
    if not args.no_cpu_baseline:
        import oracle as O
        lst = O.mask_list(I["mask"])
        calls = 0
        t0 = time.perf_counter()
        while True:
            O.mla_attn(I["q"], I["kv"], None, I["mask"], lst, w.dv, scale)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or calls >= 64:
                break
        res["cpu_baseline"] = dict(value=calls / el, unit="calls/s", cores=1, kind="oracle",
                                   sample=f"{calls} oracle list-attention calls on the same "
                                          f"inputs, single thread, {el:.1f} s")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_255181",
                    choices=["decode_255181", "decode_126253", "decode_61789", "decode_31898",
                             "tiny_decode_4k",
                             "prefill_1024_at_126253", "prefill_1024_at_126253_corr",
                             "mla_list_262144"])
    ap.add_argument("--layers", type=int, default=0, help="override the layer count")
    ap.add_argument("--eager", action="store_true", help="launch per call instead of graphs")
    ap.add_argument("--compact-gather", action="store_true")
    ap.add_argument("--rows", type=int, default=1, choices=[1, 2, 3, 4],
                    help="query rows per layer step (> 1: speculative-draft verification "
                         "steps, qsa_decode_multi)")
    ap.add_argument("--per-row", action="store_true",
                    help="prefill: per-row attention instead of the grouped-union form")
    ap.add_argument("--kernel-reps", type=int, default=240)
    ap.add_argument("--trace-hold-ms", type=float, default=40.0,
                    help="stream hold before the traced decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (a counter "
                         "calibration kernel of known size for rocprofv3 --pmc runs), then a "
                         "fill and a sum of the same size (cross-checks)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the QSA layer step has no multi-GPU path "
              "(its sharding is a design note); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy_mib:
        import torch
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        # two more kernels of known traffic, to cross-check the copy's factors: a
        # fill writes n bytes and reads none, a sum reads n bytes and writes a few
        for _ in range(3):
            dst.fill_(2)
        tot = [src.view(torch.float32).sum() for _ in range(3)]
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 3, "fills": 3, "sums": len(tot)}),
              flush=True)
        return
    if args.workload.startswith("prefill"):
        res = bench_prefill(args)
    elif args.workload.startswith("mla"):
        res = bench_mla(args)
    else:
        res = bench_decode(args)
    if "cpu_baseline" in res:
        res["cpu_baseline"].update(host_cpu())
    print(json.dumps(res), flush=True)


def host_cpu() -> dict:
    """The host the oracle ran on: CPU model and logical core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_logical_cores": os.cpu_count(),
            "usable_cores": host_threads()}


if __name__ == "__main__":
    main()
