"""Summarises rocprofv3 counter CSVs into HBM bytes per kernel launch.

    python -m sparse_attention_decode_qsa_amd.counters \
        --fetch K_FETCH.csv --write K_WRITE.csv \
        --calib-fetch C_FETCH.csv --calib-write C_WRITE.csv --calib-mib 256 \
        --kernel <substring of the mangled name> --key score_decode_kernel \
        --workload decode_255181 [--json profiles/traffic.json]

FETCH_SIZE and WRITE_SIZE (KiB per dispatch; each counter in a run of its own)
are averaged over the dispatches whose kernel name contains --kernel.  The
calibration runs (bench.py --calib-copy-mib N: a device-to-device copy of N MiB,
nothing else) give the scale factor per counter: the bytes the copy must read
(or write) / what the counter reports for the copy dispatches.  The JSON file
holds one entry per (key, workload): a figure is valid only for the workload it
was taken on.

    python -m sparse_attention_decode_qsa_amd.counters --cross-check \
        --calib-fetch C_FETCH.csv --calib-write C_WRITE.csv --calib-mib 256

prints the factors that the calibration run's fill and sum kernels imply, beside the
copy's.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))


def per_dispatch(path: str, counter: str) -> dict:
    """{(dispatch id, kernel name): value} for one counter."""
    vals = defaultdict(float)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            vals[(row["Dispatch_Id"], row["Kernel_Name"])] += float(row["Counter_Value"])
    return vals


def mean_kib(path: str, counter: str, sub: str, ids=None):
    """Mean over the dispatches whose name contains `sub` (and whose id is in `ids`,
    when given), and their count."""
    v = [x for (d, name), x in per_dispatch(path, counter).items()
         if sub in name and (ids is None or d in ids)]
    if not v:
        raise SystemExit(f"no dispatch matching {sub!r} in {path}")
    return sum(v) / len(v), len(v)


def ids_with_fetch(path: str, sub: str, min_kib: float) -> set:
    """Dispatch ids of the kernel whose FETCH_SIZE is at least min_kib (the runs of
    one command give the same ids, so the WRITE_SIZE run is read for the same ones)."""
    return {d for (d, name), x in per_dispatch(path, "FETCH_SIZE").items()
            if sub in name and x >= min_kib}


def src_hash(name: str) -> str:
    with open(os.path.join(HERE, "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cross_check(fetch_csv: str, write_csv: str, mib: int) -> dict:
    """Factors implied by the calibration run's other kernels of known traffic: the
    fill writes mib MiB (reads none), the float32 sum reads mib MiB (writes a few
    bytes).  They should agree with the copy's."""
    n = float(mib << 20)
    out = {}
    for name, sub, counter, expect in (("fill_write", "FillFunctor", "WRITE_SIZE", n),
                                       ("fill_fetch", "FillFunctor", "FETCH_SIZE", 0.0),
                                       ("sum_fetch", "reduce_kernel", "FETCH_SIZE", n),
                                       ("sum_write", "reduce_kernel", "WRITE_SIZE", 0.0),
                                       ("copy_fetch", "copyBuffer", "FETCH_SIZE", n),
                                       ("copy_write", "copyBuffer", "WRITE_SIZE", n)):
        kib, cnt = mean_kib(fetch_csv if counter == "FETCH_SIZE" else write_csv, counter, sub)
        e = dict(counter=counter, kib_per_dispatch=round(kib, 1), dispatches=cnt,
                 expected_bytes=int(expect))
        if expect:
            e["factor"] = round(expect / (kib * 1024.0), 4)
        out[name] = e
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--cross-check":
        ap = argparse.ArgumentParser()
        ap.add_argument("--cross-check", action="store_true")
        ap.add_argument("--calib-fetch", required=True)
        ap.add_argument("--calib-write", required=True)
        ap.add_argument("--calib-mib", type=int, default=256)
        a = ap.parse_args()
        print(json.dumps(cross_check(a.calib_fetch, a.calib_write, a.calib_mib), indent=1))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--calib-fetch", required=True)
    ap.add_argument("--calib-write", required=True)
    ap.add_argument("--calib-mib", type=int, default=256)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--key", required=True)
    ap.add_argument("--workload", required=True, help="the bench.py workload the runs used")
    ap.add_argument("--source", default="k_score.hip")
    ap.add_argument("--min-fetch-kib", type=float, default=None,
                    help="only the dispatches that fetch at least this much (e.g. to leave "
                         "out launches whose work groups all exit at once)")
    ap.add_argument("--json", default=None)
    a = ap.parse_args()
    cb = float(a.calib_mib << 20)
    out = {"workload": a.workload, "source_hash": src_hash(a.source), "kernel_match": a.kernel}
    total = 0.0
    ids = None
    if a.min_fetch_kib is not None:
        ids = ids_with_fetch(a.fetch, a.kernel, a.min_fetch_kib)
        out["min_fetch_kib"] = a.min_fetch_kib
    for name, kpath, cpath, counter in (("fetch", a.fetch, a.calib_fetch, "FETCH_SIZE"),
                                        ("write", a.write, a.calib_write, "WRITE_SIZE")):
        kib, n = mean_kib(kpath, counter, a.kernel, ids)
        ckib, cn = mean_kib(cpath, counter, "copyBuffer")
        factor = cb / (ckib * 1024.0)
        out[name] = dict(counter=counter, kib_per_dispatch=round(kib, 1), dispatches=n,
                         calib_kib_per_copy=round(ckib, 1), calib_copies=cn,
                         factor=round(factor, 4), bytes_per_dispatch=round(kib * 1024 * factor))
        total += kib * 1024 * factor
    out["bytes_per_launch"] = round(total)
    print(json.dumps(out, indent=1))
    if a.json:
        d = json.load(open(a.json)) if os.path.exists(a.json) else {}
        d.setdefault(a.key, {})[a.workload] = out
        with open(a.json, "w") as f:
            json.dump(d, f, indent=1)


if __name__ == "__main__":
    main()
