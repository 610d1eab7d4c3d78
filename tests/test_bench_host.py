"""Host logic of bench.py that needs no GPU: counter-measured HBM traffic is used
only for the workload and kernel source it was taken on."""
import json

import bench
import synth


def test_stored_traffic_names_its_workload():
    d = json.load(open(bench.TRAFFIC_FILE))
    assert d
    for kernel, per_wl in d.items():
        for wl, e in per_wl.items():
            assert wl in synth.WORKLOADS, (kernel, wl)
            assert synth.WORKLOADS[wl].name == wl
            assert e["workload"] == wl
            # the launch total is the two counters' sum (each rounded on its own)
            assert abs(e["bytes_per_launch"] - e["fetch"]["bytes_per_dispatch"]
                       - e["write"]["bytes_per_dispatch"]) <= 1


def test_traffic_only_for_its_workload_and_source(tmp_path, monkeypatch):
    h = bench.src_hash("k_score.hip")
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"score_decode_kernel": {
        "decode_255181": {"workload": "decode_255181", "source_hash": h, "bytes_per_launch": 123},
        "decode_126253": {"workload": "decode_126253", "source_hash": "0" * 16,
                          "bytes_per_launch": 456}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("score_decode_kernel", "k_score.hip", "decode_255181") == 123
    # another workload's figure is never borrowed
    assert bench.traffic_for("score_decode_kernel", "k_score.hip", "decode_61789") is None
    # a figure taken on another version of the kernel source is not used
    assert bench.traffic_for("score_decode_kernel", "k_score.hip", "decode_126253") is None
    assert bench.traffic_for("score_prefill_kernel", "k_score_mfma.hip", "decode_255181") is None
