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


def test_counter_cross_check_factors(tmp_path):
    # the calibration run's fill and sum give factors beside the copy's: a counter
    # that reports half the bytes read gives 2.0, one that reports them all 1.0
    from sparse_attention_decode_qsa_amd import counters
    mib = 4
    n_kib = (mib << 20) / 1024

    def write_csv(path, counter, rows):
        with open(path, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, name, kib in rows:
                # two instances per dispatch, summed by the reader
                f.write(f"{d},{name},{counter},{kib / 2}\n{d},{name},{counter},{kib / 2}\n")

    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fetch, "FETCH_SIZE", [(1, "copyBuffer", n_kib / 2), (2, "FillFunctor", 0.0),
                                    (3, "reduce_kernel", n_kib / 2)])
    write_csv(write, "WRITE_SIZE", [(1, "copyBuffer", n_kib), (2, "FillFunctor", n_kib),
                                    (3, "reduce_kernel", 0.25)])
    out = counters.cross_check(str(fetch), str(write), mib)
    assert out["copy_fetch"]["factor"] == 2.0 and out["sum_fetch"]["factor"] == 2.0
    assert out["copy_write"]["factor"] == 1.0 and out["fill_write"]["factor"] == 1.0
    assert "factor" not in out["fill_fetch"] and out["fill_fetch"]["kib_per_dispatch"] == 0.0
    assert out["sum_write"]["expected_bytes"] == 0
