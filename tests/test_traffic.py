"""Host logic of the traffic summary: calibration by the copy kernel, per
kernel averages and the per-launch bytes of a stage, and the source hash
that keeps stale figures out of the bench report."""

import csv
import json

from jagged_embedding_sparse_amd import traffic

HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
KS = "void fs::(anonymous namespace)::k_short<128, unsigned short>(fs::(anonymous namespace)::RUArgs)"
KL = "void fs::(anonymous namespace)::k_long<128, unsigned short>(fs::(anonymous namespace)::RUArgs)"
KF = "void fs::(anonymous namespace)::k_fix<128, unsigned short>(fs::(anonymous namespace)::RUArgs)"


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HDR)
        for i, (k, v) in enumerate(rows):
            w.writerow([i, k, counter, v])


def test_summary_scales_by_copy_and_sums_a_launch(tmp_path):
    gib_kib = (1 << 30) / 1024
    f, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    # the counter reads half of what is read and all of what is written
    copies = [("__amd_rocclr_copyBuffer", 100.0)] + [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3
    _csv(f, "FETCH_SIZE", copies + [(KS, 1000.0), (KS, 3000.0), (KL, 500.0), (KF, 10.0)])
    _csv(wr, "WRITE_SIZE",
         [(k, v * 2) for k, v in copies] + [(KS, 300.0), (KS, 500.0), (KL, 40.0), (KF, 4.0)])
    res = traffic.summarize(str(f), str(wr), 5, None)
    assert abs(res["calibration"]["fetch_factor"] - 0.5) < 1e-12
    assert abs(res["calibration"]["write_factor"] - 1.0) < 1e-12
    ks = res["kernels"][KS]
    assert ks["short"] == "k_short" and ks["dispatches"] == 2
    assert ks["fetch_bytes"] == 2000.0 * 1024 / 0.5
    st = res["stages"]["update_all"]
    # per launch: k_short's mean plus one k_long and one k_fix dispatch
    assert st["launches"] == 2
    want_f = (4000.0 + 500.0 + 10.0) * 1024 / 0.5 / 2
    want_w = (800.0 + 40.0 + 4.0) * 1024 / 1.0 / 2
    assert abs(st["fetch_bytes_per_launch"] - want_f) < 1e-6
    assert abs(st["write_bytes_per_launch"] - want_w) < 1e-6
    assert st["sources_sha"] == traffic.sources_sha("update_all")


def test_load_traffic_refuses_other_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"stages": {"update_all": {"bytes_per_launch": 123.0,
                                     "sources_sha": traffic.sources_sha("update_all")}}}
    (prof / "traffic_workload9.json").write_text(json.dumps(rec))
    monkeypatch.setattr(traffic, "ROOT", str(tmp_path))
    assert traffic.load_traffic(9, "update_all") == 123.0
    rec["stages"]["update_all"]["sources_sha"] = "0" * 16
    (prof / "traffic_workload9.json").write_text(json.dumps(rec))
    assert traffic.load_traffic(9, "update_all") is None
    assert traffic.load_traffic(8, "update_all") is None


def test_table_lists_kernels_per_step_and_index_total(tmp_path):
    gib_kib = (1 << 30) / 1024
    f, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    copies = [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3
    KH = "fs::(anonymous namespace)::k_heads(unsigned int const*, long const*, int, unsigned int*)"
    # two steps: k_heads reads 1000 KiB per dispatch, writes 10 KiB
    _csv(f, "FETCH_SIZE", copies + [(KS, 1000.0)] * 2 + [(KH, 500.0)] * 2)
    _csv(wr, "WRITE_SIZE", [(k, v * 2) for k, v in copies] + [(KS, 100.0)] * 2 + [(KH, 10.0)] * 2)
    res = traffic.summarize(str(f), str(wr), 5, None)
    txt = traffic.table(res, 2, index_algorithmic=1024.0 * 1000)
    # per step: fetch 500 KiB / 0.5 = 1 MiB, write 10 KiB
    heads = [ln for ln in txt.splitlines() if ln.startswith("k_heads")][0].split()
    assert abs(float(heads[2]) - 1024 * 1000 / 1e6) < 0.006
    assert abs(float(heads[3]) - 10 * 1024 / 1e6) < 0.006
    assert "index kernels" in txt and "1.01x" in txt
