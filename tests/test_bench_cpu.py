"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the kernel
attribution of each stage, the counter-CSV arithmetic behind the traffic
lines, and the staleness check that turns a changed kernel's stored traffic
into null."""
import csv
import importlib.util
import os
import subprocess
import sys

import pytest

import moe_synth as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_base_names(bench):
    assert bench.kernel_base("void qrmoe::gateup_mfma_kernel<4096, false>(qrmoe::LayerArgs, int, int)") == \
        "gateup_mfma_kernel"
    assert bench.kernel_base("qrmoe::decode_down1_kernel<2048, 1, false, 6>") == "decode_down1_kernel"
    assert bench.kernel_base("__amd_rocclr_copyBuffer") is None


def test_stage_kernels_follow_the_dispatch(bench):
    c = ms.CONFIGS
    assert bench.stage_kernel(c["decode_q8"], "gateup") == "decode_gateup1_kernel"
    assert bench.stage_kernel(c["decode_q8"], "down") == "decode_down1_kernel"
    assert bench.stage_kernel(c["hash_decode"], "gateup") == "gateup_vec_kernel"
    # 32 hash-routed tokens: one wave per token selects, the sort kernel builds the work list
    assert bench.stage_kernel(c["hash_decode"], "select") == "select_kernel"
    assert bench.stage_kernel(c["hash_decode"], "sort") == "sort_kernel"
    small = ms.LayerConfig("small", 4096, 256, 6, 2048, 8)
    assert bench.stage_kernel(small, "select") == "decode_select_kernel" and bench.stage_kernel(small, "sort") is None
    assert bench.stage_kernel(c["prefill"], "gateup") == "gateup_mfma_kernel"
    assert bench.stage_kernel(c["prefill"], "down") == "down_mfma_kernel"
    assert bench.stage_kernel(c["prefill_q2"], "gateup") == "gateup_mfma_kernel"
    # past the decode sizes, up to 224 tokens: quantization and logits in the front kernel
    mid = ms.LayerConfig("mid", 4096, 256, 6, 2048, 100)
    assert bench.stage_kernel(mid, "route") == "decode_front_kernel"
    assert bench.stage_kernel(mid, "logits") is None and bench.stage_kernel(mid, "select") == "select_kernel"
    assert bench.stage_kernel(c["prefill"], "logits") == "logits_tiled_kernel"
    # 2048 tokens x top-6 = 12,288 pairs: the chunked sort
    assert bench.stage_kernel(c["prefill"], "sort") == "sort_scatter_kernel"
    every = set(bench.KERNEL_SOURCES)
    for name in ("decode_q8", "decode_q2", "hash_decode", "prefill", "prefill_q2"):
        for stage in ("route", "quant", "logits", "select", "sort", "gateup", "down", "combine"):
            k = bench.stage_kernel(c[name], stage)
            assert k is None or k in every, (name, stage, k)


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_lines_scale_counters_by_the_copy_calibration(bench, tmp_path, monkeypatch):
    # a 1 GiB copy whose counters read half (fetch) and all (write) of its bytes
    gib_kib = (1 << 30) / 1024
    _pmc_csv(tmp_path / "cf.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3)
    _pmc_csv(tmp_path / "cw.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib)] * 3)
    k = "void qrmoe::gateup_mfma_kernel<4096, false>(qrmoe::LayerArgs)"
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(k, 1000.0), (k, 3000.0), ("other_kernel", 5.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(k, 10.0), (k, 30.0)])
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))

    class Args:
        config = "prefill"
        pmc_fetch, pmc_write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
        copy_fetch, copy_write = str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv")

    bench.traffic_from(Args)
    lines = [l.split() for l in open(out) if not l.startswith("#")]
    assert len(lines) == 1 and lines[0][:2] == ["prefill", "gateup_mfma_kernel"]
    kv = dict(x.split("=", 1) for x in lines[0][2:])
    # mean fetch 2000 KiB x factor 2, mean write 20 KiB x factor 1
    assert float(kv["fetch_factor"]) == pytest.approx(2.0) and float(kv["write_factor"]) == pytest.approx(1.0)
    assert float(kv["bytes"]) == pytest.approx(2000 * 1024 * 2 + 20 * 1024)
    assert kv["src"] == bench.source_hash("gateup_mfma_kernel")
    cfg = ms.CONFIGS["prefill"]
    assert bench.stored_traffic(cfg, "gateup_mfma_kernel") == pytest.approx(2000 * 1024 * 2 + 20 * 1024)
    # a line taken from other kernel sources is stale: no traffic is reported
    text = open(out).read().replace("src=" + kv["src"], "src=0000000000000000")
    out.write_text(text)
    assert bench.stored_traffic(cfg, "gateup_mfma_kernel") is None
