"""bench.py's output contract: one JSON line with the fields the benchmark
driver reads, the roofline and CPU-baseline objects, and a refusal of more
than one GPU; plus the host-side pieces it is built from."""
import json
import os
import subprocess
import sys

import pytest

import bench
from tests.conftest import ROOT
from whisper_audio_encoder_amd import wenc
from whisper_audio_encoder_amd.configs import CONFIGS


def _run_bench(args, env_extra=None, timeout=240):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], None), ([], {"WORLD_SIZE": "2"})):
        r = _run_bench(args, env, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", list(CONFIGS))
def test_site_work_covers_every_profiled_site(name):
    cfg = CONFIGS[name]
    work = bench.site_work(cfg, cfg.batch)
    assert set(wenc.SITES) <= set(work)
    for site, (kind, amount) in work.items():
        assert kind in ("mfma", "hbm", "alu") and amount > 0, site
    # the MFMA sites add up to the metric's FLOPs per window times the batch
    per_batch = sum(work[s][1] for s in ("conv1", "conv2")) + cfg.n_layer * sum(
        work[s][1] for s in ("qkv", "attn", "oproj", "fc1", "fc2"))
    assert per_batch == pytest.approx(cfg.flops_per_window() * cfg.batch, rel=1e-12)


def test_measured_traffic_requires_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("c4", "fc1") is None  # no summary
    rec = {"site": "fc1", "workload": "c4", "kernel_source_sha256": bench.kernel_source_hash("fc1"),
           "hbm_bytes_per_launch": 123.0}
    (tmp_path / "traffic_fc1_c4.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("c4", "fc1") == 123.0
    rec["kernel_source_sha256"] = "0" * 64  # taken on other kernel sources
    (tmp_path / "traffic_fc1_c4.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("c4", "fc1") is None


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_bench_json_line():
    """A short run at whisper-tiny shapes, with the frontend, two decoder
    layers of cross-attention and the oracle baseline."""
    r = _run_bench(["--workload", "c0", "--steps", "3", "--warmup", "2", "--frontend", "--cross", "2"])
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["vs_baseline"] is None
    assert d["value"] == pytest.approx(CONFIGS["c0"].batch / (d["ms_per_step"] * 1e-3), rel=1e-9)
    assert "c0" in d["config"]["workload"]
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and roof["unit"] in ("TFLOP/s", "GB/s")
    assert roof["achieved"] > 0 and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert roof["kernel"] in wenc.SITES
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert d["cross_kv"]["n_dec_layer"] == 2 and d["cross_kv"]["decode_step_argmax"]["us_per_call"] > 0
    assert d["log_mel"]
    for part in (d, d["graph_replay"]):
        pc = part["per_call_ms"]
        assert 0 < pc["min"] <= pc["median"] and pc["calls"] >= 3


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_bench_nested_workload_record():
    """--also adds a nested record per extra workload on the same line, with
    its own throughput, roofline and CPU baseline."""
    r = _run_bench(["--workload", "c1", "--also", "c0", "--steps", "3", "--warmup", "2"])
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert "c1" in d["config"]["workload"]
    sub = d["c0"]
    assert "c0" in sub["config"]["workload"] and sub["steps"] == 3 and sub["warmup"] == 2
    assert sub["value"] == pytest.approx(CONFIGS["c0"].batch / (sub["ms_per_step"] * 1e-3), rel=1e-9)
    assert sub["roofline"]["achieved"] > 0 and sub["roofline"]["kernel"] in wenc.SITES
    assert sub["cpu_baseline"]["kind"] == "oracle" and sub["cpu_baseline"]["value"] > 0
