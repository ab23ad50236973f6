"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the rocprofv3
summaries, the traffic figure's tie to the kernel sources, the host record
of the CPU baseline and the algorithmic byte count of a decode step."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr or "single MI355X" in p.stderr


def test_summarize_kernel_stats(tmp_path, capsys):
    d = tmp_path / "trace"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void coli::(anonymous namespace)::gateup_stream_kernel<3, 2, 0, coli::(anonymous '
        'namespace)::CodecI4>(coli::Layer, coli_moe_route)","12","278280","23190.0","61.5",'
        '"22800.0","23900.0","0"\n')
    bench.summarize_rocprof(str(d))
    out = capsys.readouterr().out
    assert "| `gateup_stream_kernel<3, 2, 0, CodecI4>` | 12 | 23.19 | 22.80 | 23.90 | 61.5% |" in out


def test_summarize_counters(tmp_path, capsys):
    d = tmp_path / "pmc"
    d.mkdir()
    rows = ['"Kernel_Name","Counter_Name","Counter_Value"']
    for v in (100.0, 300.0):
        rows.append('"void coli::(anonymous namespace)::single_kernel<4>(float const*)",'
                    '"FETCH_SIZE","%s"' % v)
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(str(d))
    out = capsys.readouterr().out
    assert "| `single_kernel<4>` | 2 | FETCH_SIZE | 200.0 |" in out


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    text = open(bench.TRAFFIC_PROFILE).read()
    recorded = text.split("kernel source digest: `")[1][:16]
    monkeypatch.setattr(bench, "kernel_digest", lambda: recorded)
    val = bench.measured_traffic()
    assert isinstance(val, int) and val > 0
    monkeypatch.setattr(bench, "kernel_digest", lambda: "0" * 16)
    assert bench.measured_traffic() is None


def test_kernel_digest_covers_the_decode_sources():
    d = bench.kernel_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f


def test_cpu_host_record():
    h = bench.cpu_host()
    assert h["nproc"] == os.cpu_count()
    json.dumps(h)


def test_union_bytes_counts_distinct_experts_once():
    spec = synth.LayerSpec(128, 64, 8, 1, 2, sigmoid=True, renorm=True)
    # two layers: token rows choosing {7, 6} and {1, 0}; 2 tokens sharing {7, 6}
    lg1 = torch.tensor([[0, 0, 0, 0, 0, 0, 5, 9.0]])
    lg2 = torch.tensor([[9.0, 5, 0, 0, 0, 0, 0, 0], [9.0, 5, 0, 0, 0, 0, 0, 0]])
    per_expert = spec.expert_total_bytes
    assert bench.union_bytes(spec, [lg1], 2) == 3 * per_expert  # 2 routed + shared
    assert bench.union_bytes(spec, [lg1, lg2], 2) == 6 * per_expert
