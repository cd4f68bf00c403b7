"""The benchmark's readers of the committed rocprofv3 summaries, on the host:
each summary parses, carries the hash of the kernel sources it was taken on,
and a reader returns nothing once that hash no longer matches (a changed
kernel must not be reported with another kernel's counters), nor when a
summary of the bf16 / row-scaled fp8 launches was taken on another call
sequence of the layer (other launches)."""

import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402

READERS = [
    ("gate_up_v3_prefill_traffic.txt", bench.measured_traffic),
    ("gate_up_v3_prefill_fp8_traffic.txt", bench.measured_traffic),
    ("decode_v3_fp8_traffic.txt", bench.measured_traffic),
    ("gemm_mfma_util.txt", bench.measured_mfma_util),
    ("gemm_clock.txt", bench.measured_clock),
]


def _key(path, key):
    for line in path.read_text().splitlines():
        if line.startswith(key):
            return line.split("=", 1)[1].strip()
    return None


def _sha(path):
    return _key(path, "kernel_src_sha")


def _current(path):
    """Taken on the current kernel sources and, but for the fine-grained fp8
    traffic (its launches hold the shared experts), on the current call
    sequence."""
    seq_ok = (path.name == "gate_up_v3_prefill_fp8_traffic.txt"
              or _key(path, "layer_sequence") == bench.LAYER_SEQUENCE)
    return _sha(path) == bench.kernel_source_hash() and seq_ok


@pytest.mark.parametrize("name,reader", READERS, ids=[r[0] for r in READERS])
def test_summary_has_command_and_hash(name, reader):
    path = ROOT / "profiles" / name
    text = path.read_text()
    assert "rocprofv3" in text and "command:" in text
    assert _sha(path) is not None


@pytest.mark.parametrize("name,reader", READERS, ids=[r[0] for r in READERS])
def test_reader_gated_by_source_hash(name, reader, tmp_path):
    path = ROOT / "profiles" / name
    value = reader(str(path))
    if _current(path):
        assert value  # current summary: a number or a non-empty table
    else:
        assert not value
    stale = tmp_path / name
    stale.write_text(path.read_text().replace(_sha(path), "0" * 16))
    assert not reader(str(stale))
    if name != "gate_up_v3_prefill_fp8_traffic.txt" and _current(path):
        other = tmp_path / ("seq_" + name)
        other.write_text(path.read_text().replace(bench.LAYER_SEQUENCE, "another-sequence"))
        assert not reader(str(other))


def test_values_in_physical_range():
    if not _current(ROOT / "profiles" / "gemm_clock.txt"):
        pytest.skip("clock summary taken on other kernel sources or another call sequence")
    clock = bench.measured_clock()
    for name, c in clock.items():
        assert 0.5 < c["ghz"] <= 2.45, name            # engine clock at most the 2.4 GHz peak
        assert 0.0 < c["mfma_busy_pct"] <= 100.0, name
        assert c["bf16_ceiling_TFLOPs"] <= bench.MFMA_BF16_PEAK_TFLOPS * 2.45 / 2.4
    decode = bench.measured_traffic(bench.DECODE_TRAFFIC_FILE)
    if decode:
        assert 7.0e9 < decode < 1.0e10                  # 168 active experts x 44.09 MB, read once


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    base = "// header\nint f(int x) {\n  return x + 1;  /* inc */\n}\n"
    src.write_text(base)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    h0 = bench.kernel_source_hash()
    src.write_text("// other words\n/* a block\n comment */ int f(int x) {\n    return x + 1;\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text(base.replace("x + 1", "x + 2"))
    assert bench.kernel_source_hash() != h0


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    import os
    import subprocess
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, str(ROOT / "bench.py")] + argv, capture_output=True,
                       text=True, env=e, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""
