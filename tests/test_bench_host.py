"""Host-side checks of bench.py that need no GPU: the workload tables, the
roofline arithmetic, the guard on the stored traffic figure, and the refusal
of more than one GPU."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_tables_have_unique_names_and_positive_bytes():
    step, extra = bench.kernel_table(), bench.extra_table()
    names = [r[0] for r in step + extra]
    assert len(names) == len(set(names))
    for name, nbytes, flops, kind in step + extra:
        assert nbytes > 0 and flops >= 0 and kind in ("hbm", "fp8", "fp16"), name
        if kind != "hbm":
            assert flops > 0, name


def test_decode_step_bytes():
    # the KV INT8 quantizer moves x (fp32), its codes and one scale per token
    row = {r[0]: r for r in bench.kernel_table()}["kv_int8_quant"]
    assert row[1] == bench.KV_T * bench.KV_D * 5 + bench.KV_T * 4
    # the attention call reads both caches once (codes and scales) plus q and out
    a = {r[0]: r for r in bench.extra_table()}[f"attn_decode_int8_T{bench.ATTN_T}"]
    rows = bench.ATTN_T * bench.ATTN_HKV
    assert a[1] == 2 * rows * (bench.ATTN_D + 4) + 2 * bench.ATTN_HQ * bench.ATTN_D * 4


def test_roofline_picks_the_binding_roof():
    # 1 GB in 1 ms: 1 TB/s of 8 -> HBM-bound, frac 0.125
    r = bench.roofline_for("x", 10**9, 0, "hbm", 1e-3)
    assert r["bound"] == "hbm" and r["achieved"] == 1000.0 and r["frac"] == 0.125
    # 1 MB and 1e13 flop in 10 ms: far above the FP8 ridge -> MFMA-bound
    r = bench.roofline_for("y", 10**6, 10**13, "fp8", 1e-2)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["achieved"] == 1000.0
    assert r["frac"] == round(1000.0 / bench.FP8_PEAK_TFLOPS, 4)


def test_stored_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    # the figure is reported only while every listed source hashes (comments
    # aside) to the digest it was measured on
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() { int a = 1; }\n")
    digest = bench.code_digest(src)
    monkeypatch.setattr(bench, "TRAFFIC", {"kern": {"bytes": 1234, "sources": {str(src): digest}}})
    assert bench.measured_traffic("kern") == 1234
    assert bench.measured_traffic("other") is None
    src.write_text("__global__ void k() { int a = 1; }  // a comment\n/* and another */\n")
    assert bench.code_digest(src) == digest and bench.measured_traffic("kern") == 1234
    src.write_text("__global__ void k() { int a = 2; }\n")
    assert bench.measured_traffic("kern") is None


def test_stored_traffic_digests_name_existing_sources():
    for entry in bench.TRAFFIC.values():
        assert entry["bytes"] > 0
        for src in entry["sources"]:
            assert (ROOT / src).exists(), src


def test_cold_plan_spans_the_rotation():
    # a 64.6 MB working set needs 9 copies for 512 MiB, launches a multiple of them
    copies, launches = bench.cold_plan(64_616_448, 100)
    assert copies == 9 and launches % copies == 0 and launches >= 100
    assert copies * 64_616_448 >= bench.COLD_BYTES
    # a tiny working set: as many copies as allowed, one pass
    copies, launches = bench.cold_plan(12_292, 100)
    assert copies == bench.MAX_COPIES and launches == copies
    # every kernel of the step and beside it gets a plan covering 512 MiB or MAX_COPIES copies
    for name, nbytes, _, _ in bench.kernel_table() + bench.extra_table():
        c, n = bench.cold_plan(nbytes, 100)
        assert c * nbytes >= bench.COLD_BYTES or c == bench.MAX_COPIES, name


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    p = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr
