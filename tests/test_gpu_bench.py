"""bench.py's one-line JSON report: the keys and types the measurement
contract fixes, checked on a short run in a child process (few steps, the
oracle baseline on its bounded sample)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_reports_the_contract_fields():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5",
                          "--no-extra"], cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, out.stdout[-2000:]
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], kind), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5 and d["value"] > 0
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["peak"] > 0 and 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    # Replay statistics, the measured floors and the warm number.
    assert d["replays"] >= 10
    assert d["ms_per_step_p10"] <= d["ms_per_step_median"] <= d["ms_per_step_p90"]
    assert d["copy_peak_GBps"] > 0 and 0 < d["hbm_frac_vs_floor"]
    assert d["warm_us_per_layer"] > 0
    assert r["read_floor_us_same_bytes"] > 0
    mp = d["mfma_peak_measured"]
    for dt in ("bf16", "f16"):
        assert mp[dt]["checked"] is True and 0 < mp[dt]["TFLOPs"] < 1.2 * 2500
    assert d["mfma_frac_layer_vs_measured_bf16"] > 0
    assert 0 < d["hbm_frac_vs_copy_peak"] < 1.5
    pv = d["provenance"]
    assert pv["seed"] == 0 and len(pv["inputs_sha256"]) == 64 and len(pv["sources_sha256"]) == 64


def test_bench_runs_a_grouped_workload():
    # Another workload through the same contract: the grouped path's GEMMs
    # are timed by their own start/end events and the dominant one carries
    # the roofline.
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "batch_m21", "--steps", "8",
                          "--warmup", "2", "--replays", "3", "--no-extra", "--no-cpu-baseline"],
                         cwd=ROOT, capture_output=True, text=True, timeout=150)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, out.stdout[-2000:]
    d = json.loads(lines[0])
    assert d["config"]["path"] == "grouped" and d["config"]["M"] == 21 and d["value"] > 0
    r = d["roofline"]
    assert "grouped_gemm" in r["kernel"] and 0 < r["frac"] < 1 and r["read_floor_us_same_bytes"] > 0
    assert set(r["kernel_us_all"]) == set(r["dispatch_event_us"])
    assert d["cpu_baseline"] is None


def test_measurement_kernels_read_and_copy_every_byte():
    # The streaming-read kernel's per-workgroup XORs combine to the XOR of
    # every word of the buffer, and the copy reproduces the buffer, on a size
    # with a partial last tile.
    import numpy as np
    import torch
    import ctypes
    from mixture_experts_ffn_align_amd import _binding as B
    L = B.bench_lib()
    n = (3 << 20) + 4096 + 16          # bytes: 192 whole 16 KiB tiles and a ragged tail
    host = np.random.default_rng(5).integers(0, 2**32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    grid = ctypes.c_int32(0)
    s = torch.cuda.current_stream().cuda_stream
    want = np.bitwise_xor.reduce(host)
    for unroll in (1, 2, 4, 8, 16):
        sink.zero_()
        assert L.moe_bench_stream_read(src.data_ptr(), n, sink.data_ptr(), sink.numel(), unroll, ctypes.byref(grid),
                                       None, None, s) == 0
        dst = torch.zeros_like(src)
        assert L.moe_bench_copy(src.data_ptr(), dst.data_ptr(), n, unroll, None, None, s) == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink[:grid.value].cpu().numpy().view(np.uint32))
        assert grid.value == -(-n // (256 * unroll * 16)) and got == want, unroll
        assert torch.equal(src, dst), unroll


def test_measurement_mfma_kernel_runs_every_product():
    # With every operand 1.0 each MFMA adds 32 to every accumulator element:
    # each wave's lane 0 reports 8 chains x 32 x iters exactly, on every
    # wave of the grid, for both operand types; the seeded pattern runs too.
    import ctypes
    import torch
    from mixture_experts_ffn_align_amd import _binding as B
    L = B.bench_lib()
    s = torch.cuda.current_stream().cuda_stream
    for fp16 in (0, 1):
        for grid, iters in ((1, 1), (37, 5), (512, 64)):
            sink = torch.full((4 * grid + 4,), -1.0, dtype=torch.float32, device="cuda")
            flops = ctypes.c_double(0.0)
            assert L.moe_bench_mfma(fp16, 0, iters, grid, sink.data_ptr(), ctypes.byref(flops), None, None, s) == 0
            torch.cuda.synchronize()
            assert torch.all(sink[:4 * grid] == 8 * 32 * iters), (fp16, grid, iters)
            assert torch.all(sink[4 * grid:] == -1.0)
            assert flops.value == grid * 4 * iters * 8 * 2 * 16 * 16 * 32
        sink = torch.zeros(4 * 64, dtype=torch.float32, device="cuda")
        assert L.moe_bench_mfma(fp16, 1, 16, 64, sink.data_ptr(), None, None, None, s) == 0
        torch.cuda.synchronize()
        assert torch.all(torch.isfinite(sink)) and torch.all(sink > 8 * 32 * 16)
