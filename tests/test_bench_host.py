"""Host-side checks of the benchmark (no GPU): the one-GPU contract, the
algorithmic byte and flop counts its roofline divides by, and that the
committed counter summaries it reads were taken on the GEMM source as it
stands (a stale summary would silently turn `traffic` and `mfma_busy` into
null)."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_counts(bench):
    """Bytes and flops of one launch, written out from the shapes: the
    layer GEMM reads each code once, its 1x128 A scales and 128x128 B
    scales once, and writes bf16 C; each quantizer reads bf16 once and writes
    one byte per element plus its scales."""
    alg = bench.algorithmic()
    M, N, K = bench.LM, bench.LN, bench.LK
    assert (M, N, K) == (16384, 18432, 7168)
    assert alg["gemm_flop"] == 2 * M * N * K
    codes = M * K + N * K
    scales = 4 * (M * (K // 128)) + 4 * ((N // 128) * (K // 128))
    assert alg["gemm_bytes"] == codes + scales + 2 * M * N
    n = bench.DS_ROWS * bench.DS_COLS
    assert alg["quantize_tensor_bytes"] == 3 * n + 4
    assert alg["quantize_dq_bytes"] == 5 * n + 4
    assert alg["dequantize_bytes"] == 3 * n + 4
    assert alg["quantize_1x128_bytes"] == 3 * M * K + 4 * M * (K // 128)
    assert alg["quantize_mx_bytes"] == 3 * M * K + M * K // 32


def test_stream_kinds_proportions(bench):
    """Every streaming yardstick keeps the read:write proportion it is named for."""
    want = {"copy": (1, 1), "bf16_to_codes": (2, 1), "fp32_to_codes": (4, 1), "codes_to_bf16": (1, 2),
            "codes_to_bf16_wide": (1, 2), "bf16_to_codes_and_bf16": (2, 3)}
    assert set(bench.STREAM_KINDS) == set(want)
    for k, (rd, wr) in bench.STREAM_KINDS.items():
        a, b = want[k]
        assert rd * b == wr * a, k


def test_counter_summaries_match_the_gemm_source(bench):
    """The traffic and MFMA summaries under profiles/ record the hash of the
    GEMM source they were taken on; it must be the current one."""
    assert bench.measured_traffic() is not None, "traffic summary taken on other GEMM source"
    busy = bench.counter_field(bench.MFMA_SUMMARY, "mfma_busy", float)
    clock = bench.counter_field(bench.MFMA_SUMMARY, "clock_ghz", float)
    assert busy is not None and 0.0 < busy <= 1.0
    assert clock is not None and 1.0 < clock < 2.5
    # the traffic is a per-launch byte count of the layer GEMM: at least its
    # algorithmic bytes
    assert bench.measured_traffic() >= bench.algorithmic()["gemm_bytes"]
