"""Host-side checks of bench.py (no GPU): the algorithmic byte counts its
roofline divides by, counted here tensor by tensor from the layouts, the
one-GPU guard, and the traffic records' key."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_bytes_of_the_headline_workload():
    # B=1, T=8192, H=32, D=128 bf16: q, k, v read and o written (8192 x 32 x
    # 128 x 2 B = 64 MiB each), g read (fp32, 1 MiB), the final state written
    # (32 x 128 x 128 fp32 = 2 MiB); no initial state.
    mib = 1 << 20
    assert bench.prefill_bytes(1, 8192, 32, 128, 128) == 4 * 64 * mib + 1 * mib + 2 * mib
    # An initial state adds one more read of the same size.
    assert (bench.prefill_bytes(1, 8192, 32, 128, 128, with_s0=True)
            - bench.prefill_bytes(1, 8192, 32, 128, 128)) == 2 * mib


def test_prefill_bytes_fp32_and_odd_sizes():
    # fp32 elements, Dk != Dv: per token and head 2 Dk + 2 Dv elements of 4 B
    # plus the 4-byte gate; one state of Dk x Dv fp32 per (sequence, head).
    B, T, H, Dk, Dv = 3, 100, 5, 64, 128
    tok = B * T * H * ((2 * Dk + 2 * Dv) * 4 + 4)
    assert bench.prefill_bytes(B, T, H, Dk, Dv, elem=4) == tok + B * H * Dk * Dv * 4


def test_decode_bytes_of_the_batched_decode_workload():
    # 256 rows x 32 heads: each (row, head) reads and writes its 128 x 128 fp32
    # state (64 KiB each way), reads q, k, v (256 B each in bf16) and g (4 B),
    # and writes o (256 B): 1,082,163,200 B per step.
    per = 2 * 65536 + 3 * 256 + 4 + 256
    assert bench.decode_bytes(256, 32, 128, 128) == 256 * 32 * per == 1082163200
    # A bf16 pool halves the state traffic only.
    assert (bench.decode_bytes(256, 32, 128, 128)
            - bench.decode_bytes(256, 32, 128, 128, state_elem=2)) == 256 * 32 * 2 * 32768


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_records_key_on_the_kernel_sources():
    # Each workload's record is keyed by a hash of the sources its kernels are
    # built from; workloads with different kernels get different keys.
    a = bench.kernel_source_hash(bench.PREFILL)
    assert a == bench.kernel_source_hash(bench.PREFILL)
    assert a != bench.kernel_source_hash(bench.DECODE)
