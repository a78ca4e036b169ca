"""The benchmark's host-side arithmetic, on the CPU: the algorithmic byte and
flop counts that every reported fraction of a peak divides by, against the
figures derived by hand from the workloads' shapes (and, for the chunked
scan, against the MFMA count the instruction counters measured), and the
one-GPU guard of bench.py."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_256_sequences():
    """256 sequences x 32 heads x S = 128: the state read and written
    (2 x 512 MiB), q, k, v read and y written (4 x 4 MiB), g and beta."""
    from linear_attention_ssm_recurrence_amd import inputs
    b = _bench().decode_bytes(inputs.WORKLOADS[2])
    assert b["state"] == 2 * 256 * 32 * 128 * 128 * 4 == 1_073_741_824
    assert b["total"] == 1_073_741_824 + 4 * 256 * 32 * 128 * 4 + 2 * 256 * 32 * 4 == 1_090_584_576


def test_block_layer_bytes_64_sequences():
    """One fused bf16 layer at 64 sequences, 16 -> 32 heads, C = 8192, K = 4:
    state 268,435,456 + conv history 12,582,912 + qkv 1,048,576 + z 524,288 +
    out 1,048,576 + conv weights 131,072 + a, b 16,384 + A_log, dt_bias 256 +
    norm weight 512 bytes."""
    per_layer = _bench().block_layer_bytes(64, 32, 16, 128, 4)
    assert per_layer == (268_435_456 + 12_582_912 + 1_048_576 + 524_288 + 1_048_576 + 131_072
                         + 16_384 + 256 + 512) == 283_788_032
    assert 48 * per_layer == 13_621_825_536


def test_chunked_mfma_flops_match_the_counted_instructions():
    """The scan kernel's 8,388,608 MFMAs per launch (256 blocks x 4 waves x
    128 x 64 chunks) and the preparation's 2048 blocks x 704, as the
    instruction counters counted them at 1 x 4096 positions x 32 heads, at
    2048 flop per v_mfma_f32_16x16x4f32."""
    flops = _bench().chunked_mfma_flops(1, 4096, 32)
    assert flops == 2048.0 * (256 * 4 * 128 * 64 + 2048 * 704)


def test_scan_method_flops():
    """The scan workload's own work, 1 sequence x 4096 tokens x 32 heads x
    S = 128 = 2,147,483,648 element-tokens at 7 flop: 1.503e10 flop. The
    chunked form executes 1.34 times as much on the matrix pipes (the
    fraction reported as the chunked scan's roofline uses this count)."""
    b = _bench()
    f = b.scan_method_flops(1, 4096, 32, 128)
    assert f == 7 * 2_147_483_648 == 15_032_385_536
    assert 1.33 < b.chunked_mfma_flops(1, 4096, 32) / f < 1.35


def test_bench_refuses_more_than_one_gpu():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 2
    assert "one GPU" in run.stderr
    assert run.stdout == ""
