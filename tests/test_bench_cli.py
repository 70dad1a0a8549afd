"""bench.py's host-side contract, without a GPU: the one-GPU refusal, the algorithmic byte count of the headline
workload, the stale-profile rule for the reported HBM traffic, and the steps per host wait of the chained run."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT,
                             env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
        assert out.returncode == 2, out
        assert "one GPU" in out.stderr and not out.stdout.strip()


def test_algorithmic_bytes_of_the_headline_workload():
    # the weights once (bf16), the LM head once, the final norm, the embedding row, and for every layer the K and V
    # rows of all 8192 positions plus the row written at pos
    w = synth.workload("llama8b-bf16-cap8192")
    m = w.model
    L, d, F, V, hd, nq, nkv = m.n_layers, m.d_model, m.ffn_dim, m.vocab, m.head_dim, m.n_q_heads, m.n_kv_heads
    weights = L * (d * (nq + 2 * nkv) * hd + nq * hd * d + 3 * d * F + 2 * d) + V * d + d
    expect = 2 * weights + 2 * d + L * 2 * w.cap * nkv * hd * 2 + L * 2 * nkv * hd * 2
    assert bench.algorithmic_bytes(w) == expect == 16_083_730_432


def test_traffic_is_withheld_when_the_kernel_sources_changed(monkeypatch):
    real = bench.sources_sha256("decode_step_fused")
    monkeypatch.setattr(bench, "sources_sha256", lambda kind: "0" * 64 if kind == "decode_step_fused" else real)
    assert bench.pmc_traffic("decode_step_fused", "llama8b-bf16-cap8192") is None


def test_chained_run_keeps_several_wall_samples():
    assert bench.steps_per_host_wait(32, 504) == 32      # the default run: 16 waits
    assert bench.steps_per_host_wait(32, 20) == 4        # a short run still gives five wall-time samples
    assert bench.steps_per_host_wait(32, 3) == 1
    assert bench.steps_per_host_wait(0, 504) == 0        # --chain 0: one host pick per step
    for steps in range(1, 200):
        c = bench.steps_per_host_wait(32, steps)
        assert 1 <= c <= 32 and (-(-steps // c) >= 5 or c == 1)
