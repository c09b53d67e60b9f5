"""Host logic of bench.py (no GPU): the algorithmic work it divides by, the
roofline it reports, and the single-GPU contract.

The feature count is derived here from the feature map itself ([OAL] Eq. 5-7:
a constant, the d_h linear features and the d_h (d_h + 1) / 2 products
q_r q_t with r <= t), not taken from bench.py."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

D_H = 64
D = 1 + D_H + D_H * (D_H + 1) // 2      # 2145 features
W = D_H + 1                              # value channels + the all-ones channel


def test_feature_count_matches_the_feature_map():
    assert D == 2145 and bench.D_CANON == D and bench.W == W


@pytest.mark.parametrize("n_q,n_kv,chunk,mflop", [
    (14, 2, 64, 4.579), (14, 2, 128, 4.695), (14, 2, 256, 4.926), (32, 8, 128, 11.687)])
def test_prefill_work_per_token(n_q, n_kv, chunk, mflop):
    """State build 2 D W per KV head, readout 2 D W per query head, and the causal
    triangle: on average (C + 1) / 2 keys per query, each a kappa (d_h MACs) and a
    [v; 1] accumulation (W MACs), 2 flops per MAC."""
    fl = bench.prefill_flops_per_token(n_q, n_kv, chunk)
    assert fl["build"] == 2 * D * W * n_kv
    assert fl["readout"] == 2 * D * W * n_q
    assert fl["intra"] == n_q * 2 * ((chunk + 1) / 2) * (D_H + W)
    assert fl["total"] / 1e6 == pytest.approx(mflop, abs=5e-4)


def test_decode_bytes_per_step():
    """Batch 64, 32 query / 8 KV heads: the fp32 state of 512 units read and
    written once (571.08 MB), bf16 q and y (262,144 B each), bf16 k and v."""
    b = bench.decode_bytes_per_step(64, 32, 8)
    state = 64 * 8 * D * W * 4
    assert state == 285_542_400
    assert b == 2 * state + 2 * (64 * 32 * D_H) * 2 + 2 * 2 * (64 * 8 * D_H)
    assert b == 571_740_160


def test_roofline_uses_the_timed_duration_of_the_dominant_kernel():
    class W3:
        batch, seq_len, n_q_heads, n_kv_heads = 1, 32768, 14, 2
    kt = {"k_expand": {"total_ms": 0.2, "launches": 20, "avg_ms": 0.01},
          "k_state_mfma": {"total_ms": 0.9, "launches": 20, "avg_ms": 0.045},
          "k_readout_mfma": {"total_ms": 4.4, "launches": 20, "avg_ms": 0.22}}
    timed = {"k_readout_mfma": {"total_ms": 5.0, "launches": 20, "avg_ms": 0.25}}
    r = bench.roofline_prefill(kt, timed, W3, 128)
    fl = bench.prefill_flops_per_token(14, 2, 128)
    work = 32768 * (fl["readout"] + fl["intra"])
    assert r["kernel"] == "k_readout_mfma" and r["bound"] == "mfma"
    assert r["work_per_launch"] == work
    assert r["avg_launch_ms"] == pytest.approx(0.25)
    assert r["achieved"] == pytest.approx(work / 0.25e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, rel=1e-3)
    # without a timed measurement the breakdown's duration is used
    r2 = bench.roofline_prefill(kt, {}, W3, 128)
    assert r2["avg_launch_ms"] == pytest.approx(0.22)


def test_more_than_one_gpu_exits_with_a_message():
    env = dict(os.environ, WORLD_SIZE="1")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""
