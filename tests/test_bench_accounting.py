"""The benchmark's bookkeeping, checked on the CPU.

The roofline figures the benchmark prints divide algorithmic work by
measured time, so the work counts are pinned here to values worked out by
hand for the Llama-style 7B shape (32 layers, d 4096, 32 query / 8 KV heads
of 128, SwiGLU 14336, vocab 32000, bf16):

* bytes of one splice forward = every weight once + the K/V cache of
  L + N positions + the span's embeddings, mask words and outputs;
* FLOPs = 2 per weight per row + 4 * Hq * hd * (N * L + N (N + 1) / 2) for
  causal attention over the cache and the span;
* the attention kernel's share at N = 512, L = 16384: 4 * 32 * 128 *
  (512 * 16384 + 512 * 513 / 2) = 139 590 631 424 FLOPs.

It also checks that a request for more than one GPU is refused with a
message instead of running.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

S = synth.LLAMA_7B


@pytest.mark.parametrize("N,gbytes,gflops", [
    (1, 16.37, 22.8),
    (16, 16.37, 365.0),
    (128, 16.39, 2924.0),
    (512, 16.44, 11748.0),
])
def test_forward_work_7b(N, gbytes, gflops):
    b, f = bench.forward_work(S, N, 16384)
    assert abs(b / 1e9 - gbytes) < 0.01
    assert abs(f / 1e9 - gflops) / gflops < 1e-3


def test_weight_bytes_7b():
    # 32 layers x (QKV 6144 x 4096 + O 4096 x 4096 + gate/up 28672 x 4096 +
    # down 4096 x 14336) + LM head 32000 x 4096, two bytes each
    per_layer = 6144 * 4096 + 4096 * 4096 + 28672 * 4096 + 4096 * 14336
    p_lin = 32 * per_layer + 32000 * 4096
    assert p_lin == 7_110_393_856
    b0, _ = bench.forward_work(S, 1, 0)
    # at L = 0 and N = 1: weights, norm gains, one embedding row, one K/V
    # position per layer, the mask row and the outputs
    kv = 32 * 2 * 8 * 128 * 2
    assert b0 - 2 * p_lin - kv == pytest.approx(2 * 4096 * 65 + 2 * 4096 + 4 * 1000 + 8, abs=64)


def test_attention_family_flops_7b():
    _, f = bench.family_work(S, "attention", 512, 16384)
    assert f == 139_590_631_424


def test_projection_family_flops_7b():
    # 2 x rows x weight elements per launch
    assert bench.family_work(S, "gemm_gate_up", 512, 16384)[1] == 2 * 512 * 28672 * 4096
    assert bench.family_work(S, "gemm_down", 512, 16384)[1] == 2 * 512 * 4096 * 14336
    assert bench.family_work(S, "gemm_qkv", 512, 16384)[1] == 2 * 512 * 6144 * 4096
    assert bench.family_work(S, "gemm_o", 512, 16384)[1] == 2 * 512 * 4096 * 4096
    assert bench.family_work(S, "gemm_lm_head", 512, 16384)[1] == 2 * 512 * 32000 * 4096


def test_lm_head_bytes_carry_the_mask_and_no_logits():
    """The LM head takes the masked argmax in its epilogue: per launch it
    reads the 32000 x 4096 bf16 head, the 512 activation rows and 512 mask
    rows of 1000 words, and writes no logits (262 MB of weights, 4 KB of
    activations per row, 4000 bytes of mask per row)."""
    b, _ = bench.family_work(S, "gemm_lm_head", 512, 16384)
    assert b == 262_144_000 + 4_194_304 + 2_048_000


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
