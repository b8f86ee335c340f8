"""bench.py's host-side arithmetic and contract, checked without a GPU: the
algorithmic byte counts behind every roofline figure, written out term by
term from the operator's inputs and outputs, and the refusal of more than
one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_token_bytes_of_the_4b_geometry():
    # q, k: 16 heads x 128; v, z, y: 32 heads x 128; a, b: 32 each; bf16
    assert bench.TOKEN_BYTES == 2 * (16 * 128 * 2 + 32 * 128 * 3 + 32 * 2) == 32896


def test_operator_bytes_at_T2048():
    state = 32 * 128 * 128 * 4          # one sequence's fp32 state
    params = 4 * (32 + 32 + 128)        # A_log, dt_bias, norm_w
    assert bench.algorithmic_bytes(2048, 16, 32, 128) == 2048 * 32896 + 2 * state + params
    # without the gated norm: no z, no norm_w
    assert bench.algorithmic_bytes(2048, 16, 32, 128, norm=False) == (
        2048 * (32896 - 32 * 128 * 2) + 2 * state + 4 * 64)
    # the roofline time at 8 TB/s
    assert abs(bench.algorithmic_bytes(2048, 16, 32, 128) / 8e12 * 1e6 - 8.9458) < 1e-3


def test_stage_bytes_split_the_operator_bytes():
    sb = bench.stage_bytes(2048, 16, 32, 128)
    T, state = 2048, 32 * 128 * 128 * 4
    assert sb["prep"] == T * 2 * (2 * 16 * 128 + 2 * 32)       # q, k, a, b
    assert sb["chain"] == T * 2 * (32 * 128) + 2 * state      # v, state in/out
    assert sb["out"] == T * 2 * (2 * 32 * 128)                # z, y
    # each operator byte counted once: the parts add up to the operator's
    # algorithmic bytes (less the per-head parameters)
    params = 4 * (32 + 32 + 128)
    assert sum(sb.values()) == bench.algorithmic_bytes(2048, 16, 32, 128) - params
    assert sum(sb.values()) == T * bench.TOKEN_BYTES + 2 * state


def test_git_info_outside_a_checkout_knows_nothing(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.git_info() == (None, None)


def test_tree_hash_covers_the_sources():
    h = bench.tree_sources_sha256()
    assert len(h) == 64 and h == bench.tree_sources_sha256()


def test_flops_of_the_chunked_form():
    # per chunk and key head: K K^T and Q K^T; per chunk and value head: the
    # inverse (C^3/3 multiply-adds), Tb R and MP V', K H, Q H and K^T V'
    C, D, nch = 64, 128, 32
    want = (nch * 16 * 2 * 2 * C * C * D
            + nch * 32 * (C ** 3 / 3) * 2
            + nch * 32 * (2 * 2 * C * C * D + 3 * 2 * C * D * D))
    assert bench.algorithmic_flops(2048, 16, 32, 128) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
