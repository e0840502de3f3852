"""Host logic of bench.py (no GPU): the work and byte counts behind the reported rates,
the shader-clock parser, and the single-GPU guard.

The counts are pinned to closed forms worked out by hand: 4*D FLOPs per in-window
(query, key) pair and branch (2 multiply-adds per element of Q K^T and of P V), and
L(2w+1) - w(w+1) in-window pairs per head for a symmetric window of half-width w
(each of the w rows at either end loses 1, 2, ..., w keys past the sequence ends).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rope_attention_core_amd import synth  # noqa: E402


def _brute_pairs(L, w):
    return sum(1 for i in range(L) for j in range(L) if w < 0 or abs(i - j) <= w)


@pytest.mark.parametrize("L,w", [(1, -1), (7, -1), (7, 0), (7, 2), (7, 6), (7, 50), (64, 17), (100, 33)])
def test_pairs_per_head_match_brute_force(L, w):
    cfg = synth.config("tiny", B=1, H=1, L=L, window=w)
    assert bench.pairs(cfg) == _brute_pairs(L, w)


def test_long_latent_work():
    cfg = synth.config("dit_long")
    assert bench.pairs(cfg) == 2 * 24 * 4096 * 4096
    assert bench.flops(cfg) == 4 * 64 * 2 * 24 * 4096 ** 2          # 206.16 GFLOP
    assert abs(bench.flops(cfg) / 1e9 - 206.158) < 1e-3
    assert bench.exps(cfg) == 2 * 24 * 4096 ** 2


def test_windowed_differential_work():
    cfg = synth.config("samel_swa")                                  # L 8192, w 256, two branches
    per_head = 8192 * 513 - 256 * 257
    assert per_head == 4136704
    assert bench.pairs(cfg) == 16 * per_head
    assert bench.flops(cfg) == 4 * 64 * 16 * per_head * 2
    assert bench.exps(cfg) == 2 * 16 * per_head


def test_compulsory_bytes():
    cfg = synth.config("dit_long")
    n = 2 * 24 * 4096 * 64
    # q, k, v bf16 read once, fp32 out written once, the fp32 cos and sin tables read once
    assert bench.compulsory_bytes(cfg) == 3 * 2 * n + 4 * n + 2 * 4096 * 32 * 4
    d = synth.config("samel_swa")
    m = 16 * 8192 * 64
    assert bench.compulsory_bytes(d) == 4 * 2 * m + 2 * m + 4 * m + 2 * 8192 * 32 * 4


@pytest.mark.parametrize("text,want", [
    ("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 94.0),
    ("0: 500Mhz\n1: 2400Mhz *\n", 2400.0),
    ("0: 500Mhz\nS: 2105Mhz *\n1: 2400Mhz\n", 2105.0),
    ("0: 500Mhz\n1: 2400Mhz\n", None),
])
def test_shader_clock_parser(tmp_path, text, want):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    assert bench.read_sclk_mhz(str(p)) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
