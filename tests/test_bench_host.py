"""Host-side pieces of the benchmark (no GPU): the algorithmic work that the
roofline figures divide by, the phase-record summary, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from generative_recommender_sequence_amd import hstu  # noqa: E402


def _pairs_brute(c, t, T):
    """Visible (query, key) pairs of one user by enumeration of the mask:
    a history query at position i sees keys 0..i; a candidate (the last T
    positions) sees the history and itself."""
    L = c + t
    hist = L - T
    n = 0
    for i in range(c, L):
        for j in range(L):
            if i < hist:
                n += j <= i
            else:
                n += j < hist or j == i
    return n


def test_user_pairs_matches_the_mask():
    for c in range(0, 13):
        for t in range(0, 13):
            for T in range(0, t + 1):
                assert bench.user_pairs(c, t, T) == _pairs_brute(c, t, T), (c, t, T)


def test_attention_work_formulas():
    H, dh = 4, 128
    cached, new, T = [100, 0, 7], [64, 300, 0], [64, 20, 0]
    pairs = sum(_pairs_brute(c, t, k) for c, t, k in zip(cached, new, T))
    assert bench.attention_flops(cached, new, T, H, dh) == 4.0 * dh * H * pairs
    # K and V of every key of users with new tokens (bf16), the queries once
    # (bf16) and the fp32 output once; the user without new tokens reads nothing
    kv_rows = (100 + 64) + (0 + 300)
    assert bench.attention_bytes(cached, new, H, dh) == kv_rows * H * dh * 2 * 2 + 364 * H * dh * (2 + 4)


def test_roofline_fractions():
    r = bench.mfma_roof(2.5e9, 1.0, 2000.0)  # 2.5 GFLOP in 1 us = 2.5 PFLOP/s
    assert r["frac"] == 1.0 and r["frac_of_achievable"] == 1.25
    h = bench.hbm_roof(8e3, 1.0, None)  # 8 kB in 1 us = 8 GB/s
    assert h["achieved"] == 8.0 and "achievable_peak" not in h


def _records(rows):
    a = np.zeros(len(rows), dtype=hstu.ATTN_STAMP_DTYPE)
    for k, (start, setup, loop, end, xcc, cu, tiles) in enumerate(rows):
        a[k] = (start, setup, loop, end, cu << 8, xcc, k, tiles)
    return a


def test_summarize_phases():
    # two CUs on two XCDs; times in 10 ns ticks
    a = _records([(1000, 1400, 2400, 2500, 0, 3, 5),    # 4 us set-up, 10 us loop over 5 tiles, 1 us write
                  (1000, 1200, 1600, 1700, 0, 3, 2),
                  (1100, 1300, 2300, 2600, 1, 7, 10),
                  (0, 0, 0, 0, 0, 0, 0)])               # a padding block writes nothing
    s = bench.summarize_phases(a)
    assert s["blocks"] == 3 and s["cus_used"] == 2
    assert s["span_us"] == 16.0                          # 1000 .. 2600 ticks
    assert s["setup_us"]["max"] == 4.0 and s["write_us"]["max"] == 3.0
    assert s["tile_loop_us_per_tile"]["max"] == 2.0      # 10 us / 5 tiles and 4 us / 2 tiles
    assert s["xcd_last_end_us"] == {0: 15.0, 1: 16.0}
    assert s["busy_share"] == round((15 + 7 + 15) / (2 * 2 * 16), 3)
    assert bench.summarize_phases(_records([(0, 0, 0, 0, 0, 0, 0)])) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
