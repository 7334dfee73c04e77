"""Host-side logic of bench.py (no GPU): the tokens-per-round figure against
the closed form of the pages, and the pass-1 kernel a launch's line names."""
import itertools
import sys
from pathlib import Path

import numpy as np
import pytest

sys.path.insert(0, str(Path(__file__).resolve().parents[1]))
import bench  # noqa: E402


def test_closed_form_matches_the_worked_example():
    # alpha = 0.8, gamma = 4: (1 - 0.8^5) / (1 - 0.8) = 3.3616 tokens per round
    # (the study notes' "roughly 3", Speedup math)
    B, g = 1000, 4
    r = bench.closed_form_tokens(np.full(B * g, 0.8), np.full(B, g), np.full(B, 2))
    assert r["closed_form_tokens_per_sequence"] == pytest.approx(3.3616, abs=1e-12)
    assert r["observed_tokens_per_sequence"] == 3.0 and r["sequences"] == B


def test_closed_form_variance_by_enumeration():
    # n + 1 from independent acceptances: mean and variance by enumerating
    # every accept/reject pattern of three positions
    a = np.array([0.9, 0.35, 0.6])
    vals, probs = [], []
    for bits in itertools.product([0, 1], repeat=3):
        p = np.prod([a[j] if bits[j] else 1 - a[j] for j in range(3)])
        n = next((j for j in range(3) if not bits[j]), 3)  # first rejection
        vals.append(n + 1)
        probs.append(p)
    vals, probs = np.array(vals, float), np.array(probs)
    mu = (vals * probs).sum()
    var = (vals * vals * probs).sum() - mu * mu
    r = bench.closed_form_tokens(a, np.array([3]), np.array([1]))
    assert r["closed_form_tokens_per_sequence"] == pytest.approx(mu, rel=1e-12)
    assert r["standard_error"] == pytest.approx(np.sqrt(var), rel=1e-12)


def test_closed_form_greedy_and_failed_sequences():
    # alpha in {0, 1} (greedy): the round's length is determined, no error;
    # failed sequences (n = -1) and NaN rates are left out; gamma = 0 emits 1
    alpha = np.array([1.0, 1.0, 0.0, 1.0, np.nan, 0.5])
    gamma = np.array([4, 0, 1, 1])
    n = np.array([2, 0, 0, -1])
    r = bench.closed_form_tokens(alpha, gamma, n)
    assert r["sequences"] == 2
    assert r["closed_form_tokens_per_sequence"] == pytest.approx((3 + 1) / 2)
    assert r["standard_error"] == 0.0 and r["z"] == 0.0


@pytest.mark.parametrize("vocab,size,gamma,kernel", [
    (1000, 4, [4] * 16, "k1_short_rows"),          # the tiny fp32 workload's rows: 4000 B
    (1024, 4, [4] * 16, "k1_short_rows"),          # exactly one 4 KiB tile
    (1025, 4, [4] * 16, "k1_row_stats"),           # two tiles
    (2048, 2, [3] * 16, "k1_short_rows"),          # one bf16 tile
    (2044, 2, [3] * 16, "k1_row_stats"),           # 4088 B: not a multiple of 16 bytes
    (32128, 2, [5] * 16, "k1_row_stats"),          # the T5-XXL-like rows
    (1000, 4, [1, 2] * 8, "k1_row_stats"),         # ragged, planned inside pass 1
    (1000, 4, [1, 2] * 600, "k1_short_rows"),      # ragged past 1024 sequences: plan launch
])
def test_pass1_kernel_of_a_launch(vocab, size, gamma, kernel):
    assert bench.pass1_kernel(vocab, size, np.array(gamma, np.int32)) == kernel


def test_pass2_bytes_counts_the_selected_rows():
    # gamma 3, V 10, fp32: a residual reads two rows, a bonus one, greedy and
    # failed sequences none
    g = np.array([3, 3, 3, 3, 3, 0], np.int32)
    T = np.array([1.0, 1.0, 0.0, 0.7, 1.0, 1.0], np.float32)
    n = np.array([0, 3, 1, 2, -1, 0], np.int32)
    # seq 0: residual (2 rows); 1: bonus (1); 2: greedy (0); 3: residual (2);
    # 4: failed (0); 5: gamma 0, every draft accepted: bonus (1)
    assert bench.pass2_bytes(10, 4, g, T, n) == (2 + 1 + 2 + 1) * 10 * 4
    assert bench.pass2_bytes(10, 2, g[:0], T[:0], n[:0]) == 0
