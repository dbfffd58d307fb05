"""The work counts behind the benchmark's roofline figures, against brute force.

The roofline's `achieved` divides the algorithmic work of one score-sweep
launch by its time: one d-length dot product (2d flop) per unordered pair
(i, j) with j - i > window, since a pair counts for both i and j ("TwinKV: A
Composable Repair Pass ...", section 3.2, Eq. 2).  The repair figure counts
every position against the K retained columns (section 3.4, Eq. 4).
"""
import itertools

import pytest

import bench


@pytest.mark.parametrize("N,w", [(1, 0), (2, 0), (2, 1), (5, 0), (9, 2), (40, 7), (64, 64), (65, 64), (130, 64)])
def test_algorithmic_gram_flops_counts_unordered_nonlocal_pairs(N, w):
    pairs = sum(1 for i, j in itertools.combinations(range(N), 2) if j - i > w)
    for d, G in ((64, 1), (128, 3)):
        assert bench.algorithmic_gram_flops(N, d, w, G) == G * pairs * 2 * d


def test_restricted_gram_flops():
    assert bench.restricted_gram_flops(32768, 16384, 64, 128) == 128 * 32768 * 16384 * 2 * 64


def test_default_workload_figures():
    # the Llama-3.2-1B shape the benchmark line is quoted on
    alg = bench.algorithmic_gram_flops(32768, 64, 64, 128)
    assert alg == 8761498927104.0
    # both orders of every pair, as the sweep executes them, is a little over twice that
    assert 2.0 * 128 * 32768 * 32768 * 64 / alg == pytest.approx(2.0078, abs=1e-4)
