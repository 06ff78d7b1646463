"""Pins of the oracle's structured subset (R26) against brute force over
Python sets and its special cases: no stride = sinks plus a recent window,
a window covering the sequence = every row, an empty sequence = no row."""
import numpy as np
import pytest

import oracle as O


def _brute(n, n_sink, n_recent, stride):
    rows = set(range(min(n, n_sink))) | set(range(max(0, n - n_recent), n))
    if stride > 0:
        rows |= set(range(n_sink, n, stride))
    return sorted(rows)


@pytest.mark.parametrize("n_sink,n_recent,stride", [(4, 16, 3), (0, 5, 1), (7, 0, 0), (3, 2, 7), (64, 1024, 4)])
def test_subset_policy_against_brute_force(n_sink, n_recent, stride):
    n_body = [0, 1, 3, 5, 9, 17, 40, 100, 257, 2000]
    got = O.subset_policy(n_body, n_sink, n_recent, stride)
    for n, a in zip(n_body, got):
        assert a.tolist() == _brute(n, n_sink, n_recent, stride), n


def test_subset_policy_special_cases():
    n_body = np.array([0, 10, 50])
    no_stride = O.subset_policy(n_body, 3, 5, 0)
    assert no_stride[2].tolist() == [0, 1, 2, 45, 46, 47, 48, 49]
    assert all(len(a) == 0 for a in O.subset_policy([0], 4, 4, 2))
    everything = O.subset_policy(n_body, 0, 1000, 0)
    assert all(a.tolist() == list(range(n)) for a, n in zip(everything, n_body))
    assert O.subset_policy([20], 0, 0, 1)[0].tolist() == list(range(20))          # stride 1 keeps all
    # sorted and unique, every row < n
    for a, n in zip(O.subset_policy(n_body, 2, 7, 4), n_body):
        assert np.all(np.diff(a) > 0) and (len(a) == 0 or a[-1] < n)
