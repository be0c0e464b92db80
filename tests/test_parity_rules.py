"""CPU checks of the comparison rules the GPU parity tests apply.

The tie band of ``tests/parity.py`` claims that any GPU whose column masses
are each within the mass tolerance of the oracle's keeps exactly the
oracle's top-k outside the band.  Here that claim is tried directly: random
pools with near-ties at the boundary, masses perturbed anywhere inside the
tolerance (including both extremes), ranked with the budget's rule (larger
first, lower index on ties), must agree with the oracle's kept set on every
candidate outside the band.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import parity as P  # noqa: E402


def topk_flags(m, k):
    flags = np.zeros(len(m), bool)
    flags[np.lexsort((np.arange(len(m)), -m))[:k]] = True
    return flags


@pytest.mark.parametrize("rtol", [2e-3, 1e-4])
def test_tie_band_covers_every_tolerated_perturbation(rtol):
    rng = np.random.default_rng(5)
    opened = 0
    for trial in range(400):
        n = int(rng.integers(2, 60))
        k = int(rng.integers(1, n))
        m = rng.random(n) * rng.choice([1e-4, 1e-2, 1.0, 30.0])
        # Put a cluster of near-equal masses at the boundary in most trials.
        if trial % 4:
            base = np.sort(m)[::-1][k - 1]
            idx = rng.choice(n, size=min(n, int(rng.integers(2, 8))), replace=False)
            m[idx] = base * (1 + rtol * rng.uniform(-3, 3, size=len(idx)))
        if trial % 7 == 0:
            m[rng.choice(n, size=2, replace=False)] = m[0]  # exact ties
        band = P.tie_band(m, k, rtol)
        opened += bool(band.any())
        ref = topk_flags(m, k)
        t = np.maximum(rtol * np.abs(m), 1e-6)
        for _ in range(40):
            u = rng.choice([-1.0, 1.0, 0.0, 0.5, -0.5], size=n) if _ % 2 else rng.uniform(-1, 1, size=n)
            g = m + u * t
            got = topk_flags(g, k)
            assert np.array_equal(got[~band], ref[~band]), (trial, m, k)
    assert opened > 50  # the trials do exercise open bands


def test_tie_band_is_empty_for_clear_gaps_and_edges():
    m = np.array([5.0, 4.0, 3.0, 2.0, 1.0])
    for k in range(6):
        assert not P.tie_band(m, k, 2e-3).any()
    m = np.array([1.0, 1.0, 0.5])
    assert P.tie_band(m, 1, 2e-3).tolist() == [True, True, False]
    m = np.array([1.0, -np.inf, -np.inf])
    assert not P.tie_band(m, 2, 2e-3).any()
    # A gap just above 2 tau leaves no candidate in the band.
    tau = 2e-3 * 1.0 / (1 - 4e-3)
    m = np.array([1.0, 1.0 - 2.01 * tau, 0.1])
    assert not P.tie_band(m, 1, 2e-3).any()
    m = np.array([1.0, 1.0 - 1.99 * tau, 0.1])
    assert P.tie_band(m, 1, 2e-3).tolist() == [True, True, False]
