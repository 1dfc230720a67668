"""bsga_redistribute (host-side head-wise budget redistribution) against the
oracle's exact-rational solution of the same definition."""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bsga_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "budget_worked.json")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_global_bsga_amd import bsga
    return bsga


def test_redistribute_worked_cases(lib):
    for c in json.load(open(GOLDEN))["cases"]:
        got = lib.redistribute(c["weights"], c["mean_rho"], c["rho_min"], c["rho_max"])
        want = [float(Fraction(x)) for x in c["rho"]]
        assert np.allclose(got, want, rtol=0, atol=1e-14), (c["note"], got)


def test_redistribute_matches_oracle(lib):
    rng = np.random.default_rng(2024)
    for trial in range(300):
        H = int(rng.integers(1, 40))
        w = np.exp(rng.normal(0.0, 2.0, size=H))
        if trial % 5 == 0:
            w[: H // 2] = w[0]  # exact ties
        lo_r, hi_r = sorted(rng.uniform(0.0, 1.0, size=2))
        if trial % 7 == 0:
            lo_r, hi_r = 0.5, 0.95
        mean = float(rng.uniform(lo_r, hi_r))
        got = np.array(lib.redistribute(w.tolist(), mean, lo_r, hi_r))
        want = np.array(O.redistribute_budget(w, mean, lo_r, hi_r))
        assert np.allclose(got, want, rtol=0, atol=1e-12), (trial, np.abs(got - want).max())
        # the integer budgets bsga_select derives agree as well
        for B in (16, 343, 2140):
            assert [lib.keep_count(B, r) for r in got] == [O.keep_count(B, r) for r in want]


def test_redistribute_edge_bounds(lib):
    w = [1.0, 2.0, 5.0]
    assert lib.redistribute(w, 0.6, 0.6, 0.6) == [0.6, 0.6, 0.6]
    assert np.allclose(lib.redistribute(w, 0.9, 0.5, 0.9), [0.9, 0.9, 0.9])  # all at the sparse bound
    assert np.allclose(lib.redistribute(w, 0.5, 0.5, 0.9), [0.5, 0.5, 0.5])  # all at the dense bound


@pytest.mark.parametrize("args", [
    ([1.0, 0.0], 0.5, 0.1, 0.9),            # weight not positive
    ([1.0, float("nan")], 0.5, 0.1, 0.9),   # not finite
    ([1.0, float("inf")], 0.5, 0.1, 0.9),
    ([1.0, 2.0], 0.05, 0.1, 0.9),           # mean below rho_min
    ([1.0, 2.0], 0.5, 0.6, 0.4),            # bounds out of order
    ([1.0, 2.0], 0.5, -0.1, 0.9),
    ([1.0, 2.0], 0.5, 0.1, 1.1),
    ([], 0.5, 0.1, 0.9),                    # no heads
    ([1.0] * 257, 0.5, 0.1, 0.9),           # more than the per-head table holds
])
def test_redistribute_rejects_bad_arguments(lib, args):
    with pytest.raises(lib.BsgaError):
        lib.redistribute(*args)
