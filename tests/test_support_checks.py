"""The support comparison the GPU parity tests use, checked on the CPU: a list
that breaks the selection rule is rejected even when every one of its
differences from the oracle lies inside the tie band, and a list that only
swaps exactly tied candidates is accepted."""

import numpy as np
import pytest

import oracle as O
from tests import _support as S


def _boundary_row(seed, p, n=3000, n_near=6):
    """Scores whose top-p threshold sits in a cluster of near-equal scores
    (within 1e-5 of each other), so the tie band holds several candidates on
    both sides of the boundary."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * 2.0
    core = O.select_topp(x, p)
    tau = x[core].min()
    near = np.argsort(np.abs(x - tau))[:n_near]
    x[near] = tau + rng.uniform(-1e-5, 1e-5, n_near)
    core = O.select_topp(x, p)
    return x, core


def _ranked(x, S_):
    order = O.candidate_order(x)
    rank = np.empty(len(x), dtype=np.int64)
    rank[order] = np.arange(len(x))
    return sorted(S_, key=lambda j: rank[j]), order


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_support_passes(seed):
    p = 0.9
    x, core = _boundary_row(seed, p)
    assert S.check_support(core, x, core, L=len(x), p=p) == 0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topp_dropping_a_band_member_fails(seed):
    p = 0.9
    x, core = _boundary_row(seed, p)
    ranked, _ = _ranked(x, core)
    P = O.softmax_mass(x)
    short = np.array(sorted(ranked[:-1]))
    assert p - P[short].sum() > 5 * S.MASS_EPS  # well below p, not a rounding case
    assert ranked[-1] in S.allowed_diff(x, core, p=p)  # the difference lies in the band
    with pytest.raises(AssertionError, match="mass"):
        S.check_support(short, x, core, L=len(x), p=p)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topp_adding_a_band_member_fails(seed):
    p = 0.9
    x, core = _boundary_row(seed, p)
    _, order = _ranked(x, core)
    nxt = int(order[len(core)])
    P = O.softmax_mass(x)
    assert P[core].sum() - p > 5 * S.MASS_EPS  # the oracle set is clearly past p
    assert nxt in S.allowed_diff(x, core, p=p)
    longer = np.array(sorted(core.tolist() + [nxt]))
    with pytest.raises(AssertionError, match="not minimal"):
        S.check_support(longer, x, core, L=len(x), p=p)


def test_topp_swap_of_exact_ties_passes():
    p = 0.9
    x, core = _boundary_row(5, p)
    ranked, order = _ranked(x, core)
    last, nxt = ranked[-1], int(order[len(core)])
    x[nxt] = x[last]  # an exact tie across the boundary
    core = O.select_topp(x, p)
    ranked, order = _ranked(x, core)
    a, b = ranked[-1], int(order[len(core)])
    assert x[a] == x[b]
    swapped = np.array(sorted((set(core.tolist()) - {a}) | {b}))
    assert S.check_support(swapped, x, core, L=len(x), p=p) == 2


def test_difference_outside_the_band_fails():
    p = 0.9
    x, core = _boundary_row(3, p)
    ranked, order = _ranked(x, core)
    far = int(order[-1])  # the lowest score of the row
    bad = np.array(sorted(ranked[:-1] + [far]))
    with pytest.raises(AssertionError, match="outside the tie band"):
        S.check_support(bad, x, core, L=len(x), p=p)


def test_topk_size_must_match():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(500)
    x[10] = x[11]  # a tie inside the list does not matter here
    core = O.select_topk(x, 40)
    ranked, _ = _ranked(x, core)
    x2 = x.copy()
    x2[ranked[-1]] = x2[ranked[-2]] - 1e-9  # the last member sits in the band
    core2 = O.select_topk(x2, 40)
    ranked2, _ = _ranked(x2, core2)
    with pytest.raises(AssertionError, match="size"):
        S.check_support(np.array(sorted(ranked2[:-1])), x2, core2, L=len(x2), k=40)


def test_forced_tokens_must_match():
    p = 0.9
    x, core = _boundary_row(6, p, n=800)
    full = O.with_sink_window(core, 800, 4, 32)
    broken = np.array([j for j in full if j != 2])  # a sink token missing
    with pytest.raises(AssertionError, match="forced"):
        S.check_support(broken, x, core, L=800, p=p, n_sink=4, n_window=32)
