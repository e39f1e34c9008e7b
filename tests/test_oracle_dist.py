"""Pins for the oracle's truncated distribution (readings R1-R4 of the pages'
open points; deniz.in "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head…",
section "Kesme her iki tarafta eşleşmek zorunda").

Expected values come from scipy's softmax, from brute-force orderings written
with Python's ``sorted`` and from hand-worked arithmetic, never from the
oracle itself."""
import math

import numpy as np
import pytest
from scipy.special import softmax

pytestmark = []


def _rng(seed=0):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("T", [1.0, 0.6, 2.5, 1e-3])
def test_untruncated_is_softmax(oracle_mod, T):
    l = _rng(1).normal(0, 3, 50)
    p, cm = oracle_mod.dist(l, T, 0, 1.0)
    np.testing.assert_allclose(p, softmax(l / T), rtol=1e-12, atol=1e-300)
    assert cm == math.inf


@pytest.mark.parametrize("k", [1, 2, 5, 20, 49])
def test_top_k_matches_bruteforce(oracle_mod, k):
    V = 50
    l = np.round(_rng(2).normal(0, 2, V) * 4) / 4  # coarse grid -> many ties
    order = sorted(range(V), key=lambda i: (-l[i], i))[:k]
    expect = np.zeros(V)
    expect[order] = softmax(l[order] / 0.7)
    p, _ = oracle_mod.dist(l, 0.7, k, 1.0)
    np.testing.assert_allclose(p, expect, rtol=1e-12, atol=0)


def test_top_k_disabled_outside_range(oracle_mod):
    l = _rng(3).normal(0, 1, 12)
    full, _ = oracle_mod.dist(l, 1.0, 0, 1.0)
    for k in (-3, 0, 12, 13, 1000):
        p, _ = oracle_mod.dist(l, 1.0, k, 1.0)
        np.testing.assert_array_equal(p, full)


def test_tie_at_kth_boundary_keeps_lower_id(oracle_mod):
    l = np.array([0.0, 3.0, 1.0, 3.0, 1.0, 1.0])
    p, _ = oracle_mod.dist(l, 1.0, 3, 1.0)
    # order: id1 (3), id3 (3), then the first of the tied 1.0s -> id2
    e3, e1 = math.exp(3.0), math.exp(1.0)
    z = 2 * e3 + e1
    np.testing.assert_allclose(p, [0, e3 / z, e1 / z, e3 / z, 0, 0], rtol=1e-14)


def test_top_p_hand_worked(oracle_mod):
    # P' = [0.5, 0.3, 0.2] exactly (logits are their logs).
    l = np.log(np.array([0.5, 0.3, 0.2]))
    # mass before id1 = 0.5 < 0.6 -> keep; before id2 = 0.8 >= 0.6 -> drop.
    p, cm = oracle_mod.dist(l, 1.0, 0, 0.6)
    np.testing.assert_allclose(p, [0.5 / 0.8, 0.3 / 0.8, 0.0], rtol=1e-14)
    assert cm == pytest.approx(0.1, abs=1e-12)  # min(0.6-0.5, 0.8-0.6)
    # top_p = 0.5: mass before id1 is 0.5, not < 0.5 -> only id0 survives.
    p, _ = oracle_mod.dist(l, 1.0, 0, 0.5)
    np.testing.assert_array_equal(p, [1.0, 0.0, 0.0])
    # tiny top_p keeps the top token only (the crossing token is kept).
    p, _ = oracle_mod.dist(l, 1.0, 0, 1e-9)
    np.testing.assert_array_equal(p, [1.0, 0.0, 0.0])


def test_top_p_is_walked_over_renormalised_top_k(oracle_mod):
    # Full-vocab mass of the top 2 is small, but after top_k=2 renormalisation
    # the first token alone carries 2/3 >= 0.6, so the cut keeps only it.
    l = np.log(np.array([0.2, 0.1] + [0.7 / 20] * 20))
    p, _ = oracle_mod.dist(l, 1.0, 2, 0.6)
    expect = np.zeros(22)
    expect[0] = 1.0
    np.testing.assert_allclose(p, expect, rtol=1e-14)
    # with top_p=0.7 the second token is kept (mass before it 2/3 < 0.7)
    p, _ = oracle_mod.dist(l, 1.0, 2, 0.7)
    expect[:2] = [2 / 3, 1 / 3]
    np.testing.assert_allclose(p, expect, rtol=1e-13)


def test_temperature_then_truncation(oracle_mod):
    l = np.array([1.0, 0.5, 0.0, -1.0])
    T = 0.5
    w = np.exp((l - 1.0) / T)
    Pp = w / w.sum()
    # P' = [0.657, 0.242, 0.089, 0.012]; walk with top_p = 0.85: the mass
    # before id2 is 0.899 >= 0.85, so two tokens survive.
    keep, cum = 0, 0.0
    for v in Pp:
        if cum < 0.85:
            keep += 1
            cum += v
    assert keep == 2
    p, _ = oracle_mod.dist(l, T, 0, 0.85)
    expect = np.zeros(4)
    expect[:keep] = w[:keep] / w[:keep].sum()
    np.testing.assert_allclose(p, expect, rtol=1e-14)


def test_top_k_one_is_point_mass_at_argmax(oracle_mod):
    l = np.array([0.0, 2.0, 2.0, 1.0])
    p, _ = oracle_mod.dist(l, 0.8, 1, 0.95)
    np.testing.assert_array_equal(p, [0, 1, 0, 0])


def test_shift_and_scale_invariance(oracle_mod):
    l = np.round(_rng(4).normal(0, 2, 40) * 8) / 8  # exact in binary
    base, _ = oracle_mod.dist(l, 1.0, 20, 0.9)
    shifted, _ = oracle_mod.dist(l + 1.0, 1.0, 20, 0.9)
    scaled, _ = oracle_mod.dist(l * 2.0, 2.0, 20, 0.9)
    np.testing.assert_array_equal(base, shifted)
    np.testing.assert_array_equal(base, scaled)


def test_neg_inf_logits(oracle_mod):
    l = np.array([-np.inf, 1.0, -np.inf, 0.0])
    p, _ = oracle_mod.dist(l, 1.0, 0, 1.0)
    np.testing.assert_allclose(p, [0, math.e / (math.e + 1), 0, 1 / (math.e + 1)], rtol=1e-15)
    with pytest.raises(ValueError):
        oracle_mod.dist(np.full(4, -np.inf), 1.0, 0, 1.0)
