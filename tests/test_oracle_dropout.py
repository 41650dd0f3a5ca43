"""Pins of the oracle's LoRA dropout: the counter-based generator, the mask, and the forward
and backward with the mask applied to the adapter input."""

import numpy as np
import pytest

import oracle
from oracle import dropout as od


@pytest.mark.parametrize("key", [(0, 0), (123, 456), (2**64 - 1, 2**63 + 5)])
def test_philox_blocks_match_numpy(key):
    """numpy ships its own Philox4x64-10; it advances the counter before producing each
    block, so its state at counter c - 1 yields block c."""
    for c in (1, 2, 3, 2**32 + 7, 2**64 - 1):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                              counter=np.array([c - 1, 0, 0, 0], dtype=np.uint64))
        want = [int(v) for v in bg.random_raw(4)]
        assert list(od.philox4x64_10((c, 0, 0, 0), key)) == want, c
    # a counter with every word in use (carry into the upper words is numpy's)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array([2**64 - 1, 5, 9, 11], dtype=np.uint64))
    want = [int(v) for v in bg.random_raw(4)]
    assert list(od.philox4x64_10((0, 6, 9, 11), key)) == want


def test_vectorised_mask_equals_block_by_block():
    for T, K, p, seed in ((7, 200, 0.05, 99), (3, 64, 0.5, 2**40 + 3), (1, 13, 0.9, 0)):
        assert np.array_equal(od.keep_mask(T, K, p, seed), od.keep_mask_scalar(T, K, p, seed))


def test_kept_fraction_is_binomial():
    T, K, p = 512, 2048, 0.05
    keep = od.keep_mask(T, K, p, 2024)
    n = T * K
    sd = np.sqrt(n * p * (1 - p))
    assert abs((n - keep.sum()) - n * p) < 6 * sd
    # rows and columns are not correlated into stripes: per-column drop counts are binomial too
    col = (~keep).sum(axis=0)
    assert abs(col.mean() - T * p) < 6 * np.sqrt(T * p * (1 - p) / K)
    assert od.keep_mask(4, 64, 0.0, 1).all()
    assert od.keep_threshold(0.05) == round(0.05 * 2**32)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_zero_probability_is_the_plain_layer():
    rng = np.random.default_rng(40)
    T, N, K, r, s = 5, 7, 64, 3, 0.75
    x, w, a, b, dy = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r), _rand(rng, T, N)
    keep = od.keep_mask(T, K, 0.0, 5)
    y, u = od.forward_f64(x, w, a, b, s, keep, 0.0)
    y0, u0 = oracle.forward_f64(x, w, a, b, s)
    assert np.array_equal(y, y0) and np.array_equal(u, u0)
    g = od.backward_f64(dy, x, w, a, b, s, keep, 0.0)
    g0 = oracle.backward_f64(dy, x, w, a, b, s)
    for got, want in zip(g, g0):
        assert np.array_equal(got, want)


def test_u_is_unbiased_over_seeds():
    """Inverted dropout: the mean of u over many masks is x A^T.  Without the 1 / (1 - p)
    factor the mean would be off by 5.3% at p = 0.05, far outside the statistical band."""
    rng = np.random.default_rng(41)
    T, K, r, p = 2, 2048, 3, 0.05
    x, a = np.abs(_rand(rng, T, K)), np.abs(_rand(rng, r, K))  # positive: no cancellation
    w, b = np.zeros((1, K)), np.zeros((1, r))
    want = x @ a.T
    us = [od.forward_f64(x, w, a, b, 1.0, od.keep_mask(T, K, p, seed), p)[1] for seed in range(300)]
    mean = np.mean(us, axis=0)
    rel_sd = np.std(us, axis=0) / np.sqrt(len(us)) / want
    assert np.all(np.abs(mean / want - 1) < 6 * rel_sd + 1e-12)
    assert np.all(6 * rel_sd < 0.01)  # the band is far narrower than a missing factor


def test_dropped_inputs_reach_y_only_through_the_base_product():
    rng = np.random.default_rng(42)
    T, N, K, r, s, p = 4, 6, 64, 5, 2.0, 0.3
    x, w, a, b = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r)
    keep = od.keep_mask(T, K, p, 77)
    y0, _ = od.forward_f64(x, w, a, b, s, keep, p)
    dropped = np.argwhere(~keep)
    kept = np.argwhere(keep)
    assert len(dropped) > 10 and len(kept) > 10
    for (t, k) in list(dropped[:5]) + list(kept[:5]):
        x1 = x.copy()
        x1[t, k] += 1.0
        y1, _ = od.forward_f64(x1, w, a, b, s, keep, p)
        base = np.zeros_like(y0)
        base[t] = w[:, k]
        lora = np.zeros_like(y0)
        lora[t] = s / (1 - p) * (b @ a[:, k])
        want = base + (lora if keep[t, k] else 0.0)
        np.testing.assert_allclose(y1 - y0, want, rtol=1e-9, atol=1e-9)


def test_backward_is_the_adjoint_of_the_forward():
    """y is linear in x, in A and in B for a fixed mask, so <dy, y(z + d) - y(z)> equals
    <grad_z, d> for each of them up to rounding."""
    rng = np.random.default_rng(43)
    T, N, K, r, s, p = 6, 9, 128, 4, 0.5, 0.2
    x, w, a, b, dy = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r), _rand(rng, T, N)
    keep = od.keep_mask(T, K, p, 13)
    gx, ga, gb = od.backward_f64(dy, x, w, a, b, s, keep, p)
    y0, _ = od.forward_f64(x, w, a, b, s, keep, p)
    dx, da, db = _rand(rng, T, K), _rand(rng, r, K), _rand(rng, N, r)
    for got_dir, grad, d in (
        (od.forward_f64(x + dx, w, a, b, s, keep, p)[0] - y0, gx, dx),
        (od.forward_f64(x, w, a + da, b, s, keep, p)[0] - y0, ga, da),
        (od.forward_f64(x, w, a, b + db, s, keep, p)[0] - y0, gb, db),
    ):
        lhs, rhs = float(np.sum(dy * got_dir)), float(np.sum(grad * d))
        assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + abs(rhs) + 1)
