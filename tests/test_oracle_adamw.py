"""Pins of the oracle's AdamW update of the adapters.

Each pin is chosen so that a plausible mistake fails it: a missing bias
correction, or one taken at the wrong step; a sign error; the weight decay
coupled into the gradient, or dropped; beta1 and beta2 swapped; a wrong order
of the square root and the eps.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

HYPER = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _state(rng, n):
    p = rng.standard_normal(n).astype(np.float32)
    return p, np.zeros(n, np.float32), np.zeros(n, np.float32)


def test_matches_torch_adamw_over_several_steps():
    """torch.optim.AdamW (decoupled decay, bias-corrected moments) is an
    independent implementation of the same update; its roundings differ
    (it blends the first moment with lerp), so agreement is to fp32 rounding.
    Each step starts torch from the oracle's state, so rounding differences
    do not accumulate across steps."""
    rng = np.random.default_rng(70)
    n = 4099
    p, m, v = _state(rng, n)
    tp = torch.tensor(p.copy(), requires_grad=True)
    opt = torch.optim.AdamW([tp], foreach=False, fused=False, betas=(HYPER["beta1"], HYPER["beta2"]),
                            lr=HYPER["lr"], eps=HYPER["eps"], weight_decay=HYPER["weight_decay"])
    for step in range(1, 8):
        # Gradients over several decades, with some exact zeros.
        g = (rng.standard_normal(n) * 10.0 ** rng.integers(-4, 2, n)).astype(np.float32)
        g[::97] = 0.0
        m_prev = m.astype(np.float64)
        if step > 1:
            with torch.no_grad():
                tp.copy_(torch.tensor(p))
            st = opt.state[tp]
            st["exp_avg"].copy_(torch.tensor(m))
            st["exp_avg_sq"].copy_(torch.tensor(v))
            assert int(st["step"]) == step - 1
        bits = oracle.adamw_step(p, g, m, v, step, **HYPER)
        tp.grad = torch.tensor(g.copy())
        opt.step()
        st = opt.state[tp]
        tm, tv = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
        # The first moment mixes signs, so its rounding is relative to the
        # size of the two terms, not of their sum.
        scale = HYPER["beta1"] * np.abs(m_prev) + (1 - HYPER["beta1"]) * np.abs(g.astype(np.float64))
        assert np.all(np.abs(m.astype(np.float64) - tm) <= 4 * 2.0 ** -24 * scale)
        np.testing.assert_allclose(v, tv, rtol=4e-7, atol=0)
        # The update has size about lr; allow a few fp32 ulps of p plus 1e-5 of the update.
        diff = np.abs(p.astype(np.float64) - tp.detach().numpy().astype(np.float64))
        bound = 4 * np.spacing(np.abs(p)).astype(np.float64) + 1e-5 * HYPER["lr"]
        assert np.all(diff <= bound), (step, float((diff - bound).max()))
        assert np.array_equal(bits, oracle.bf16_rne_bits(p))


def test_zero_gradient_is_pure_decay():
    """With g = 0 the moments stay 0, the update m / (sqrt(v)/c + eps) is 0,
    and the weight is multiplied by 1 - lr wd each step: p_t = p_0 (1 - lr wd)^t
    up to one fp32 rounding per step."""
    rng = np.random.default_rng(71)
    p, m, v = _state(rng, 257)
    p0 = p.astype(np.float64)
    g = np.zeros_like(p)
    t = 25
    for step in range(1, t + 1):
        oracle.adamw_step(p, g, m, v, step, **HYPER)
    assert not m.any() and not v.any()
    decay = 1.0 - HYPER["lr"] * HYPER["weight_decay"]
    expect = p0 * decay ** t
    # fp32 decay factor is off by at most half an ulp of 1 (2^-24 relative),
    # and each step rounds once more.
    rel = np.abs(p.astype(np.float64) - expect) / np.abs(expect)
    assert rel.max() <= t * 2.0 ** -23


def test_first_step_moves_each_weight_by_lr_against_the_gradient_sign():
    """At step 1 the bias-corrected moments are g and g^2, so with no decay
    the update is lr g / (|g| + eps): lr times the sign of g when |g| >> eps."""
    rng = np.random.default_rng(72)
    p, m, v = _state(rng, 1000)
    p0 = p.copy().astype(np.float64)
    g = (rng.choice([-1.0, 1.0], 1000) * 10.0 ** rng.uniform(-3, 2, 1000)).astype(np.float32)
    hyper = dict(HYPER, weight_decay=0.0)
    oracle.adamw_step(p, g, m, v, 1, **hyper)
    step = p.astype(np.float64) - p0
    g64 = g.astype(np.float64)
    expect = -hyper["lr"] * g64 / (np.abs(g64) + hyper["eps"])
    assert np.all(np.abs(step - expect) <= 1e-6 * hyper["lr"] + 2 * np.spacing(np.abs(p)))
    # and the size of that step is lr to within eps / |g| (at most 1e-5 here)
    assert np.all(np.abs(np.abs(step) - hyper["lr"]) <= 2e-5 * hyper["lr"] + 2 * np.spacing(np.abs(p)))


def test_constant_gradient_keeps_unit_steps_at_every_step():
    """With a constant gradient, m_t = g (1 - b1^t) and v_t = g^2 (1 - b2^t),
    so the bias-corrected ratio is sign(g) at every step t; a correction taken
    at step t+1 instead shrinks the first step to about 0.74 lr."""
    rng = np.random.default_rng(73)
    p, m, v = _state(rng, 64)
    g = (rng.choice([-1.0, 1.0], 64) * 0.5).astype(np.float32)
    hyper = dict(HYPER, weight_decay=0.0)
    for step in range(1, 41):
        before = p.astype(np.float64)
        oracle.adamw_step(p, g, m, v, step, **hyper)
        moved = p.astype(np.float64) - before
        assert np.all(np.abs(moved + hyper["lr"] * np.sign(g)) <= 2e-6 * hyper["lr"] + 2 * np.spacing(np.abs(p)))
        b1t, b2t = hyper["beta1"] ** step, hyper["beta2"] ** step
        np.testing.assert_allclose(m, g * (1 - b1t), rtol=2e-6 * step)
        np.testing.assert_allclose(v, (g.astype(np.float64) ** 2) * (1 - b2t), rtol=2e-6 * step)


def test_decay_is_decoupled_from_the_moments():
    """AdamW scales the weight by 1 - lr wd and leaves the moments to the
    gradient alone: the moments after a step do not depend on wd."""
    rng = np.random.default_rng(74)
    n = 300
    g = rng.standard_normal(n).astype(np.float32)
    out = []
    for wd in (0.0, 0.5):
        p, m, v = _state(np.random.default_rng(75), n)
        oracle.adamw_step(p, g, m, v, 1, **dict(HYPER, weight_decay=wd))
        out.append((p.copy(), m.copy(), v.copy()))
    assert np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])
    p0 = _state(np.random.default_rng(75), n)[0].astype(np.float64)
    # The weight difference is exactly the decay term lr wd p0 (to rounding).
    np.testing.assert_allclose(out[0][0] - out[1][0], 1e-2 * 0.5 * p0, rtol=1e-3, atol=1e-8)


def test_step_scalars_from_their_definitions():
    """Closed forms of the per-step scalars at t = 1 and t = 2."""
    s1 = oracle.step_scalars(1, 1e-2, 0.9, 0.999, 1e-8, 0.1)
    b1, b2 = 0.9, 0.999
    assert s1["step_size"] == np.float32(1e-2 / (1 - b1))
    assert s1["bc2_sqrt"] == np.float32(math.sqrt(1 - b2))
    s2 = oracle.step_scalars(2, 1e-2, 0.9, 0.999, 1e-8, 0.1)
    assert abs(float(s2["step_size"]) - 1e-2 / (1 - b1 * b1)) <= 1e-9
    assert abs(float(s2["bc2_sqrt"]) - math.sqrt((1 - b2) * (1 + b2))) <= 1e-9
    assert s1["decay"] == np.float32(1 - 1e-2 * 0.1)
    assert s1["c_m"] == np.float32(0.1) and s1["c_v"] == np.float32(1 - 0.999)
    assert s1["b1"] == np.float32(0.9) and s1["b2"] == np.float32(0.999)


def _rn32_exact(q: Fraction) -> float:
    """Round a positive rational to the nearest fp32 value, ties to even (normal range)."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    # q = m * 2^(e - 23) with 2^23 <= m < 2^24
    m = q / Fraction(2) ** (e - 23)
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(Fraction(n) * Fraction(2) ** (e - 23))


def _rn32_sqrt_exact(q: Fraction) -> float:
    """Round sqrt(q) of a positive rational to the nearest fp32 value, ties to even."""
    assert q > 0
    e = 0
    while Fraction(4) ** e > q:
        e -= 1
    while Fraction(4) ** (e + 1) <= q:
        e += 1
    # sqrt(q) = s * 2^(e - 23) with 2^23 <= s < 2^24, s^2 = X
    x = q / Fraction(4) ** (e - 23)
    y = 4 * x  # (2 s)^2
    t2 = math.isqrt(y.numerator // y.denominator)  # floor(2 s)
    n = t2 // 2
    if t2 % 2 == 1:  # s >= n + 1/2
        if Fraction(t2 * t2) != y or n % 2 == 1:
            n += 1
    return float(Fraction(n) * Fraction(2) ** (e - 23))


def test_step_scalars_equal_the_exact_values_rounded_once():
    """step_size = RN32(lr / (1 - b1^t)) and bc2_sqrt = RN32(sqrt(1 - b2^t)) of the exact real
    numbers the fp64 hyperparameters stand for, with b^t an exact rational power (no libm): the
    oracle's fp64 evaluation must round to the same fp32 values at every step the tests run and
    over a sweep of steps and hyperparameters.  A power taken at the wrong step, a missing
    square root or a swapped beta fails it."""
    from fractions import Fraction as F

    cases = [(1e-2, 0.9, 0.999), (2e-4, 0.9, 0.999), (1e-2, 0.8, 0.99), (1e-3, 0.95, 0.9999), (3e-4, 0.5, 0.75)]
    steps = list(range(1, 41)) + [63, 64, 100, 255, 999, 1000, 1001, 1002, 1003, 4096, 10000]
    for lr, b1, b2 in cases:
        fb1, fb2 = F(b1), F(b2)
        p1, p2 = F(1), F(1)
        t_prev = 0
        for t in steps:
            p1 *= fb1 ** (t - t_prev)
            p2 *= fb2 ** (t - t_prev)
            t_prev = t
            s = oracle.step_scalars(t, lr, b1, b2, 1e-8, 0.0)
            assert float(s["step_size"]) == _rn32_exact(F(lr) / (1 - p1)), (lr, b1, t)
            assert float(s["bc2_sqrt"]) == _rn32_sqrt_exact(1 - p2), (b2, t)
        assert float(oracle.step_scalars(1, lr, b1, b2, 1e-8, 0.1)["decay"]) == _rn32_exact(1 - F(lr) * F(0.1))
