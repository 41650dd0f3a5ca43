"""Pins of the oracle's fp32 / bf16 / e4m3 roundings."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.rounding import _E4M3_TABLE


def _rn_bits(q: Fraction, p: int, emin: int) -> Fraction:
    """Brute force: nearest value with p significant bits (exponent >= emin), ties even."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - (p - 1), emin - (p - 1))
    unit = Fraction(2) ** qe
    lo = (a // unit) * unit
    hi = lo + unit
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if (lo / unit) % 2 == 0 else hi
    return r if q > 0 else -r


def test_rn32_from_fraction_vs_numpy_and_brute_force():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000))
    # exact ties halfway between adjacent fp32 numbers, including subnormal ones
    for f in rng.standard_normal(300).astype(np.float32).tolist() + [1e-45, 3e-45, 1e-40, 1.0, 3.0]:
        f = np.float32(f)
        nxt = np.nextafter(f, np.float32(np.inf))
        xs.append((float(f) + float(nxt)) / 2)
    for x in xs:
        want = np.float32(x)  # numpy's double -> float conversion rounds to nearest even
        got = oracle.rn32_from_fraction(Fraction(x))
        assert got.view(np.uint32) == want.view(np.uint32), x
    for x in xs[:200]:
        assert Fraction(float(oracle.rn32_from_fraction(Fraction(x)))) == _rn_bits(Fraction(x), 24, -126)


def test_bf16_rne_vs_torch_cast():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    bits[::4] = (bits[::4] & 0xFFFF0000) | 0x8000  # exact ties
    bits[1::4] = (bits[1::4] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    got = oracle.bf16_rne_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rne_vs_brute_force():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 30, 3000)).astype(np.float32)
    got = oracle.bf16_bits_to_f32(oracle.bf16_rne_bits(x))
    for xi, gi in zip(x.tolist(), got.tolist()):
        assert Fraction(gi) == _rn_bits(Fraction(xi), 8, -126), xi


def test_e4m3_table_facts():
    vals = [v for v in _E4M3_TABLE[:128] if not math.isnan(v)]
    assert len(vals) == 127  # +0 and 126 positive finite values
    assert max(vals) == 448.0
    assert min(v for v in vals if v > 0) == 2.0 ** -9
    assert math.isnan(_E4M3_TABLE[0x7F]) and math.isnan(_E4M3_TABLE[0xFF])
    assert _E4M3_TABLE[0x08] == 2.0 ** -6  # smallest normal


def test_e4m3_roundtrip_every_byte():
    for byte in range(256):
        if byte in (0x7F, 0xFF):
            continue
        v = _E4M3_TABLE[byte]
        assert oracle.e4m3_encode_f64(np.array([v]))[0] == byte
        if byte != 0x80:
            assert oracle.e4m3_encode_exact(Fraction(v)) == byte


def test_e4m3_exact_vs_torch_cast_of_clamped_values():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-4, 3, 200000)).astype(np.float32)
    # midpoints between neighbouring e4m3 values are exact ties
    pos = np.array(sorted({abs(v) for v in _E4M3_TABLE if not math.isnan(v)}))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.array([447.0, 448.0, 449.0, 464.0, 470.0, 1e6], np.float32)])
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode_f64(x.astype(np.float64))
    # torch keeps the sign of values that round to zero, as the oracle does
    assert np.array_equal(got, want)


def test_e4m3_f64_quotient_vs_exact_rational():
    """The vectorised encoder on an fp64 quotient of two fp32 numbers equals the brute-force
    encoder on the exact rational quotient, including quotients hugging rounding boundaries."""
    rng = np.random.default_rng(5)
    pos = sorted({abs(v) for v in _E4M3_TABLE if not math.isnan(v)})
    bounds = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    cases = []
    for _ in range(1500):
        s2 = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-6, 2))
        d = np.float32(rng.uniform(-448, 448) * float(s2))
        cases.append((d, s2))
    for bnd in bounds:  # numerators as close as fp32 allows to boundary * s2
        for _ in range(6):
            s2 = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-5, 2))
            d0 = np.float32(bnd * float(s2))
            for d in (np.nextafter(d0, np.float32(-np.inf)), d0, np.nextafter(d0, np.float32(np.inf))):
                cases.append((np.float32(d), s2))
                cases.append((np.float32(-d), s2))
    d = np.array([c[0] for c in cases], np.float32)
    s = np.array([c[1] for c in cases], np.float32)
    got = oracle.e4m3_encode_f64(d.astype(np.float64) / s.astype(np.float64))
    for i, (di, si) in enumerate(cases):
        assert got[i] == oracle.e4m3_encode_exact(Fraction(float(di)) / Fraction(float(si))), (di, si)
