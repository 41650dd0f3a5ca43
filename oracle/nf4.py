"""Blockwise NF4 quantization with FP8 double quantization, and its decode.

Test infrastructure only (see the package docstring).

Source: "qlora" encyclopedia entry (tonho.wtf), sections "a ideia" and
"como funciona": 4-bit storage, BFloat16 compute; blocks of 64 elements, one
absmax constant per block so that an outlier cannot spoil the scale of the
whole tensor; the constants (0.5 bit/param in fp32) are quantized to FP8 in
blocks of 256 (0.127 bit/param); zero is exact, so padding quantizes without
error; the weight is dequantized to BFloat16 each time it is used.

Steps and the readings taken where the page is silent:

blocking (``block_absmax``)
    W is flattened row-major; block b holds elements [64 b, 64 b + 64); a
    partial last block is padded with zeros.  c1_b = max |x| over the block,
    exact.  A bf16 source is first widened exactly to fp32.
normalisation + nearest code (``nearest_codes``)
    The code of x is the index of the level nearest to the exact real x / c1_b
    (never rounded).  Tie reading: the level of smaller magnitude wins
    (toward zero).  c1_b = 0 gives code 7 (the exact zero) everywhere.
    Written as exact threshold counting: with midpoints M_j between levels j
    and j+1, code = #{j : x > M_j c1} + #{j : x == M_j c1 and M_j < 0}; M_j c1
    is exact in fp64 (26 + 24 significant bits).
packing (``pack_codes``)
    byte i = code[2i] | code[2i+1] << 4 (low nibble first); an odd tail gets
    high nibble 7 (zero).
mean (``exact_mean_f32``)
    One per tensor (a per-group mean would cost 32/(64*256*256) more and the
    page's 0.127 bit/param leaves room for exactly one fp32 per 256
    constants): mu = RN32(exact sum of c1 / number of blocks).
double quantization (``double_quantize``)
    d_b = fl32(c1_b - mu); for each group g of 256 consecutive blocks (last one
    partial) a_g = max |d_b| and s2_g = fl32(a_g / 448) (IEEE division);
    q_b = e4m3 nearest to the exact real d_b / s2_g (ties even, saturating).
    s2_g = 0 (a_g = 0, or a_g so small that the division underflows) gives
    q_b = 0 for the whole group.
constant decode (``dequantize_constants``)
    c1hat_b = fl32(fl32(e4m3(q_b) * s2_g) + mu): two roundings, no fused
    multiply-add.
weight decode (``dequantize``)
    w_hat = bf16_RNE(fl32(CB[code] * c1hat_b)).
without double quantization (``quantize(..., double_quant=False)``)
    The page prices the fp32 constants before their FP8 quantization at
    0.5 bit/param; the variant stores c1_b itself (fp32, one per block; no
    mean, no FP8 bytes, no group scales) and decodes with c1hat_b = c1_b:
    4.5 bits per parameter.

Pins (tests/test_oracle_nf4.py): Fraction brute-force nearest code on tiny
tensors and on crafted blocks (ties at the four fp32-representable
midpoints, zeros, subnormal absmax, ulp sweeps around every threshold);
"every non-zero block holds code 0 or 15"; "every group with a_g > 0 holds
|q| = 448"; exact round trip of zeros and padding; the bit budget of the page
(0.5 bit/param for fp32 constants at block 64, 0.127 after FP8 at block
256); the mean against an independent Fraction sum; decode of zero codes is
exactly zero.
"""

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .codebook import nf4_codebook
from .rounding import bf16_bits_to_f32, bf16_rne_bits, e4m3_decode, e4m3_encode_f64, rn32_from_fraction

BLOCK = 64
GROUP = 256
ZERO_CODE = 7


@dataclass
class NF4Quantized:
    n_out: int
    n_in: int
    codes: np.ndarray  # uint8 [ceil(numel/2)]
    absmax_fp8: np.ndarray  # uint8 [nblocks]
    absmax_scale: np.ndarray  # float32 [ngroups]
    absmax_mean: np.float32
    absmax: np.ndarray  # float32 [nblocks] first-level constants (not stored; kept for checks)
    double_quant: bool = True  # False: absmax_scale holds the nblocks fp32 constants c1 themselves

    @property
    def numel(self) -> int:
        return self.n_out * self.n_in


def _as_f32(w, src: str) -> np.ndarray:
    if src == "f32":
        return np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if src == "bf16":
        return bf16_bits_to_f32(np.asarray(w, dtype=np.uint16).reshape(-1))
    raise ValueError(src)


def _blocks(flat: np.ndarray) -> np.ndarray:
    nblocks = -(-flat.size // BLOCK)
    pad = np.zeros(nblocks * BLOCK, dtype=np.float32)
    pad[: flat.size] = flat
    return pad.reshape(nblocks, BLOCK)


def block_absmax(flat: np.ndarray) -> np.ndarray:
    """c1_b = max |x| over each zero-padded 64-element block (exact)."""
    return np.abs(_blocks(flat)).max(axis=1).astype(np.float32)


def nearest_codes(flat: np.ndarray, c1: np.ndarray) -> np.ndarray:
    """Code of every element (padded to whole blocks), by exact threshold counting."""
    cb = nf4_codebook().astype(np.float64)
    mid = (cb[:-1] + cb[1:]) / 2.0  # exact in fp64
    xb = _blocks(flat).astype(np.float64)  # [nblocks, 64]
    c = c1.astype(np.float64)[:, None]
    codes = np.zeros(xb.shape, dtype=np.int64)
    for j in range(15):
        t = mid[j] * c  # exact in fp64
        codes += xb > t
        if mid[j] < 0:
            codes += xb == t  # tie goes to the level of smaller magnitude
    return codes.astype(np.uint8)


def pack_codes(codes: np.ndarray, numel: int) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)[:numel]
    if numel % 2:
        c = np.concatenate([c, np.array([ZERO_CODE], dtype=np.uint8)])
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, numel: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out[:numel]


def exact_mean_f32(c1: np.ndarray) -> np.float32:
    """RN32 of the exact arithmetic mean of fp32 values."""
    # Every fp32 value is an integer multiple of 2^-149; scaling by 2^149 in
    # fp64 is exact and gives that integer, so the sum below is exact.
    scaled = np.asarray(c1, dtype=np.float32).astype(np.float64) * 2.0 ** 149
    total = sum(int(v) for v in scaled.tolist())
    return rn32_from_fraction(Fraction(total, len(c1) << 149))


def double_quantize(c1: np.ndarray, mu: np.float32):
    """FP8 double quantization of the block constants -> (q bytes, fp32 group scales)."""
    c1 = np.asarray(c1, dtype=np.float32)
    d = (c1 - np.float32(mu)).astype(np.float32)  # fp32 subtraction, RN
    ngroups = -(-c1.size // GROUP)
    q = np.zeros(c1.size, dtype=np.uint8)
    s2 = np.zeros(ngroups, dtype=np.float32)
    for g in range(ngroups):
        dg = d[g * GROUP:(g + 1) * GROUP]
        a = np.float32(np.abs(dg).max())
        s = np.float32(a / np.float32(448.0))  # IEEE fp32 division
        s2[g] = s
        if s > 0:
            q[g * GROUP:(g + 1) * GROUP] = e4m3_encode_f64(dg.astype(np.float64) / np.float64(s))
    return q, s2


def dequantize_constants(q: np.ndarray, s2: np.ndarray, mu: np.float32) -> np.ndarray:
    """c1hat_b = fl32(fl32(e4m3(q_b) * s2_g) + mu), separate roundings."""
    q = np.asarray(q, dtype=np.uint8)
    g = np.arange(q.size) // GROUP
    prod = (e4m3_decode(q) * np.asarray(s2, dtype=np.float32)[g]).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


def quantize(w, n_out: int, n_in: int, src: str = "f32", double_quant: bool = True) -> NF4Quantized:
    """Quantize a [n_out x n_in] weight (fp32, or bf16 bit patterns) to NF4 + FP8 constants
    (or, with double_quant=False, NF4 + the fp32 block constants)."""
    flat = _as_f32(w, src)
    if flat.size != n_out * n_in:
        raise ValueError("shape mismatch")
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite weight")
    c1 = block_absmax(flat)
    codes = nearest_codes(flat, c1).reshape(-1)
    packed = pack_codes(codes, flat.size)
    if not double_quant:
        return NF4Quantized(n_out, n_in, packed, np.zeros(0, np.uint8), c1.copy(), np.float32(0.0), c1,
                            double_quant=False)
    mu = exact_mean_f32(c1)
    q, s2 = double_quantize(c1, mu)
    return NF4Quantized(n_out, n_in, packed, q, s2, np.float32(mu), c1)


def dequantize(qw: NF4Quantized) -> np.ndarray:
    """Decode to bf16 bit patterns [n_out x n_in]: bf16_RNE(fl32(CB[code] * c1hat))."""
    cb = nf4_codebook()
    codes = unpack_codes(qw.codes, qw.numel)
    if qw.double_quant:
        c1hat = dequantize_constants(qw.absmax_fp8, qw.absmax_scale, qw.absmax_mean)
    else:
        c1hat = np.asarray(qw.absmax_scale, dtype=np.float32)
    blk = np.arange(qw.numel) // BLOCK
    w32 = (cb[codes] * c1hat[blk]).astype(np.float32)
    return bf16_rne_bits(w32).reshape(qw.n_out, qw.n_in)


def bits_per_param(n_out: int, n_in: int, double_quant: bool = True) -> float:
    """Storage cost in bits per parameter of the packed format."""
    numel = n_out * n_in
    nblocks = -(-numel // BLOCK)
    ngroups = -(-nblocks // GROUP)
    code_bits = 8 * (-(-numel // 2))
    if double_quant:
        const_bits = 8 * nblocks + 32 * ngroups + 32
    else:
        const_bits = 32 * nblocks
    return (code_bits + const_bits) / numel


def relative_error(w_f32: np.ndarray, w_hat_bits: np.ndarray) -> float:
    """||W_hat - W|| / ||W|| (informational only; parity unpinned, never compared)."""
    w = np.asarray(w_f32, dtype=np.float64).reshape(-1)
    wh = bf16_bits_to_f32(w_hat_bits.reshape(-1)).astype(np.float64)
    return float(np.linalg.norm(wh - w) / np.linalg.norm(w))
