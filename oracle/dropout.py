"""LoRA dropout on the adapter input (oracle).

TEST INFRASTRUCTURE ONLY: see the package docstring.

What the pages fix
------------------
The training recipe sets a dropout probability on the LoRA adapters, 0.05,
next to the rank and alpha -- "Tutorial fine-tuning LLM LoRA/QLoRA"
(nexusinovation), section "Código Completo", step "4. Configuração LoRA"
(``lora_dropout``).  The pages say nothing more about it.

Readings
--------
* Dropout acts on the input of the adapter path only (the frozen base
  product sees x unchanged): y = x W^T + s * u B^T with
  u = (1 / (1 - p)) * (keep (.) x) A^T  ("inverted" dropout: kept values are
  scaled so that the expectation of u is x A^T).
* The backward uses the same mask:
      grad_x = dy W + (s / (1 - p)) * keep (.) (v A),      v = dy B
      grad_A = (s / (1 - p)) * v^T (keep (.) x)
      grad_B = s * dy^T u
* The mask is drawn from a counter-based generator, Philox4x64-10 (Salmon,
  Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC 2011), so that the forward and the backward (and the GPU) regenerate
  the same mask from (seed, position) alone.  Element e = t K + k of the
  [T x K] input takes 32-bit word e mod 8 of the block for counter
  (e div 8, 0, 0, 0) under key (seed, 0): the block's four 64-bit outputs in
  order, low half first.  The element is kept iff its word is at least
  thresh = min(2^32 - 1, floor(p 2^32 + 1/2)); p = 0 keeps everything.

Pins (tests/test_oracle_dropout.py): the generator against numpy's own
Philox4x64-10 (an independent implementation; numpy steps its counter before
each block, so its counter c - 1 gives block c); the kept fraction within
binomial bounds; p = 0 reduces to the plain layer exactly; unbiasedness of u
over many seeds (the 1 / (1 - p) factor); inputs at dropped positions reach y
only through the base product; and the backward against the forward by the
adjoint identities <dy, y(x + d) - y(x)> = <grad_x, d> (and likewise for A
and B), which hold exactly for a fixed mask because y is linear in each.
"""

import numpy as np

from .rounding import bf16_bits_to_f32

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157  # round multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B  # key increments (Weyl sequence)
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """The Philox4x64 block function with 10 rounds: 4 x 64-bit counter words and
    2 x 64-bit key words (Python ints) -> 4 x 64-bit output words."""
    c0, c1, c2, c3 = (int(v) & _MASK64 for v in counter)
    k0, k1 = (int(v) & _MASK64 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK64
            k1 = (k1 + _W1) & _MASK64
        p0 = _M0 * c0  # 128-bit products, split into high and low words
        p1 = _M1 * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & _MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64
    return c0, c1, c2, c3


def keep_threshold(p: float) -> int:
    """32-bit threshold: a uniform word below it drops the element."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min((1 << 32) - 1, int(np.floor(p * 2.0 ** 32 + 0.5)))


def keep_mask_scalar(T: int, K: int, p: float, seed: int) -> np.ndarray:
    """bool [T x K]: True where element (t, k) of the adapter input is kept (one block
    function call at a time, Python integers)."""
    thresh = keep_threshold(p)
    n = T * K
    words = np.empty(((n + 7) // 8) * 8, dtype=np.uint64)
    for c in range((n + 7) // 8):
        out = philox4x64_10((c, 0, 0, 0), (seed, 0))
        for j in range(4):
            words[8 * c + 2 * j] = out[j] & 0xFFFFFFFF
            words[8 * c + 2 * j + 1] = out[j] >> 32
    return (words[:n] >= thresh).reshape(T, K)


def _mulhilo64(a: int, b: np.ndarray):
    """High and low 64-bit words of a * b for a constant a and a uint64 array b, from
    32-bit halves (every partial product fits in 64 bits; numpy wraps modulo 2^64)."""
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    ah, al = np.uint64(a >> 32), np.uint64(a & 0xFFFFFFFF)
    bh, bl = b >> s32, b & m32
    ll, lh, hl, hh = al * bl, al * bh, ah * bl, ah * bh
    mid = (ll >> s32) + (lh & m32) + (hl & m32)  # < 3 * 2^32
    lo = (ll & m32) | ((mid & m32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def keep_mask(T: int, K: int, p: float, seed: int) -> np.ndarray:
    """keep_mask_scalar for all blocks at once (numpy uint64 arrays); the tests pin the
    two against each other."""
    thresh = keep_threshold(p)
    n = T * K
    nc = (n + 7) // 8
    c0 = np.arange(nc, dtype=np.uint64)
    z = np.zeros(nc, dtype=np.uint64)
    c1, c2, c3 = z.copy(), z.copy(), z.copy()
    k0, k1 = int(seed) & _MASK64, 0
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = (k0 + _W0) & _MASK64
                k1 = (k1 + _W1) & _MASK64
            hi0, lo0 = _mulhilo64(_M0, c0)
            hi1, lo1 = _mulhilo64(_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    out = np.stack([c0, c1, c2, c3], axis=1)  # [nc, 4]
    m32 = np.uint64(0xFFFFFFFF)
    words = np.stack([out & m32, out >> np.uint64(32)], axis=2).reshape(-1)  # low half first
    return (words[:n] >= np.uint64(thresh)).reshape(T, K)


def _f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def forward_f64(x, w, a, b, scale: float, keep, p: float):
    """(y, u) in fp64 with dropout on the adapter input (no rounding anywhere)."""
    xd = np.where(keep, x, 0.0)
    u = (xd @ a.T) / (1.0 - p)
    y = x @ w.T + float(scale) * (u @ b.T)
    return y, u


def backward_f64(dy, x, w, a, b, scale: float, keep, p: float):
    """(grad_x, grad_A, grad_B) in fp64 for the same mask."""
    s = float(scale)
    xd = np.where(keep, x, 0.0)
    u = (xd @ a.T) / (1.0 - p)
    v = dy @ b
    grad_x = dy @ w + (s / (1.0 - p)) * np.where(keep, v @ a, 0.0)
    grad_a = (s / (1.0 - p)) * (v.T @ xd)
    grad_b = s * (dy.T @ u)
    return grad_x, grad_a, grad_b


def forward(x_bits, w_hat_bits, a_bits, b_bits, scale: float, p: float, seed: int):
    """(y, u) in fp64 for bf16 inputs, the mask drawn from (p, seed)."""
    x = _f64(x_bits)
    keep = keep_mask(x.shape[0], x.shape[1], p, seed)
    return forward_f64(x, _f64(w_hat_bits), _f64(a_bits), _f64(b_bits), scale, keep, p)


def backward(dy_bits, x_bits, w_hat_bits, a_bits, b_bits, scale: float, p: float, seed: int):
    """(grad_x, grad_A, grad_B) in fp64 for bf16 inputs, the mask drawn from (p, seed)."""
    x = _f64(x_bits)
    keep = keep_mask(x.shape[0], x.shape[1], p, seed)
    return backward_f64(_f64(dy_bits), x, _f64(w_hat_bits), _f64(a_bits), _f64(b_bits), scale, keep, p)
