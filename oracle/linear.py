"""Forward and backward of the QLoRA linear layer, evaluated in fp64.

Test infrastructure only (see the package docstring).

Sources:
* "qlora" encyclopedia entry (tonho.wtf), section "a ideia": the frozen base
  weight is dequantized to BFloat16 for the matrix product; the gradient
  crosses the frozen weight and lands only in the LoRA adapters, the only
  parameters with their own gradient, kept in 16 bits.
* "Tutorial fine-tuning LLM LoRA/QLoRA" (nexusinovation blog), section
  "LoRA: O Padrão Ouro de Eficiência": W' = W + a.AB with a low rank r.

Naming used throughout: the weight is W [n_out x n_in]; the adapters are
A [r x n_in] and B [n_out x r], so the adapted weight is W' = W_hat + s.B.A,
and for activations x [T x n_in]:

    Y      = x W_hat^T + s (x A^T) B^T
    u      = x A^T                       (saved for the backward pass)
    v      = dy B
    grad_x = dy W_hat + s v A
    grad_A = s v^T x
    grad_B = s dy^T u
    (no gradient for W_hat: it is frozen)

The scale s is an argument.  The tutorial writes the factor as alpha; the
configurations give alpha and r separately, and the reading taken for them is
s = alpha / r (the usual LoRA convention); nothing here depends on it.

All inputs are the exact bf16 values (uint16 bit patterns) widened to fp64;
no intermediate is rounded.

Pins (tests/test_oracle_linear.py): the forward equals x W'^T with the merged
weight W' = W_hat + s B A written out element by element on tiny inputs;
grad_A and grad_B equal the chain rule through the merged weight
(s B^T (dy^T x) and s (dy^T x) A^T); adjoint identities
<grad_x, x> = <dy, Y>, <grad_A, A> = <grad_B, B> = <dy, Y - x W_hat^T>;
central finite differences of <dy, Y> with respect to x, A and B.
"""

import numpy as np

from .rounding import bf16_bits_to_f32


def _f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def forward_f64(x, w, a, b, scale: float):
    """Y and u from fp64 arrays (the definition; no rounding anywhere)."""
    u = x @ a.T
    y = x @ w.T + float(scale) * (u @ b.T)
    return y, u


def backward_f64(dy, x, w, a, b, scale: float):
    """grad_x, grad_A, grad_B from fp64 arrays."""
    s = float(scale)
    u = x @ a.T
    v = dy @ b
    grad_x = dy @ w + s * (v @ a)
    grad_a = s * (v.T @ x)
    grad_b = s * (dy.T @ u)
    return grad_x, grad_a, grad_b


def forward(x_bits, w_hat_bits, a_bits, b_bits, scale: float):
    """Return (Y, u) in fp64 for bf16 inputs x [T x K], W_hat [N x K], A [r x K], B [N x r]."""
    return forward_f64(_f64(x_bits), _f64(w_hat_bits), _f64(a_bits), _f64(b_bits), scale)


def backward(dy_bits, x_bits, w_hat_bits, a_bits, b_bits, scale: float):
    """Return (grad_x, grad_A, grad_B) in fp64; there is no gradient for the frozen weight."""
    return backward_f64(_f64(dy_bits), _f64(x_bits), _f64(w_hat_bits), _f64(a_bits), _f64(b_bits), scale)
