"""AdamW update of the LoRA adapters (oracle).

TEST INFRASTRUCTURE ONLY: see the package docstring.

What the pages fix
------------------
* Only the adapters are trained; the optimizer keeps, for each trained value,
  two extra values (the Adam moments) -- "LoRA vs. QLoRA vs. Full
  Fine-Tuning" (cloudzy), section "Quanta VRAM cada método precisa?".
* The states of the optimizer may live in memory the CPU also holds and are
  brought back when the update runs ("paged optimizers") -- "qlora"
  encyclopedia entry (tonho.wtf), section "como funciona"; "IA para Todos"
  (e-tribuna), section "NF4 e Paged Optimizers".
* The training recipe uses an Adam-type optimizer with learning rate 2e-4 --
  "Tutorial fine-tuning LLM LoRA/QLoRA" (nexusinovation), section "Código
  Completo", step "6. Trainer".

Readings (the pages do not write the update out)
------------------------------------------------
* The update is AdamW: Adam with bias-corrected moments and weight decay
  decoupled from the gradient (Loshchilov and Hutter, "Decoupled Weight Decay
  Regularization").
* States and the master copy of the adapters are fp32 (the 32-bit state
  variant); the bf16 copy the linear layer reads is the master value rounded
  to nearest even.
* Every operation is one fp32 operation with one rounding, in the order
  below; no fused multiply-add.  The hyperparameters are given as fp64
  numbers; the scalars that depend only on them and on the step are formed
  from them in fp64 and rounded once to fp32; b^t is the C library's fp64
  pow (a library primitive; a last-bit difference in it changes the fp32
  scalar only when that scalar sits on a rounding boundary).

    c_m = fl32(1 - b1)      c_v = fl32(1 - b2)      decay = fl32(1 - lr wd)
    step_size = fl32(lr / (1 - b1^t))               bc2_sqrt = fl32(sqrt(1 - b2^t))

    m  <- fl(fl(b1 m) + fl(c_m g))
    v  <- fl(fl(b2 v) + fl(c_v fl(g g)))
    d   = fl(fl(sqrt(v) / bc2_sqrt) + eps)
    p  <- fl(p decay)
    p  <- fl(p - fl(step_size fl(m / d)))
    p_bf16 = bf16_rne(p)

Pins (tests/test_oracle_adamw.py): torch.optim.AdamW on the CPU (an
independent implementation of the same algorithm) over several steps; the
closed form of a zero gradient (p decays by exactly `decay` per step, the
moments stay 0); the first step with no decay (|p1 - p0| = lr up to eps for
|g| >> eps); a constant gradient (m / (1 - b1^t) -> g).
"""

import math

import numpy as np

from .rounding import bf16_rne_bits

f32 = np.float32


def step_scalars(step, lr, beta1, beta2, eps, weight_decay):
    """The fp32 scalars of step `step` (1-based), formed as the module docstring states."""
    b1, b2, lr, wd = float(beta1), float(beta2), float(lr), float(weight_decay)
    p1, p2 = math.pow(b1, step), math.pow(b2, step)
    return {
        "b1": f32(b1),
        "b2": f32(b2),
        "c_m": f32(1.0 - b1),
        "c_v": f32(1.0 - b2),
        "decay": f32(1.0 - lr * wd),
        "step_size": f32(lr / (1.0 - p1)),
        "bc2_sqrt": f32(math.sqrt(1.0 - p2)),
        "eps": f32(eps),
    }


def adamw_step(param, grad, exp_avg, exp_avg_sq, step, lr, beta1, beta2, eps, weight_decay):
    """One AdamW update in fp32, one rounding per operation.

    param, exp_avg, exp_avg_sq: float32 arrays, updated in place; grad: float32.
    Returns the bf16 bit patterns (uint16) of the updated param.
    """
    for a in (param, grad, exp_avg, exp_avg_sq):
        assert a.dtype == np.float32
    s = step_scalars(step, lr, beta1, beta2, eps, weight_decay)
    g = grad
    with np.errstate(over="ignore", invalid="ignore"):
        m = (s["b1"] * exp_avg) + (s["c_m"] * g)
        v = (s["b2"] * exp_avg_sq) + (s["c_v"] * (g * g))
        d = (np.sqrt(v) / s["bc2_sqrt"]) + s["eps"]
        p = param * s["decay"]
        p = p - (s["step_size"] * (m / d))
    assert m.dtype == v.dtype == d.dtype == p.dtype == np.float32
    exp_avg[...] = m
    exp_avg_sq[...] = v
    param[...] = p
    return bf16_rne_bits(p)
