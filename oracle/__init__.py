"""CPU oracle for the QLoRA linear layer (NF4 storage, FP8 double quantization, LoRA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, links or
calls this package; only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark do.  It is a plain, slow, deliberately unoptimised
statement of what the method computes, written from the pages' description:

* "qlora" encyclopedia entry (tonho.wtf), sections "a ideia" and
  "como funciona": 4-bit storage type built from standard-normal quantiles,
  normalised to [-1, 1] by the absolute maximum, asymmetric so that zero is
  exact, blocks of 64 elements with one constant each; the constants are
  themselves quantised to FP8 in blocks of 256; every use of the weight
  dequantises it to BFloat16 for the matrix product; gradients pass through
  the frozen weight into 16-bit LoRA adapters only.
* "Tutorial fine-tuning LLM LoRA/QLoRA" (nexusinovation blog), section
  "LoRA: O Padrão Ouro de Eficiência": the adapted weight is W' = W + a.AB.

Floating point: every codec step has one named rounding (fp32 round to
nearest even, bf16 round to nearest even, e4m3 round to nearest even with
saturation); the matrix products are evaluated in fp64 from the exact inputs.

Modules
-------
codebook  the 16 NF4 levels from their definition
rounding  fp32 / bf16 / e4m3 rounding written from the IEEE-style definitions
nf4       blocking, nearest code, packing, mean, double quantization, decode
linear    forward and backward of the adapted linear layer in fp64
adamw     the AdamW update of the adapters (fp32 states, fp32 master copy)
dropout   LoRA dropout on the adapter input: Philox4x64-10 mask, forward and backward

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` (see each module's docstring for its pins), except
the one noted in ``nf4.relative_error`` (informational, not compared).
"""

from .codebook import nf4_codebook, nf4_codebook_f64, nf4_midpoints  # noqa: F401
from .rounding import (  # noqa: F401
    bf16_bits_to_f32,
    bf16_rne_bits,
    e4m3_decode,
    e4m3_encode_f64,
    e4m3_encode_exact,
    rn32_from_fraction,
)
from .nf4 import (  # noqa: F401
    NF4Quantized,
    bits_per_param,
    block_absmax,
    dequantize,
    dequantize_constants,
    double_quantize,
    exact_mean_f32,
    nearest_codes,
    pack_codes,
    quantize,
    unpack_codes,
)
from .linear import backward, backward_f64, forward, forward_f64  # noqa: F401
from . import dropout  # noqa: F401
from .adamw import adamw_step, step_scalars  # noqa: F401
