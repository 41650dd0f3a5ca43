"""Seeded synthetic inputs for the QLoRA linear layer.

This module only draws random numbers: it holds none of the method's
arithmetic.  It serves the tests, the smoke check and the benchmark alike.
Every tensor is drawn in fp64 with numpy's ``default_rng``, rounded to fp32
(round to nearest even), and activations/adapters are then rounded once more
to bf16 with torch's CPU cast (round to nearest even); bf16 tensors are
returned as uint16 bit patterns.

Workloads (LLaMA-shaped, as the method targets LLaMA 7B and 65B; the pages'
models and datasets are not needed, these stand in for them):

* ``tiny``      W 512x256 ~N(0, 0.02); r=8, alpha=16; A, B ~N(0, 0.01);
                x 16x256 ~N(0, 1); dy 16x512 ~N(0, 1); seed 0, drawn in that
                order from one generator.
* ``7b_attn``   W 4096x4096 ~N(0, 0.02); r=64, alpha=16; A, B ~N(0, 0.01);
                x, dy T x 4096 ~N(0, 1) (T = 1 or 2048 = batch 4 x seq 512);
                seed 2, one child stream per tensor.
* ``7b_layer``  the seven LLaMA-7B decoder linears (q, k, v, o 4096x4096;
                gate, up 11008x4096; down 4096x11008), each as ``7b_attn``;
                T = 2048; seed 3.
* ``65b_layer`` the seven LLaMA-65B decoder linears (q, k, v, o 8192x8192;
                gate, up 22016x8192; down 8192x22016); W = 0.02 Student-t(5)
                with 0.1% of positions (without replacement) scaled by 20;
                T = 4096 = 8 sequences x 512 with the last 26 tokens of every
                sequence zero (5.08% padding rows); seed 4.
* ``65b_bulk``  80 layers of the 65B shapes, W ~N(0, 0.02), one child seed per
                layer from SeedSequence(5).
* ``adamw``     a flat adapter buffer of n values: master weights ~N(0, 0.01)
                with the B half of each adapter (here: every second 4096-run)
                zero, as LoRA starts B at zero; gradients ~N(0, 1) times
                10^U(-6, -1) (six decades, as adapter gradients spread), with
                1% exact zeros; states start at zero; one child stream per
                step from SeedSequence(seed).  The 7B layer set's adapters at
                r = 64 hold 32 x 4,997,120 values (``adapter_numel``).
"""

from dataclasses import dataclass

import numpy as np

SHAPES_7B = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
             ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
SHAPES_65B = [("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
              ("gate", 22016, 8192), ("up", 22016, 8192), ("down", 8192, 22016)]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns via torch's CPU cast (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _normal(rng, shape, std) -> np.ndarray:
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


@dataclass
class LinearCase:
    name: str
    n_out: int
    n_in: int
    r: int
    alpha: float
    w: np.ndarray  # float32 [n_out, n_in]
    a: np.ndarray  # bf16 bits [r, n_in]
    b: np.ndarray  # bf16 bits [n_out, r]
    x: np.ndarray  # bf16 bits [T, n_in]
    dy: np.ndarray  # bf16 bits [T, n_out]

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    @property
    def tokens(self) -> int:
        return self.x.shape[0]


def tiny_case() -> LinearCase:
    rng = np.random.default_rng(0)
    w = _normal(rng, (512, 256), 0.02)
    a = _normal(rng, (8, 256), 0.01)
    b = _normal(rng, (512, 8), 0.01)
    x = _normal(rng, (16, 256), 1.0)
    dy = _normal(rng, (16, 512), 1.0)
    return LinearCase("tiny", 512, 256, 8, 16.0, w, to_bf16_bits(a), to_bf16_bits(b),
                      to_bf16_bits(x), to_bf16_bits(dy))


def custom_case(n_out: int, n_in: int, tokens: int, r: int, alpha: float, seed: int,
                w_std: float = 0.02, name: str = "custom") -> LinearCase:
    """Same recipe as the 7B projection at any shape (for ragged / multi-tile parity)."""
    streams = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(5)]
    w = _normal(streams[0], (n_out, n_in), w_std)
    a = _normal(streams[1], (r, n_in), 0.01)
    b = _normal(streams[2], (n_out, r), 0.01)
    x = _normal(streams[3], (tokens, n_in), 1.0)
    dy = _normal(streams[4], (tokens, n_out), 1.0)
    return LinearCase(name, n_out, n_in, r, alpha, w, to_bf16_bits(a), to_bf16_bits(b),
                      to_bf16_bits(x), to_bf16_bits(dy))


def attn7b_case(tokens: int = 2048) -> LinearCase:
    return custom_case(4096, 4096, tokens, 64, 16.0, seed=2, name=f"7b_attn_T{tokens}")


def layer7b_cases(tokens: int = 2048):
    """The seven 7B linears, one child seed each (seed 3)."""
    seeds = np.random.SeedSequence(3).spawn(len(SHAPES_7B))
    for (name, n, k), ss in zip(SHAPES_7B, seeds):
        yield custom_case(n, k, tokens, 64, 16.0, seed=int(ss.generate_state(1)[0]), name=f"7b_{name}")


def student_t_weight(rng, n_out: int, n_in: int) -> np.ndarray:
    """0.02 * Student-t(5) with exactly round(0.001 * numel) positions scaled by 20."""
    w = (rng.standard_t(5, size=(n_out, n_in)) * 0.02).astype(np.float32)
    flat = w.reshape(-1)
    k = int(round(0.001 * flat.size))
    idx = rng.choice(flat.size, size=k, replace=False)
    flat[idx] = (flat[idx].astype(np.float64) * 20.0).astype(np.float32)
    return w


def padded_tokens_x(rng, tokens: int, n_in: int, seq: int = 512, pad: int = 26) -> np.ndarray:
    """x ~N(0, 1) with the last ``pad`` tokens of every ``seq``-token sequence zero."""
    x = _normal(rng, (tokens, n_in), 1.0)
    for s0 in range(0, tokens, seq):
        x[s0 + seq - pad: s0 + seq] = 0.0
    return x


def layer65b_cases(tokens: int = 4096, shapes=None, names=None):
    """The 65B linears (seed 4, one child seed per linear).  `names` keeps only those
    linears (each keeps its own seed); `shapes` replaces the shape list."""
    seeds = np.random.SeedSequence(4).spawn(len(SHAPES_65B))
    for (name, n, k), ss in zip(shapes or SHAPES_65B, seeds):
        if names is not None and name not in names:
            continue
        streams = [np.random.default_rng(s) for s in ss.spawn(5)]
        w = student_t_weight(streams[0], n, k)
        a = _normal(streams[1], (64, k), 0.01)
        b = _normal(streams[2], (n, 64), 0.01)
        x = padded_tokens_x(streams[3], tokens, k)
        dy = _normal(streams[4], (tokens, n), 1.0)
        yield LinearCase(f"65b_{name}", n, k, 64, 16.0, w, to_bf16_bits(a), to_bf16_bits(b),
                         to_bf16_bits(x), to_bf16_bits(dy))


def bulk65b_layer_weights(layer: int):
    """fp32 weights of one of the 80 layers of the 65B bulk store, in SHAPES_65B order."""
    ss = np.random.SeedSequence(5).spawn(80)[layer]
    rng = np.random.default_rng(ss)
    for name, n, k in SHAPES_65B:
        yield name, _normal(rng, (n, k), 0.02)


def crafted_weight(seed: int, n_out: int, n_in: int) -> np.ndarray:
    """A weight exercising the codec's corner cases: exact ties at the four fp32-representable
    NF4 midpoints (blocks with power-of-two absmax), all-zero blocks, single outliers,
    subnormal and tiny blocks, negative-only blocks, and ordinary N(0, 0.02) elsewhere."""
    rng = np.random.default_rng(seed)
    w = _normal(rng, (n_out, n_in), 0.02).reshape(-1)
    nblk = w.size // 64
    # The four midpoints of adjacent fp32 NF4 levels that are themselves fp32 numbers; they
    # are inputs here (points of interest), not computed.
    ties = np.array([-0.45999518036842346, -0.045524988323450089,
                     0.039790157228708267, 0.86147832870483398], dtype=np.float32)
    for b in range(nblk):
        blk = w[64 * b: 64 * b + 64]
        kind = b % 8
        if kind == 1:  # power-of-two absmax and exact ties
            scale = np.float32(2.0 ** int(rng.integers(-8, 2)))
            blk[:] = (rng.uniform(-1, 1, 64) * scale).astype(np.float32)
            blk[0] = scale
            blk[1:5] = ties * scale
            blk[5:9] = -ties * scale
        elif kind == 2:
            blk[:] = 0.0
            if b % 16 == 2:
                blk[7] = -0.0
        elif kind == 3:  # one outlier
            blk[int(rng.integers(0, 64))] *= 50.0
        elif kind == 4:  # subnormal magnitudes
            blk[:] = (rng.integers(-2000, 2000, 64).astype(np.float64) * 2.0 ** -149).astype(np.float32)
        elif kind == 5:  # negative-only block
            blk[:] = -np.abs(blk)
        elif kind == 6:  # tiny normal block
            blk[:] = (blk * 1e-30).astype(np.float32)
    return w.reshape(n_out, n_in)


def adapter_numel(shapes, r: int, layers: int = 1) -> int:
    """Values in the A [r x n_in] and B [n_out x r] adapters of `layers` copies of `shapes`."""
    return layers * sum(r * k + n * r for _, n, k in shapes)


def adamw_params(seed: int, n: int) -> np.ndarray:
    """Initial fp32 master copy of n adapter values (see ``adamw`` above)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    p = _normal(rng, (n,), 0.01)
    idx = np.arange(n)
    p[(idx // 4096) % 2 == 1] = 0.0
    return p


def adamw_grads(seed: int, n: int, steps: int):
    """`steps` fp32 gradient vectors of n values, one child stream per step."""
    out = []
    for ss in np.random.SeedSequence(seed).spawn(steps + 1)[1:]:
        rng = np.random.default_rng(ss)
        g = rng.standard_normal(n) * 10.0 ** rng.uniform(-6.0, -1.0, n)
        g[rng.random(n) < 0.01] = 0.0
        out.append(g.astype(np.float32))
    return out
