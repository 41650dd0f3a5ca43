"""Bit-exact decode inside the fused GEMM on shapes where every tile is full.

A tile is full when all of its rows, output columns and contraction steps are in range; then the
kernel decodes each block from register byte tables (16 products bf16(fl32(level * constant))
selected per code), which is the form every full-size launch runs.  One-hot activation rows with
A = 0 make y row t equal to column k_t of the dequantized weight, and one-hot dy rows with B = 0
make grad_x row t equal to row n_t: a single product is exact in fp32, so the result must equal
the oracle's dequantized BF16 weight bit for bit ("qlora" entry, sections "a ideia" and "como
funciona": the 4-bit weight is dequantized to BFloat16 on every use).  Together the calls cover
every element of every weight, in both storage forms.  T = 40 and 64 run grad_x on the 64-row
few-token tiles (every wave decoding, split contraction; at T = 40 rows 40..63 read row 39 and are
never stored) and, on this shape, the forward on the few-token kernels' matrix tiles (three and four
tiles of 16 tokens); a weight with long forward spans keeps the forward on the 64-row tiles; T = 128
runs the 128-row few-token tiles, T = 256 and 512 the 256 x 128 tiles.
"""

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import announce, dev_bf16, dev_f32, host_bits

pytestmark = pytest.mark.gpu

N_OUT, N_IN, R = 512, 1024, 16  # n_out a multiple of 128, n_in of 64: every tile of both directions is full


def _weight(seed, n_out=N_OUT, n_in=N_IN):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n_out, n_in)) * 0.02).astype(np.float32), rng


def _one_hot(T, width, idx):
    a = np.zeros((T, width), np.float32)
    a[np.arange(T), idx] = 1.0
    return workloads.to_bf16_bits(a)


def _zeros(*shape):
    return np.zeros(shape, np.uint16)


@pytest.mark.parametrize("T", [40, 64])
def test_forward_on_the_few_token_tiles_every_column(T):
    """4096 x 8256 (every tile full; forward spans long enough that its 40- or 64-token x tile would
    not fit the few-token kernels' limit): the forward runs the fused GEMM's 64-row few-token tiles,
    and one-hot rows cover every column of the weight."""
    n_out, n_in = 4096, 8256
    announce(f"few-token tiles one-hot forward {n_out}x{n_in} T={T}")
    w, rng = _weight(700 + T, n_out, n_in)
    q = qlora.quantize(dev_f32(w))
    wh = oracle.dequantize(oracle.quantize(w, n_out, n_in))
    b_rand = dev_bf16(workloads.to_bf16_bits((rng.standard_normal((n_out, R)) * 0.01).astype(np.float32)))
    a_zero = dev_bf16(_zeros(R, n_in))
    cols = rng.permutation(n_in)
    for part in range(-(-n_in // T)):
        ks = cols[(part * T) % n_in:][:T]
        ks = np.concatenate([ks, cols[:T - ks.size]])
        y, _ = qlora.linear_fwd(dev_bf16(_one_hot(T, n_in, ks)), q, a_zero, b_rand, 0.5)
        assert np.array_equal(host_bits(y), wh[:, ks].T), ("forward", part)


@pytest.mark.parametrize("double_quant", [True, False])
@pytest.mark.parametrize("T", [40, 64, 128, 256, 512])
def test_single_linear_every_element(T, double_quant):
    announce(f"full-tile one-hot {N_OUT}x{N_IN} T={T} double_quant={double_quant}")
    w, rng = _weight(300 + T + double_quant)
    q = qlora.quantize(dev_f32(w), double_quant=double_quant)
    wh = oracle.dequantize(oracle.quantize(w, N_OUT, N_IN, double_quant=double_quant))
    bits = workloads.to_bf16_bits
    b_rand = dev_bf16(bits((rng.standard_normal((N_OUT, R)) * 0.01).astype(np.float32)))
    a_rand = dev_bf16(bits((rng.standard_normal((R, N_IN)) * 0.01).astype(np.float32)))
    # forward: the columns of W_hat, every column at least once over the calls
    cols = rng.permutation(N_IN)
    for part in range(-(-N_IN // T)):
        ks = cols[(part * T) % N_IN:][:T]
        ks = np.concatenate([ks, cols[:T - ks.size]])
        y, _ = qlora.linear_fwd(dev_bf16(_one_hot(T, N_IN, ks)), q, dev_bf16(_zeros(R, N_IN)), b_rand, 0.5)
        assert np.array_equal(host_bits(y), wh[:, ks].T), ("forward", part)
    # grad_x: the rows of W_hat, every row once over the calls
    rows = rng.permutation(N_OUT)
    x = dev_bf16(bits(rng.standard_normal((T, N_IN)).astype(np.float32)))
    for part in range(-(-N_OUT // T)):
        ns = rows[(part * T) % N_OUT:][:T]
        ns = np.concatenate([ns, rows[:T - ns.size]])
        gx, _, _ = qlora.linear_bwd(dev_bf16(_one_hot(T, N_OUT, ns)), x, q, a_rand, dev_bf16(_zeros(N_OUT, R)), 0.5)
        assert np.array_equal(host_bits(gx), wh[ns, :]), ("grad_x", part)


@pytest.mark.parametrize("double_quant", [True, False])
def test_two_member_set(double_quant):
    """A set of two weights (512 and 256 output rows) at T = 512: each member's y columns, and the
    summed grad_x with one member's dy row one-hot and the other's zero (alternating by row)."""
    T = 512
    announce(f"full-tile one-hot set (512, 256) x {N_IN} T={T} double_quant={double_quant}")
    n_outs = (512, 256)
    ws, qs, whs = [], [], []
    rng = np.random.default_rng(400 + double_quant)
    for i, n in enumerate(n_outs):
        w, _ = _weight(410 + 7 * i + double_quant, n, N_IN)
        ws.append(w)
        qs.append(qlora.quantize(dev_f32(w), double_quant=double_quant))
        whs.append(oracle.dequantize(oracle.quantize(w, n, N_IN, double_quant=double_quant)))
    bits = workloads.to_bf16_bits
    bs = [dev_bf16(bits((rng.standard_normal((n, R)) * 0.01).astype(np.float32))) for n in n_outs]
    a_set = dev_bf16(bits((rng.standard_normal((2 * R, N_IN)) * 0.01).astype(np.float32)))
    cols = rng.permutation(N_IN)
    for part in range(N_IN // T):
        ks = cols[part * T:(part + 1) * T]
        ys, _ = qlora.linear_set_fwd(dev_bf16(_one_hot(T, N_IN, ks)), qs, dev_bf16(_zeros(2 * R, N_IN)), bs, 0.5)
        for i in range(2):
            assert np.array_equal(host_bits(ys[i]), whs[i][:, ks].T), ("forward", i, part)
    x = dev_bf16(bits(rng.standard_normal((T, N_IN)).astype(np.float32)))
    want = np.empty((T, N_IN), np.uint16)
    dys = []
    for i, n in enumerate(n_outs):
        d = np.zeros((T, n), np.float32)
        rows_i = np.arange(i, T, 2)  # member i owns rows of its parity
        ns = rng.integers(0, n, rows_i.size)
        d[rows_i, ns] = 1.0
        want[rows_i] = whs[i][ns, :]
        dys.append(dev_bf16(bits(d)))
    gx, _, _ = qlora.linear_set_bwd(dys, x, qs, a_set, [dev_bf16(_zeros(n, R)) for n in n_outs], 0.5)
    assert np.array_equal(host_bits(gx), want)
