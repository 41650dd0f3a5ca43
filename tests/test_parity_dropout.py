"""GPU parity of LoRA dropout: the mask (keep words and the masked input) bit-exact against
the oracle's Philox4x64-10 mask; the dropout forward and backward within the normwise bar of
the fp64 oracle on the fused GEMM path and on the few-token path; p = 0 identical to the plain
calls bit for bit."""

import numpy as np
import pytest

import oracle
from oracle import dropout as od
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import NORMWISE_TOL, announce, bf16_to_f64, dev_bf16, dev_f32, host, host_bits, normwise_rel

pytestmark = pytest.mark.gpu


def _words(keep):
    """bool [T x K] -> uint32 [ceil(T/32) x K], bit b of word [tb][k] = keep[32 tb + b, k]."""
    T, K = keep.shape
    tb = (T + 31) // 32
    pad = np.zeros((tb * 32, K), dtype=np.uint64)
    pad[:T] = keep
    w = np.zeros((tb, K), dtype=np.uint64)
    for b in range(32):
        w |= pad[b::32] << np.uint64(b)
    return w.astype(np.uint32)


@pytest.mark.parametrize("T,K,p,seed", [(1, 8, 0.05, 1), (31, 64, 0.05, 2), (33, 200, 0.5, 2**63 + 11),
                                        (100, 4096, 0.05, 12345), (64, 1024, 0.0, 7), (7, 336, 0.9, 0)])
def test_mask_bit_exact(T, K, p, seed):
    announce(f"dropout mask T={T} K={K} p={p} seed={seed}")
    x = workloads.to_bf16_bits(np.random.default_rng(T + K).standard_normal((T, K)).astype(np.float32))
    keep_w, xd = qlora.dropout_mask(dev_bf16(x), p, seed)
    keep = od.keep_mask(T, K, p, seed)
    assert np.array_equal(host(keep_w).view(np.uint32), _words(keep))
    want_xd = np.where(keep, x, np.uint16(0))
    assert np.array_equal(host_bits(xd), want_xd)


def _check(case, p, seed, need_u=True):
    torch = __import__("torch")
    s = case.scale
    q = qlora.quantize(dev_f32(case.w))
    wh = host_bits(qlora.dequantize(q))
    assert np.array_equal(wh, oracle.dequantize(oracle.quantize(case.w, case.n_out, case.n_in)))
    x, a, b, dy = dev_bf16(case.x), dev_bf16(case.a), dev_bf16(case.b), dev_bf16(case.dy)
    y, u = qlora.linear_fwd_dropout(x, q, a, b, s, p, seed)
    gx, ga, gb = qlora.linear_bwd_dropout(dy, x, q, a, b, s, p, seed, u=u if need_u else None)
    torch.cuda.synchronize()
    y_ref, u_ref = od.forward(case.x, wh, case.a, case.b, s, p, seed)
    gx_ref, ga_ref, gb_ref = od.backward(case.dy, case.x, wh, case.a, case.b, s, p, seed)
    errs = {"y": normwise_rel(bf16_to_f64(host_bits(y)), y_ref),
            "u": normwise_rel(bf16_to_f64(host_bits(u)), u_ref),
            "grad_x": normwise_rel(bf16_to_f64(host_bits(gx)), gx_ref),
            "grad_A": normwise_rel(host(ga), ga_ref),
            "grad_B": normwise_rel(host(gb), gb_ref)}
    for k, e in errs.items():
        assert e <= NORMWISE_TOL, (case.name, p, k, e)
    # the mask matters: without it the adapter gradients would be far from the reference
    if p >= 0.05:
        _, ga0, _ = oracle.backward(case.dy, case.x, wh, case.a, case.b, s)
        assert normwise_rel(host(ga), ga0) > 10 * errs["grad_A"]
    return errs


@pytest.mark.parametrize("shape", [(300, 320, 300, 24), (1000, 640, 513, 64), (77, 192, 259, 5), (256, 128, 17, 256),
                                   (512, 2048, 40, 16), (1024, 1024, 300, 64)])
def test_fused_gemm_path(shape):
    n_out, n_in, T, r = shape
    announce(f"dropout linear n_out={n_out} n_in={n_in} T={T} r={r}")
    case = workloads.custom_case(n_out, n_in, T, r, 16.0, seed=n_out + T + 7)
    _check(case, 0.05, seed=T * 1000 + r)
    _check(case, 0.3, seed=99, need_u=False)


@pytest.mark.parametrize("shape", [(300, 320, 1, 24), (77, 192, 2, 5), (130, 2112, 3, 13), (515, 4160, 4, 64),
                                   (300, 320, 8, 24), (515, 4160, 16, 64), (300, 320, 27, 24)])
def test_few_token_path(shape):
    n_out, n_in, T, r = shape
    announce(f"dropout few-token n_out={n_out} n_in={n_in} T={T} r={r}")
    case = workloads.custom_case(n_out, n_in, T, r, 16.0, seed=n_out + 5 * T)
    _check(case, 0.05, seed=5)
    _check(case, 0.5, seed=2**40 + 1, need_u=False)


@pytest.mark.parametrize("T", [200, 3])
def test_zero_probability_equals_the_plain_calls(T):
    """p = 0 keeps every element and the factor 1 / (1 - p) is exactly 1, so the dropout
    calls reproduce the plain calls bit for bit."""
    torch = __import__("torch")
    announce(f"dropout p=0 equals plain, T={T}")
    case = workloads.custom_case(320, 256, T, 16, 16.0, seed=31 + T)
    q = qlora.quantize(dev_f32(case.w))
    x, a, b, dy = dev_bf16(case.x), dev_bf16(case.a), dev_bf16(case.b), dev_bf16(case.dy)
    y0, u0 = qlora.linear_fwd(x, q, a, b, case.scale)
    g0 = qlora.linear_bwd(dy, x, q, a, b, case.scale, u=u0)
    y1, u1 = qlora.linear_fwd_dropout(x, q, a, b, case.scale, 0.0, 123)
    g1 = qlora.linear_bwd_dropout(dy, x, q, a, b, case.scale, 0.0, 123, u=u1)
    torch.cuda.synchronize()
    for t0, t1 in zip((y0, u0) + tuple(g0), (y1, u1) + tuple(g1)):
        assert np.array_equal(host(t0), host(t1))


def test_7b_projection_T2048_dropout():
    announce("dropout linear 7b_attn T=2048 p=0.05 full")
    errs = _check(workloads.attn7b_case(2048), 0.05, seed=2026)
    print("7b_attn T=2048 dropout normwise errors:", errs)
