"""GPU parity of projection sets (linears sharing their input, run as one fused GEMM per
direction): every member's y, the summed grad_x, grad_A_set and every grad_B against the fp64
oracle within the normwise bar; a one-member set bit-identical to the single-linear calls."""

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import NORMWISE_TOL, announce, bf16_to_f64, dev_bf16, dev_f32, host, host_bits, normwise_rel

pytestmark = pytest.mark.gpu


def _members(n_outs, n_in, T, r, seed):
    cases = [workloads.custom_case(n, n_in, T, r, 16.0, seed=seed + 17 * i) for i, n in enumerate(n_outs)]
    x = cases[0].x
    for c in cases:
        c.x = x
    return cases


def _run_set(cases, need_u=True, double_quant=True):
    torch = __import__("torch")
    s = cases[0].scale
    qs = [qlora.quantize(dev_f32(c.w), double_quant=double_quant) for c in cases]
    x = dev_bf16(cases[0].x)
    a_set = dev_bf16(np.concatenate([c.a for c in cases], axis=0))
    bs = [dev_bf16(c.b) for c in cases]
    dys = [dev_bf16(c.dy) for c in cases]
    ys, u = qlora.linear_set_fwd(x, qs, a_set, bs, s)
    gx, ga, gbs = qlora.linear_set_bwd(dys, x, qs, a_set, bs, s, u=u if need_u else None)
    torch.cuda.synchronize()
    return qs, ys, u, gx, ga, gbs


def _check(cases, need_u=True, double_quant=True):
    s = cases[0].scale
    qs, ys, u, gx, ga, gbs = _run_set(cases, need_u, double_quant)
    r = cases[0].a.shape[0]
    gx_ref = 0.0
    errs = {}
    for i, (c, q) in enumerate(zip(cases, qs)):
        ref = oracle.quantize(c.w, c.n_out, c.n_in, double_quant=double_quant)
        wh = oracle.dequantize(ref)
        assert np.array_equal(host_bits(qlora.dequantize(q)), wh)
        y_ref, u_ref = oracle.forward(c.x, wh, c.a, c.b, s)
        g = oracle.backward(c.dy, c.x, wh, c.a, c.b, s)
        gx_ref = gx_ref + g[0]
        errs[f"y{i}"] = normwise_rel(bf16_to_f64(host_bits(ys[i])), y_ref)
        errs[f"u{i}"] = normwise_rel(bf16_to_f64(host_bits(u))[:, i * r:(i + 1) * r], u_ref)
        errs[f"grad_A{i}"] = normwise_rel(host(ga)[i * r:(i + 1) * r], g[1])
        errs[f"grad_B{i}"] = normwise_rel(host(gbs[i]), g[2])
    errs["grad_x"] = normwise_rel(bf16_to_f64(host_bits(gx)), gx_ref)
    for k, e in errs.items():
        assert e <= NORMWISE_TOL, (k, e)
    return errs


@pytest.mark.parametrize("n_outs,n_in,T,r", [((320, 192, 256), 320, 300, 24), ((77, 130, 64), 192, 259, 5),
                                             ((1000, 640), 640, 513, 64), ((128, 128, 128, 128), 128, 17, 16),
                                             ((64, 128), 128, 40, 4), ((256, 128), 256, 256, 96),
                                             ((512, 512, 512), 1024, 40, 16), ((1000, 700, 1300), 896, 2050, 24),
                                             ((1024, 512, 768), 2048, 300, 32)])
def test_sets_against_the_oracle(n_outs, n_in, T, r):
    announce(f"set n_outs={n_outs} n_in={n_in} T={T} r={r}")
    cases = _members(n_outs, n_in, T, r, seed=T + r)
    _check(cases)
    _check(cases, need_u=False)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8, 16, 29])
def test_few_token_sets_against_the_oracle(T):
    """T <= 4: the few-token kernels run a set of several members (the forward over the
    concatenated rows, the backward over every member's rows and adapter blocks in one pass); at 8,
    16 and 29 tokens (two token tiles) the forward still, the backward on the fused GEMM; same
    layouts, same bar."""
    announce(f"few-token set n_outs=(256, 192, 320) n_in=384 T={T} r=16")
    cases = _members((256, 192, 320), 384, T, 16, seed=40 + T)
    _check(cases)
    _check(cases, need_u=False)


@pytest.mark.parametrize("T", [1, 3])
def test_few_token_set_backward_without_grad_x(T):
    """Skipping grad_x leaves only the adapter workgroups: grad_A_set and every grad_B are the
    same bits as in the call that also produces grad_x, and within the bar of the oracle."""
    announce(f"few-token set without grad_x n_outs=(192, 256, 128) n_in=256 T={T} r=32")
    cases = _members((192, 256, 128), 256, T, 32, seed=90 + T)
    qs, ys, u, gx, ga, gbs = _run_set(cases)
    s = cases[0].scale
    x = dev_bf16(cases[0].x)
    a_set = dev_bf16(np.concatenate([c.a for c in cases], axis=0))
    bs = [dev_bf16(c.b) for c in cases]
    dys = [dev_bf16(c.dy) for c in cases]
    gx2, ga2, gbs2 = qlora.linear_set_bwd(dys, x, qs, a_set, bs, s, u=u, need_grad_x=False)
    __import__("torch").cuda.synchronize()
    assert gx2 is None
    assert np.array_equal(host(ga2), host(ga))
    for g2, g in zip(gbs2, gbs):
        assert np.array_equal(host(g2), host(g))
    r = 32
    for i, c in enumerate(cases):
        wh = oracle.dequantize(oracle.quantize(c.w, c.n_out, c.n_in))
        g = oracle.backward(c.dy, c.x, wh, c.a, c.b, s)
        assert normwise_rel(host(ga2)[i * r:(i + 1) * r], g[1]) <= NORMWISE_TOL
        assert normwise_rel(host(gbs2[i]), g[2]) <= NORMWISE_TOL


@pytest.mark.parametrize("T", [2, 10])
def test_few_token_set_with_unaligned_member(T):
    """A member other than the last with a row count that is not a multiple of 64: the forward runs
    member by member on the few-token kernels, the backward still as one pass (T = 2) or on the
    fused GEMM (T = 10)."""
    announce(f"few-token set n_outs=(300, 256) n_in=256 T={T} r=8")
    cases = _members((300, 256), 256, T, 8, seed=76 + T)
    _check(cases)
    _check(cases, need_u=False)


def test_few_token_set_of_four_members_rank_256():
    announce("few-token set n_outs=(128, 64, 192, 128) n_in=256 T=4 r=256")
    cases = _members((128, 64, 192, 128), 256, 4, 256, seed=77)
    _check(cases)
    _check(cases, need_u=False)


def test_few_token_one_member_set_equals_the_single_linear_calls():
    torch = __import__("torch")
    announce("few-token set of one member vs single linear, 300x320 T=3 r=24")
    (c,) = _members((300,), 320, 3, 24, seed=12)
    q = qlora.quantize(dev_f32(c.w))
    x, a, b, dy = dev_bf16(c.x), dev_bf16(c.a), dev_bf16(c.b), dev_bf16(c.dy)
    y0, u0 = qlora.linear_fwd(x, q, a, b, c.scale)
    g0 = qlora.linear_bwd(dy, x, q, a, b, c.scale, u=u0)
    (y1,), u1 = qlora.linear_set_fwd(x, [q], a, [b], c.scale)
    g1x, g1a, (g1b,) = qlora.linear_set_bwd([dy], x, [q], a, [b], c.scale, u=u1)
    torch.cuda.synchronize()
    for t0, t1 in zip((y0, u0) + tuple(g0), (y1, u1, g1x, g1a, g1b)):
        assert np.array_equal(host(t0), host(t1))


def test_set_with_fp32_constants():
    announce("set fp32 constants n_outs=(256, 320) n_in=256 T=130 r=8")
    _check(_members((256, 320), 256, 130, 8, seed=5), double_quant=False)


@pytest.mark.parametrize("n_out,n_in,T,r", [(300, 320, 200, 24), (2048, 2048, 256, 64), (1024, 4096, 64, 16)])
def test_one_member_set_equals_the_single_linear_calls(n_out, n_in, T, r):
    """A one-member set runs the single linear's kernels, splits included (the second shape splits
    the contraction of both directions on 256-row tiles, the third on the few-token tiles), so
    every output is bit-identical."""
    torch = __import__("torch")
    announce(f"set of one member vs single linear, {n_out}x{n_in} T={T} r={r}")
    (c,) = _members((n_out,), n_in, T, r, seed=11 + T)
    q = qlora.quantize(dev_f32(c.w))
    x, a, b, dy = dev_bf16(c.x), dev_bf16(c.a), dev_bf16(c.b), dev_bf16(c.dy)
    y0, u0 = qlora.linear_fwd(x, q, a, b, c.scale)
    g0 = qlora.linear_bwd(dy, x, q, a, b, c.scale, u=u0)
    (y1,), u1 = qlora.linear_set_fwd(x, [q], a, [b], c.scale)
    g1x, g1a, (g1b,) = qlora.linear_set_bwd([dy], x, [q], a, [b], c.scale, u=u1)
    torch.cuda.synchronize()
    for t0, t1 in zip((y0, u0) + tuple(g0), (y1, u1, g1x, g1a, g1b)):
        assert np.array_equal(host(t0), host(t1))


@pytest.mark.parametrize("n_outs,n_in,T,r", [((4096, 4096), 8192, 48, 32), ((4096, 4096), 8192, 16, 32),
                                             ((4096, 4096), 8192, 24, 32), ((4096, 8192), 4096, 40, 24)])
def test_few_token_set_member_by_member(n_outs, n_in, T, r):
    """Sets at a few tokens whose members are large enough that the split cost models run them
    member by member on the few-token tiles: the first shape in both directions (forward: each
    member with its own split and reduction, the adapter term from its columns of u_set; grad_x:
    every member's splits as fp32 partial tiles, its share of s v_set A_set in its first split,
    one reduction over all of them), the second and third the same grad_x after a forward on the
    few-token kernels (one and two tiles of 16 tokens), the fourth in the forward only (members of
    different widths, 40 tokens: clamped rows, rank 24); against the oracle."""
    announce(f"set {n_outs} x {n_in} T={T} r={r} (member by member)")
    _check(_members(n_outs, n_in, T, r, seed=41 + T))


@pytest.mark.parametrize("T", [3, 4])
def test_large_set_at_three_and_four_tokens(T):
    """Two 8192 x 8192 members (134 M weights in all): the backward on the few-token pass at 3
    tokens and on the fused GEMM at 4 (sets above 128 M weights), against the oracle."""
    announce(f"set (8192, 8192) x 8192 T={T} r=16")
    _check(_members((8192, 8192), 8192, T, 16, seed=90 + T))


def test_7b_attention_projections_T2048():
    """q, k, v of LLaMA-7B (3 x 4096 x 4096, r = 64, 2048 tokens) as one set, in full."""
    announce("set 7b q/k/v T=2048 full")
    errs = _check(_members((4096, 4096, 4096), 4096, 2048, 64, seed=2))
    print("7b q/k/v set normwise errors:", errs)


def test_7b_gate_up_T512():
    announce("set 7b gate/up T=512 full")
    errs = _check(_members((11008, 11008), 4096, 512, 64, seed=3))
    print("7b gate/up set normwise errors:", errs)
