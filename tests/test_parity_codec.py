"""GPU parity of the NF4 + FP8 codec: packed codes, FP8 constants, group scales, the mean and
the dequantized bf16 weight must equal the CPU oracle bit for bit."""

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import announce, dev_f32, dev_bf16, host, host_bits

pytestmark = pytest.mark.gpu


def _gpu_quantize(w, src="f32"):
    t = dev_f32(w) if src == "f32" else dev_bf16(w)
    q = qlora.quantize(t)
    assert qlora.status_read(q.last_workspace) == 0
    return q


def _compare_full(w, n_out, n_in, src="f32"):
    ref = oracle.quantize(w, n_out, n_in, src=src)
    q = _gpu_quantize(w.reshape(n_out, n_in), src)
    assert np.array_equal(host(q.codes), ref.codes), "codes"
    assert np.array_equal(host(q.absmax_fp8), ref.absmax_fp8), "fp8 constants"
    assert np.array_equal(host(q.absmax_scale).view(np.uint32), ref.absmax_scale.view(np.uint32)), "scales"
    assert host(q.absmax_mean).view(np.uint32)[0] == np.float32(ref.absmax_mean).view(np.uint32), "mean"
    wh = host_bits(qlora.dequantize(q))
    assert np.array_equal(wh, oracle.dequantize(ref)), "dequantized weight"
    return q, ref


def test_tiny_weight_bit_exact():
    announce("codec tiny 512x256 fp32")
    case = workloads.tiny_case()
    _compare_full(case.w, 512, 256)


@pytest.mark.parametrize("shape", [(37, 101), (1, 1), (1, 63), (3, 64), (129, 192), (5, 300)])
def test_crafted_and_ragged_weights_bit_exact(shape):
    n_out, n_in = shape
    announce(f"codec crafted {n_out}x{n_in}")
    if n_out * n_in >= 64:
        w = workloads.crafted_weight(7 + n_out, n_out, (n_in // 64) * 64 or n_in)
        full = np.random.default_rng(n_in).standard_normal((n_out, n_in)).astype(np.float32) * 0.02
        full[:, : w.shape[1]] = w
        w = full
    else:
        w = (np.random.default_rng(3).standard_normal((n_out, n_in)) * 0.02).astype(np.float32)
    _compare_full(w, n_out, n_in)


def test_crafted_block_kinds_bit_exact():
    announce("codec crafted 64x1024 (ties, zeros, outliers, subnormals)")
    w = workloads.crafted_weight(42, 64, 1024)
    q, ref = _compare_full(w, 64, 1024)
    codes = oracle.unpack_codes(ref.codes, w.size)
    assert (codes == 7).sum() > 0


def test_bf16_source_bit_exact():
    announce("codec bf16 source 256x512")
    w = workloads.to_bf16_bits((np.random.default_rng(5).standard_normal((256, 512)) * 0.02).astype(np.float32))
    _compare_full(w, 256, 512, src="bf16")


def test_all_zero_weight():
    announce("codec all-zero 16x128")
    q, ref = _compare_full(np.zeros((16, 128), np.float32), 16, 128)
    assert np.all(host(q.codes) == 0x77)


def test_nonfinite_weight_is_flagged():
    announce("codec NaN flag")
    w = np.ones((4, 64), np.float32)
    w[2, 5] = np.nan
    q = qlora.quantize(dev_f32(w))
    assert qlora.status_read(q.last_workspace) == 7
    w[2, 5] = 1.0
    q = qlora.quantize(dev_f32(w))
    assert qlora.status_read(q.last_workspace) == 0


def test_7b_projection_weight_bit_exact():
    """4096 x 4096 ~N(0, 0.02) fp32 (the 7B attention projection), every byte compared."""
    announce("codec 7b_attn 4096x4096")
    case = workloads.attn7b_case(tokens=1)
    _compare_full(case.w, 4096, 4096)


def test_65b_down_projection_sampled_groups():
    """8192 x 22016 Student-t weight with outliers (a 65B decoder linear): mean exact, and the codes,
    FP8 constants, scales and decoded weights of 64 randomly chosen DQ groups bit-exact."""
    announce("codec 65b down 8192x22016 sampled")
    case = next(workloads.layer65b_cases(tokens=8, shapes=[("down", 8192, 22016)]))
    w = case.w
    q = _gpu_quantize(w)
    flat = w.reshape(-1)
    c1 = oracle.block_absmax(flat)
    mu = oracle.exact_mean_f32(c1)
    assert host(q.absmax_mean).view(np.uint32)[0] == np.float32(mu).view(np.uint32)
    wh = qlora.dequantize(q)
    g_codes, g_fp8, g_s2 = host(q.codes), host(q.absmax_fp8), host(q.absmax_scale)
    rng = np.random.default_rng(99)
    ngroups = g_s2.size
    for g in sorted(set(rng.integers(0, ngroups, 64).tolist()) | {0, ngroups - 1}):
        b0, b1 = g * 256, min((g + 1) * 256, c1.size)
        qg, s2g = oracle.double_quantize(c1[b0:b1], mu)
        assert g_s2[g].view(np.uint32) == s2g[0].view(np.uint32)
        assert np.array_equal(g_fp8[b0:b1], qg)
        seg = flat[b0 * 64: b1 * 64]
        codes = oracle.nearest_codes(seg, c1[b0:b1]).reshape(-1)
        assert np.array_equal(g_codes[b0 * 32: b1 * 32], oracle.pack_codes(codes, seg.size))
        ref = oracle.NF4Quantized(1, seg.size, oracle.pack_codes(codes, seg.size), qg, s2g, mu, c1[b0:b1])
        got = host_bits(wh.reshape(-1)[b0 * 64: b1 * 64])
        assert np.array_equal(got, oracle.dequantize(ref).reshape(-1))


def test_quantize_is_deterministic():
    announce("codec determinism")
    w = workloads.crafted_weight(8, 128, 512)
    q1 = _gpu_quantize(w)
    q2 = _gpu_quantize(w)
    for a, b in ((q1.codes, q2.codes), (q1.absmax_fp8, q2.absmax_fp8), (q1.absmax_scale, q2.absmax_scale)):
        assert np.array_equal(host(a), host(b))


def test_dequantize_many_bit_exact():
    """Several weights of mixed shapes and both storage forms decoded in one launch equal the
    oracle's decode of each."""
    announce("codec dequantize_many (5 weights, ragged, mixed storage forms)")
    shapes = [(37, 101), (64, 1024), (1, 63), (129, 192), (300, 320)]
    rng = np.random.default_rng(77)
    ws = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    forms = [True, False, True, False, True]
    qs = [qlora.quantize(dev_f32(w), double_quant=dq) for w, dq in zip(ws, forms)]
    outs = qlora.dequantize_many(qs)
    for w, dq, o, (n, k) in zip(ws, forms, outs, shapes):
        ref = oracle.quantize(w, n, k, double_quant=dq)
        assert np.array_equal(host_bits(o), oracle.dequantize(ref)), (n, k, dq)


def test_dequantize_many_65b_layer_sampled():
    """The seven 65B linears of one layer in one launch, each checked against the single-weight
    call bit for bit (the single call is checked against the oracle elsewhere)."""
    torch = __import__("torch")
    announce("codec dequantize_many 65B layer (7 weights)")
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    qs = []
    for _, n, k in workloads.SHAPES_65B:
        w = torch.empty((n, k), dtype=torch.float32, device="cuda").normal_(0.0, 0.02, generator=g)
        qs.append(qlora.quantize(w))
        del w
    outs = qlora.dequantize_many(qs)
    for q, o in zip(qs, outs):
        single = qlora.dequantize(q)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int16), o.view(torch.int16))
        del single
