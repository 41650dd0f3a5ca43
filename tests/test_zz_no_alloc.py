"""The forward without a workspace (qlora_linear_fwd_noalloc, for callers that cannot allocate)
against the forward with one (qlora_linear_fwd): the same kernels on the same inputs, so y and u
must be bit-identical, and both within the normwise bar of the fp64 oracle.  Two calls in a row
share the library's scratch array, the second on a smaller input (the few-token path), a third
goes back to the first shape, a fourth runs 12 tokens (the few-token forward above 4 tokens) and a
fifth 28 (its two tiles of 16 tokens)."""

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import NORMWISE_TOL, announce, bf16_to_f64, dev_bf16, dev_f32, host_bits, normwise_rel

pytestmark = pytest.mark.gpu


def _compare(case, save_u: bool):
    torch = __import__("torch")
    q = qlora.quantize(dev_f32(case.w))
    x, a, b = dev_bf16(case.x), dev_bf16(case.a), dev_bf16(case.b)
    T = case.tokens
    y_ref, u_ref = qlora.linear_fwd(x, q, a, b, case.scale)
    y = torch.empty((T, case.n_out), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((T, case.r), dtype=torch.bfloat16, device="cuda") if save_u else None
    torch.cuda.synchronize()
    qlora.linear_fwd_noalloc(x, q, a, b, case.scale, y, u_out=u)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y_ref)), "y differs from qlora_linear_fwd"
    if save_u:
        assert np.array_equal(host_bits(u), host_bits(u_ref)), "u differs from qlora_linear_fwd"
    wh = oracle.dequantize(oracle.quantize(case.w, case.n_out, case.n_in))
    y_o, u_o = oracle.forward(case.x, wh, case.a, case.b, case.scale)
    assert normwise_rel(bf16_to_f64(host_bits(y)), y_o) <= NORMWISE_TOL
    if save_u:
        assert normwise_rel(bf16_to_f64(host_bits(u)), u_o) <= NORMWISE_TOL


def test_noalloc_forward_matches_the_workspace_forward_on_consecutive_calls():
    big = workloads.custom_case(1024, 2048, 700, 32, 16.0, seed=71)
    small = workloads.custom_case(512, 1024, 3, 16, 16.0, seed=72)
    announce("noalloc fwd 1024x2048 T=700 r=32 (u saved)")
    _compare(big, save_u=True)
    announce("noalloc fwd 512x1024 T=3 r=16 (few-token, u not saved)")
    _compare(small, save_u=False)
    announce("noalloc fwd 1024x2048 T=700 r=32 again (u not saved)")
    _compare(big, save_u=False)
    announce("noalloc fwd 512x1024 T=12 r=16 (few-token forward, u saved)")
    _compare(workloads.custom_case(512, 1024, 12, 16, 16.0, seed=73), save_u=True)
    announce("noalloc fwd 512x1024 T=28 r=16 (few-token forward, two token tiles)")
    _compare(workloads.custom_case(512, 1024, 28, 16, 16.0, seed=74), save_u=False)


def test_noalloc_forward_7b_projection():
    announce("noalloc fwd 4096x4096 T=2048 r=64")
    _compare(workloads.attn7b_case(2048), save_u=True)
