"""The library's calls under HIP graph capture: a captured fwd + bwd step replayed several times,
with new inputs copied in and eager work between the replays, equals the eager calls bit for bit
(the kernels are deterministic and allocate nothing; no call records a memset)."""

import numpy as np
import pytest

from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import announce, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,N,K", [(1, 512, 320), (3, 512, 320), (300, 512, 320), (40, 512, 2048)])
def test_captured_step_replays_equal_eager(T, N, K):
    """T = 40 at 512 x 2048 splits the contraction of both fused GEMMs (a reduction kernel after
    each), and its 40 rows run clamped in a 256-row tile."""
    torch = __import__("torch")
    announce(f"graph capture fwd+bwd {N}x{K} T={T} r=16")
    case = workloads.custom_case(N, K, T, 16, 16.0, seed=50 + T)
    q = qlora.quantize(dev_f32(case.w))
    a, b = dev_bf16(case.a), dev_bf16(case.b)
    x, dy = dev_bf16(case.x), dev_bf16(case.dy)
    bf, f32 = torch.bfloat16, torch.float32
    y = torch.empty((T, N), dtype=bf, device="cuda")
    u = torch.empty((T, 16), dtype=bf, device="cuda")
    gx = torch.empty((T, K), dtype=bf, device="cuda")
    ga = torch.empty((16, K), dtype=f32, device="cuda")
    gb = torch.empty((N, 16), dtype=f32, device="cuda")
    ws = qlora.linear_workspace(T, N, K, 16)

    def step():
        qlora.linear_fwd(x, q, a, b, case.scale, y=y, u_out=u, workspace=ws)
        qlora.linear_bwd(dy, x, q, a, b, case.scale, u=u, grad_x=gx, grad_A=ga, grad_B=gb, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(T)
    for rep in range(3):
        xs = workloads.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
        dys = workloads.to_bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
        x.copy_(dev_bf16(xs))
        dy.copy_(dev_bf16(dys))
        g.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in (y, u, gx, ga, gb)]
        step()  # eager, same inputs
        torch.cuda.synchronize()
        want = [host(t) for t in (y, u, gx, ga, gb)]
        for i, (gv, wv) in enumerate(zip(got, want)):
            assert np.array_equal(gv, wv), (rep, i)
        torch.zeros(1000, device="cuda").add_(1.0)  # unrelated eager work between replays
