"""Shared helpers of the GPU parity tests (host <-> device marshalling, error norms)."""

import sys

import numpy as np

import oracle


def torch_mod():
    import torch

    return torch


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says what it was doing."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev_f32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns -> CUDA bfloat16 tensor with the same bits."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def host_bits(t) -> np.ndarray:
    """CUDA bf16 tensor -> uint16 numpy bits."""
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t) -> np.ndarray:
    """CUDA tensor -> numpy (bf16 tensors come back as their uint16 bit patterns)."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return host_bits(t)
    return t.detach().cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def normwise_rel(got: np.ndarray, want: np.ndarray) -> float:
    want = np.asarray(want, np.float64)
    num = np.linalg.norm(np.asarray(got, np.float64) - want)
    den = np.linalg.norm(want)
    return float(num / den) if den > 0 else float(num)


# The bar for floating-point outputs of the linear layer: normwise relative
# error against the fp64 evaluation on the dequantized weight.
NORMWISE_TOL = 1e-2


def oracle_blocks(flat: np.ndarray, c1: np.ndarray, mu, blocks: np.ndarray) -> np.ndarray:
    """bf16 bits [len(blocks), 64] of the given NF4 blocks, from the oracle's own quantization."""
    blocks = np.asarray(blocks, dtype=np.int64)
    out = np.empty((blocks.size, 64), dtype=np.uint16)
    order = np.argsort(blocks, kind="stable")
    sb = blocks[order]
    groups = sb // 256
    bounds = np.flatnonzero(np.diff(groups)) + 1
    for part, idx in zip(np.split(sb, bounds), np.split(order, bounds)):
        g = int(part[0] // 256)
        b0, b1 = g * 256, min((g + 1) * 256, c1.size)
        qg, s2g = oracle.double_quantize(c1[b0:b1], mu)
        seg = flat[(part[:, None] * 64 + np.arange(64)).reshape(-1)]
        codes = oracle.nearest_codes(seg, c1[part]).reshape(-1)
        ref = oracle.NF4Quantized(1, seg.size, oracle.pack_codes(codes, seg.size), qg[part - b0], s2g, mu, c1[part])
        out[idx] = oracle.dequantize(ref).reshape(-1, 64)
    return out
