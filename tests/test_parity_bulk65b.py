"""The 65B bulk store checked, not only timed: layers 0, 40 and 79 of the 80-layer store (the
seven LLaMA-65B linear shapes per layer, W ~N(0, 0.02) drawn per layer from SeedSequence(5)),
quantized on the GPU, against the oracle regenerating the same layer from its seed.

For every tensor: the tensor mean of the block constants bit for bit; for 150 sampled FP8 groups
of 256 blocks per tensor (1,050 per layer, always including the last, possibly partial, group):
the packed codes, the FP8 bytes, the group scale and the decoded BF16 weights bit for bit.  The
bits per parameter come from the sizes of the buffers the store allocates: 4 + 1/8 + 1/512 +
32/numel ("qlora" entry, section "como funciona": 0.127 bit/param of constants after double
quantization).
"""

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_quant_amd import qlora, workloads
from helpers import announce, host, host_bits, oracle_blocks

pytestmark = pytest.mark.gpu

GROUPS_PER_TENSOR = 150


@pytest.mark.parametrize("layer", [0, 40, 79])
def test_bulk_store_layer(layer):
    torch = __import__("torch")
    rng = np.random.default_rng(5000 + layer)
    bits, params, groups = 0, 0, 0
    for name, w in workloads.bulk65b_layer_weights(layer):
        n, k = w.shape
        announce(f"65b bulk layer {layer} {name} {n}x{k}")
        q = qlora.quantize(torch.from_numpy(w).cuda())
        bits += 8 * q.nbytes()
        params += n * k
        flat = w.reshape(-1)
        c1 = oracle.block_absmax(flat)
        mu = oracle.exact_mean_f32(c1)
        assert host(q.absmax_mean).view(np.uint32)[0] == np.float32(mu).view(np.uint32), (name, "mean")
        nblocks = c1.size
        ngroups = -(-nblocks // 256)
        sel = np.unique(np.concatenate([rng.choice(ngroups - 1, GROUPS_PER_TENSOR - 1, replace=False),
                                        [ngroups - 1]]))
        groups += sel.size
        codes_d, fp8_d, s2_d = q.codes, q.absmax_fp8, q.absmax_scale
        wh_d = qlora.dequantize(q).reshape(-1)
        blocks = np.concatenate([np.arange(g * 256, min((g + 1) * 256, nblocks)) for g in sel])
        for g in sel:
            b0, b1 = g * 256, min((g + 1) * 256, nblocks)
            qg, s2g = oracle.double_quantize(c1[b0:b1], mu)
            seg = flat[b0 * 64:b1 * 64]
            want_codes = oracle.pack_codes(oracle.nearest_codes(seg, c1[b0:b1]).reshape(-1), seg.size)
            assert np.array_equal(host(codes_d[b0 * 32:b1 * 32]), want_codes), (name, int(g), "codes")
            assert np.array_equal(host(fp8_d[b0:b1]), qg), (name, int(g), "fp8")
            assert host(s2_d[g:g + 1]).view(np.uint32)[0] == s2g.view(np.uint32)[0], (name, int(g), "scale")
        idx = torch.from_numpy((blocks[:, None] * 64 + np.arange(64)).reshape(-1)).cuda()
        got = host_bits(wh_d[idx]).reshape(-1, 64)
        assert np.array_equal(got, oracle_blocks(flat, c1, mu, blocks)), (name, "decode")
        del q, wh_d
    assert groups >= 1000
    assert abs(bits / params - (4 + 1 / 8 + 1 / 512)) < 1e-6, bits / params
