"""Pins of the oracle's fp64 forward / backward of the QLoRA linear layer."""

import numpy as np

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_forward_equals_merged_weight_elementwise():
    """Y = x W'^T with the merged weight W' = W + s B A, written out with loops."""
    rng = np.random.default_rng(20)
    T, N, K, r, s = 3, 5, 7, 2, 0.75
    x, w, a, b = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r)
    y, u = oracle.forward_f64(x, w, a, b, s)
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                merged = w[n][k] + s * sum(b[n][j] * a[j][k] for j in range(r))
                acc += x[t][k] * merged
            assert abs(y[t][n] - acc) < 1e-12
    for t in range(T):
        for j in range(r):
            assert abs(u[t][j] - sum(x[t][k] * a[j][k] for k in range(K))) < 1e-12


def test_adapter_gradients_follow_the_chain_rule_through_the_merged_weight():
    rng = np.random.default_rng(21)
    T, N, K, r, s = 4, 6, 5, 3, 1.5
    x, w, a, b, dy = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r), _rand(rng, T, N)
    gx, ga, gb = oracle.backward_f64(dy, x, w, a, b, s)
    g_merged = np.zeros((N, K))  # dL/dW' for L = <dy, x W'^T>
    for t in range(T):
        for n in range(N):
            for k in range(K):
                g_merged[n][k] += dy[t][n] * x[t][k]
    merged = w + s * (b @ a)
    assert np.allclose(gx, dy @ merged, atol=1e-12)
    # W' = W + s B A: dL/dA = s B^T G, dL/dB = s G A^T
    assert np.allclose(ga, s * (b.T @ g_merged), atol=1e-12)
    assert np.allclose(gb, s * (g_merged @ a.T), atol=1e-12)


def test_adjoint_identities():
    rng = np.random.default_rng(22)
    T, N, K, r, s = 9, 11, 13, 4, 0.25
    x, w, a, b, dy = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r), _rand(rng, T, N)
    y, _ = oracle.forward_f64(x, w, a, b, s)
    gx, ga, gb = oracle.backward_f64(dy, x, w, a, b, s)
    lora = y - x @ w.T
    assert np.isclose(np.sum(gx * x), np.sum(dy * y), rtol=1e-12)
    assert np.isclose(np.sum(ga * a), np.sum(dy * lora), rtol=1e-12)
    assert np.isclose(np.sum(gb * b), np.sum(dy * lora), rtol=1e-12)


def test_central_finite_differences():
    rng = np.random.default_rng(23)
    T, N, K, r, s = 3, 4, 6, 2, 2.0
    x, w, a, b, dy = _rand(rng, T, K), _rand(rng, N, K), _rand(rng, r, K), _rand(rng, N, r), _rand(rng, T, N)
    gx, ga, gb = oracle.backward_f64(dy, x, w, a, b, s)

    def loss(x_, a_, b_):
        return float(np.sum(dy * oracle.forward_f64(x_, w, a_, b_, s)[0]))

    h = 1e-3
    for arr, grad, which in ((x, gx, 0), (a, ga, 1), (b, gb, 2)):
        for idx in np.ndindex(arr.shape):
            p = [x.copy(), a.copy(), b.copy()]
            m = [x.copy(), a.copy(), b.copy()]
            p[which][idx] += h
            m[which][idx] -= h
            fd = (loss(*p) - loss(*m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(grad[idx])), (which, idx)


def test_no_adapter_means_plain_product_and_zero_rows_stay_zero():
    rng = np.random.default_rng(24)
    x, w, a, b = _rand(rng, 5, 8), _rand(rng, 3, 8), np.zeros((2, 8)), _rand(rng, 3, 2)
    y, _ = oracle.forward_f64(x, w, a, b, 3.0)
    assert np.array_equal(y, x @ w.T + 0.0)
    x[2] = 0
    y, _ = oracle.forward_f64(x, w, _rand(rng, 2, 8), b, 3.0)
    assert np.all(y[2] == 0)


def test_bf16_entry_points_widen_exactly():
    rng = np.random.default_rng(25)
    from bit_quantized_finetuning_quant_amd import workloads

    x = workloads.to_bf16_bits(rng.standard_normal((2, 64)).astype(np.float32))
    w = workloads.to_bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    a = workloads.to_bf16_bits(rng.standard_normal((2, 64)).astype(np.float32))
    b = workloads.to_bf16_bits(rng.standard_normal((3, 2)).astype(np.float32))
    y, _ = oracle.forward(x, w, a, b, 0.5)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
    assert np.allclose(y - 0.5 * (xf @ oracle.bf16_bits_to_f32(a).astype(np.float64).T)
                       @ oracle.bf16_bits_to_f32(b).astype(np.float64).T, xf @ wf.T, atol=1e-9)
