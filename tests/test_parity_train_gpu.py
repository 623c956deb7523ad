"""GPU parity of the training side: fake quantization with the warm-up lambda (bf16
outputs bit-exact against the oracle's fp32 steps and bf16 rounding), the RMSNorm
factor r bit-exact, and the straight-through RMSNorm backward within a tolerance
derived from its fp64 arithmetic."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import workloads  # noqa: E402
from test_parity_gpu import dev, host  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_quantized_linear_amd as m
    return m


def bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


@pytest.mark.parametrize("N,K,lam", [(256, 1024, 0.0), (256, 1024, 0.37), (256, 1024, 1.0),
                                     (37, 68, 0.5), (1024, 4096, 0.01), (3, 4100, 1.0)])
def test_fake_quant_weights(bl, N, K, lam):
    W = workloads.weights(N, K, N + K)
    ref = oracle.fake_quant_weights(W, lam)
    Wg = dev(W)
    _, beta = bl.quantize_weights(Wg)
    out = bl.fake_quant_weights(Wg, beta, lam)
    assert np.array_equal(bits(out), ref)


def test_fake_quant_weights_special(bl):
    for W in (np.zeros((2, 8), np.float32), np.full((2, 8), 1e-40, np.float32),
              np.array([[1, 3, -1, -3], [2, 2, 2, 2]], np.float32)):
        ref = oracle.fake_quant_weights(W, 0.5)
        Wg = dev(W)
        _, beta = bl.quantize_weights(Wg)
        assert np.array_equal(bits(bl.fake_quant_weights(Wg, beta, 0.5)), ref)


@pytest.mark.parametrize("T,K,lam,gain,flags", [(1, 4096, 0.5, False, 0), (8, 1024, 1.0, True, 0),
                                                (70, 4100, 0.25, False, 0), (2, 40000, 0.7, True, 0),
                                                (3, 1024, 0.5, False, 1), (130, 2048, 0.0, True, 0)])
def test_fake_quant_acts(bl, T, K, lam, gain, flags):
    X = workloads.acts_normal(T, K, T + K)
    g = np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32) if gain else None
    ref, qo, so, ro = oracle.fake_quant_acts(X, g, 1e-6, flags, lam)
    out, Xq, xs, r = bl.fake_quant_acts(dev(X), lam, None if g is None else dev(g), 1e-6, flags)
    assert np.array_equal(host(Xq), qo) and np.array_equal(host(xs), so)
    assert np.array_equal(host(r), ro)
    assert np.array_equal(bits(out), ref)


@pytest.mark.parametrize("T,K,gain", [(1, 4096, False), (16, 4096, True), (70, 4100, True),
                                      (3, 40000, False)])
def test_rmsnorm_backward(bl, T, K, gain):
    X = workloads.acts_normal(T, K, 7 + T)
    dY = workloads.acts_normal(T, K, 9 + K)
    g = np.random.default_rng(3).uniform(0.5, 1.5, K).astype(np.float32) if gain else None
    _, _, _, r = bl.fake_quant_acts(dev(X), 0.5, None if g is None else dev(g))
    ro = oracle.rms_inv(X)
    assert np.array_equal(host(r), ro)
    dX_o, dg_o = oracle.rmsnorm_backward(X, g, ro, dY)
    dX, dg = bl.rmsnorm_backward(dev(X), r, dev(dY), None if g is None else dev(g))
    # two terms computed in fp64 from the same inputs, summed in a different order:
    # the difference is a few fp64 roundings of the terms, then one fp32 rounding
    gg = np.ones(K) if g is None else g.astype(np.float64)
    t1 = np.abs(ro[:, None] * gg[None, :] * dY.astype(np.float64))
    c = np.abs(gg[None, :] * dY.astype(np.float64) * X.astype(np.float64)).sum(1)
    t2 = np.abs(X.astype(np.float64)) * (ro ** 3 * c / K)[:, None]
    tol = 2.0 ** -23 * np.abs(dX_o.astype(np.float64)) + 1e-12 * (t1 + t2)
    assert np.all(np.abs(host(dX).astype(np.float64) - dX_o.astype(np.float64)) <= tol)
    if gain:
        sc = (np.abs(dY.astype(np.float64) * X.astype(np.float64)) * ro[:, None]).sum(0)
        tolg = 2.0 ** -23 * np.abs(dg_o.astype(np.float64)) + 1e-12 * sc
        assert np.all(np.abs(host(dg).astype(np.float64) - dg_o.astype(np.float64)) <= tolg)
