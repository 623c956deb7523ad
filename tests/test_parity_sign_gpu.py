"""GPU parity of the 1-bit sign variant (the original BitNet weight binarization):
weights, sign bits, alpha and beta bit-exact; accumulators bit-exact; Y within 1e-5
relative per element. Through the C ABI, against the CPU oracle."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import workloads  # noqa: E402
from test_parity_gpu import DEV, assert_y_close, dev, host  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_quantized_linear_amd as m
    return m


def _check_weights(bl, W):
    c, alpha, gamma, beta = oracle.sign_weights(W)
    bits_o = oracle.pack1(c)
    bits, bg, ag = bl.quantize_weights_sign(dev(W))
    assert host(ag)[0] == alpha
    assert host(bg)[0] == beta
    assert np.array_equal(host(bits), bits_o)
    return bits, bg, bits_o, beta


@pytest.mark.parametrize("N,K,seed,shift", [(256, 1024, 0, 0.0), (256, 1024, 1, 0.004),
                                            (37, 72, 2, -0.01), (1, 8, 3, 0.0),
                                            (1024, 4096, 4, 0.001), (3, 4104, 5, 0.0),
                                            (5, 40, 6, 0.02)])
def test_sign_weights_parity(bl, N, K, seed, shift):
    # n % 32 != 0 for (37, 72), (1, 8), (3, 4104) and (5, 40): the tail bytes
    W = (workloads.weights(N, K, seed) + np.float32(shift)).astype(np.float32)
    for _ in range(2):
        _check_weights(bl, W)


@pytest.mark.parametrize("seed", range(2))
def test_sign_weights_exact_signed_sum(bl, seed):
    # signed magnitudes over ~250 binades: the mean needs the exact signed sum
    W = workloads.wide_range(64 * 4096, seed, lo_exp=-149, hi_exp=60).reshape(64, 4096)
    _check_weights(bl, W)


def test_sign_weights_special_cases(bl):
    cases = [np.zeros((4, 8), np.float32),               # alpha = 0: every code -1
             np.full((3, 16), 0.37, np.float32),          # every weight equals alpha
             np.array([[1, 2, 3, 6, 3, 3, 3, 3]], np.float32),
             np.array([[1, 2, 3, -6, 0.5, 0.5, -1, 0]], np.float32)]
    W = np.full((2, 32), -1e30, np.float32)               # cancellation to 0 exactly
    W[1] = 1e30
    cases.append(W)
    for W in cases:
        _check_weights(bl, W)


def _random_sign_inputs(T, N, K, seed):
    r = np.random.default_rng(seed)
    Xq = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    c = np.where(r.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    xs = r.uniform(1.0, 300.0, T).astype(np.float32)
    beta = np.float32(r.uniform(0.005, 0.05))
    return Xq, oracle.pack1(c), xs, beta


SIGN_CASES = [
    (1, 300, 4096),     # GEMV, 32 lanes per row
    (1, 64, 128),       # GEMV, one chunk per row
    (1, 130, 2048),     # GEMV, 16 lanes per row
    (1, 4096, 14336),   # GEMV, two segments per row
    (1, 611, 16384),    # GEMV, ragged N
    (1, 65, 32768),     # GEMV, four segments
    (1, 33, 65536),     # GEMV, two chunks per lane
    (1, 100, 1000),     # generic (K % 128 != 0)
    (3, 200, 4096),     # generic (T > 1)
    (17, 70, 1032),     # generic
]


@pytest.mark.parametrize("T,N,K", SIGN_CASES)
def test_sign_forward_parity(bl, T, N, K):
    Xq, P, xs, beta = _random_sign_inputs(T, N, K, T * 7 + N + K)
    acc_o = oracle.product_sign(Xq, P, K)
    Yg, accg = bl.forward_sign(dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)),
                               with_acc=True)
    assert np.array_equal(host(accg), acc_o), "T=%d N=%d K=%d" % (T, N, K)
    assert_y_close(host(Yg), oracle.rescale(acc_o, xs, beta), "sign")


@pytest.mark.parametrize("T,K", [(1, 28672), (2, 28672)])
def test_sign_extreme_accumulators(bl, T, K):
    N = 64
    Xq = np.full((T, K), 127, np.int8)
    Xq[1::2] = -128
    c = np.ones((N, K), np.int8)
    c[1::2] = -1
    P = oracle.pack1(c)
    xs = np.full(T, 3.0, np.float32)
    beta = np.float32(0.02)
    acc_o = oracle.product_sign(Xq, P, K)
    Yg, accg = bl.forward_sign(dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)),
                               with_acc=True)
    assert np.array_equal(host(accg), acc_o)
    assert np.abs(acc_o).max() >= 127 * K
    assert_y_close(host(Yg), oracle.rescale(acc_o, xs, beta), "sign extreme")


@pytest.mark.parametrize("seed", [0, 1])
def test_sign_tiny_end_to_end(bl, seed):
    N, K = workloads.TINY_W
    W = workloads.weights(N, K, seed)
    X = workloads.acts_normal(workloads.TINY_T, K, seed + 100)
    ref = oracle.bitlinear_sign(X, W)
    bits, beta, alpha = bl.quantize_weights_sign(dev(W))
    assert np.array_equal(host(bits), ref["packed"]) and host(alpha)[0] == ref["alpha"]
    Xq, xs = bl.quantize_acts(dev(X))
    Y, acc = bl.forward_sign(Xq, xs, bits, beta, with_acc=True)
    assert np.array_equal(host(acc), ref["acc"])
    assert_y_close(host(Y), ref["Y"], "sign tiny")
    Y1, acc1 = bl.forward_sign(Xq[:1].contiguous(), xs[:1].contiguous(), bits, beta, with_acc=True)
    assert np.array_equal(host(acc1), ref["acc"][:1])


def test_sign_decode8b_layer_grouped(bl):
    # one Llama-3-8B layer at T = 1 in the sign format, seven projections in one
    # grouped call (the launch the benchmark times); every output checked
    oracle.set_threads(0)
    Ws = workloads.decode8b_layer(0)
    inputs = workloads.decode8b_inputs(1, 100)
    entries, refs = [], []
    for name, ps in workloads.LLAMA3_8B_INPUTS.items():
        X = inputs[name]
        qo, so = oracle.quantize_acts(X)
        Xq, xs = bl.quantize_acts(dev(X))
        assert np.array_equal(host(Xq), qo)
        for p in ps:
            W = Ws[p]
            bits, bg, bits_o, beta = _check_weights(bl, W)
            N = W.shape[0]
            Y = torch.empty((1, N), dtype=torch.float32, device=DEV)
            acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
            entries.append((Xq, xs, bits, bg, Y, acc))
            refs.append((p, qo, so, bits_o, beta))
    bl.bitlinear_forward_sign_grouped(entries, 1)
    for (_, _, _, _, Y, acc), (p, qo, so, bits_o, beta) in zip(entries, refs):
        acc_o = oracle.product_sign(qo, bits_o, qo.shape[1])
        assert np.array_equal(host(acc), acc_o), p
        assert_y_close(host(Y), oracle.rescale(acc_o, so, beta), p)
