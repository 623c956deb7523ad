"""GPU parity of BitDelta (a base matrix plus B per-model 1-bit deltas): the batched sign
bits and the per-model scales bit-exact; the forward within a tolerance derived from the
rounding count of its fp32 arithmetic (the oracle sums in fp64), and the same bits on a
second call."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from test_parity_gpu import dev, host  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_quantized_linear_amd as m
    return m


def _models(N, M, B, seed):
    # a base model and B fine-tunes of it (small deltas, some exactly zero)
    r = np.random.default_rng(seed)
    base = oracle.bf16_bits((r.standard_normal((N, M)) * 0.02).astype(np.float32))
    fines = []
    for i in range(B):
        d = (r.standard_normal((N, M)) * 0.001).astype(np.float32)
        d[r.random((N, M)) < 0.05] = 0.0
        fines.append((oracle.bf16_to_f32(base) + d).astype(np.float32))
    return base, fines


def _check_forward(bl, base, fines, seed):
    B = len(fines)
    N, M = base.shape
    refs = [oracle.bitdelta_compress(f, base) for f in fines]
    Dg, ag = bl.bitdelta_compress([dev(f) for f in fines], dev(base.view(np.int16)).view(torch.bfloat16))
    assert np.array_equal(host(Dg), oracle.bitdelta_interleave([r[0] for r in refs]))
    assert np.array_equal(host(ag), np.array([r[1] for r in refs], np.float32))
    X = np.random.default_rng(seed).standard_normal((B, M)).astype(np.float32)
    Y_o = oracle.bitdelta_forward(base, [r[2] for r in refs], [r[1] for r in refs], X)
    Yg = host(bl.bitdelta_forward(dev(base.view(np.int16)).view(torch.bfloat16), Dg, ag, dev(X)))
    # Rounding count of the kernel's fp32 arithmetic, per term of the sum (u = 2^-24):
    #   base term w*x: 16 chained FMAs in the lane, the add of the delta part, 6 levels
    #   of the wave's DPP tree, up to 7 adds over the waves: at most 30 roundings;
    #   delta term x: 15 adds into P (and into sum x), 2P - sum x, the product by alpha,
    #   the add to the base part, the 6 + 7 adds above: at most 31 roundings.
    # So |Y_gpu - Y_exact| <= gamma_31 * (sum |w x| + alpha * (2 sum_sel |x| + sum |x|)),
    # gamma_31 = 31u / (1 - 31u), and the oracle's one fp32 rounding of its fp64 result
    # adds u |Y|: 33u * mag with mag = sum |w x| + 3 alpha sum |x| covers both.
    bf = np.abs(oracle.bf16_to_f32(base).astype(np.float64))
    mag = np.abs(X.astype(np.float64)) @ bf.T + \
        np.array([float(r[1]) for r in refs])[:, None] * 3 * np.abs(X.astype(np.float64)).sum(1)[:, None]
    assert np.all(np.abs(Yg.astype(np.float64) - Y_o.astype(np.float64)) <= 33 * 2.0 ** -24 * mag)
    # the wave partials meet in a fixed order: a second call gives the same bits
    Yg2 = host(bl.bitdelta_forward(dev(base.view(np.int16)).view(torch.bfloat16), Dg, ag, dev(X)))
    assert np.array_equal(Yg.view(np.uint32), Yg2.view(np.uint32))
    return Yg, Y_o


@pytest.mark.parametrize("N,M,B", [(64, 1024, 8), (100, 8192, 8), (37, 208, 3), (513, 4096, 1),
                                   (300, 1040, 5)])
def test_bitdelta_parity(bl, N, M, B):
    base, fines = _models(N, M, B, N + M + B)
    _check_forward(bl, base, fines, 7)


def test_bitdelta_full_size(bl):
    # the Figure 4 shape: N = M = 8192, B = 8
    oracle.set_threads(0)
    base, fines = _models(8192, 8192, 8, 1)
    _check_forward(bl, base, fines, 2)


def test_bitdelta_zero_delta_is_base(bl):
    # fine == base: every delta is 0 -> codes -1, alpha 0, Y = base product exactly
    r = np.random.default_rng(4)
    base = oracle.bf16_bits((r.standard_normal((16, 256)) * 0.02).astype(np.float32))
    fines = [oracle.bf16_to_f32(base).copy() for _ in range(2)]
    Dg, ag = bl.bitdelta_compress([dev(f) for f in fines], dev(base.view(np.int16)).view(torch.bfloat16))
    assert np.all(host(ag) == 0.0) and np.all(host(Dg) == 0)
