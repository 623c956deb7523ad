"""GPU parity of group quantization (weights in G blocks of N/G output rows, each with
its own absmean scale): packed bytes, per-block beta and gamma bit-exact; accumulators
bit-exact; Y within 1e-5 relative per element, on every product kernel."""
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


def _grouped_weights(N, K, G, seed):
    # blocks of rows with scales a decade apart, so that one scale would not fit all
    r = np.random.default_rng(seed)
    W = workloads.weights(N, K, seed)
    return (W * np.repeat(np.float32(10.0) ** r.uniform(-1, 1, G), N // G)[:, None]
            ).astype(np.float32)


@pytest.mark.parametrize("N,K,G", [(256, 1024, 1), (256, 1024, 8), (36, 68, 4), (4096, 4096, 8),
                                   (14336, 4096, 8), (6, 4, 6)])
def test_scale_groups_quantizer(bl, N, K, G):
    W = _grouped_weights(N, K, G, N + G)
    P, beta, gamma = oracle.quantize_weights_groups(W, G)
    Pg, bg, gg = bl.quantize_weights_scale_groups(dev(W), G, with_gamma=True)
    assert np.array_equal(host(gg), gamma)
    assert np.array_equal(host(bg), beta)
    assert np.array_equal(host(Pg), P)


CASES = [("gemv", 1, 512, 4096, 8), ("gemv", 1, 300, 4096, 3), ("gemv", 1, 96, 1024, 32),
         ("gemv", 1, 4096, 14336, 8), ("skinny", 5, 512, 4096, 8), ("skinny", 16, 96, 1024, 12),
         ("skinny", 32, 200, 8192, 5), ("prefill", 70, 512, 4096, 8), ("prefill", 300, 300, 1024, 3),
         ("prefill", 130, 96, 1024, 48), ("prefill", 130, 33000, 256, 125),
         ("prefill", 300, 49140, 256, 195), ("prefill", 40, 12288, 4096, 96),
         ("generic", 3, 100, 1028, 4),
         ("auto", 1, 1024, 4096, 1)]


@pytest.mark.parametrize("kernel,T,N,K,G", CASES)
def test_scale_groups_forward(bl, kernel, T, N, K, G):
    r = np.random.default_rng(T + N + K + G)
    Xq = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    q = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    P = oracle.pack(q)
    xs = r.uniform(1.0, 300.0, T).astype(np.float32)
    beta = r.uniform(0.005, 0.05, G).astype(np.float32)
    acc_o = oracle.product(Xq, P, K)
    Y_o = oracle.rescale_groups(acc_o, xs, beta)
    Y, acc = bl.forward_scale_groups(dev(Xq), dev(xs), dev(P), dev(beta), with_acc=True,
                                     kernel=kernel)
    assert np.array_equal(host(acc), acc_o), "%s T=%d N=%d K=%d G=%d" % (kernel, T, N, K, G)
    assert_y_close(host(Y), Y_o, "%s G=%d" % (kernel, G))


def test_scale_groups_end_to_end_and_grouped_call(bl):
    # fp32 W and X through the whole path; and a grouped launch of three projections
    # with different G
    N, K, G = 512, 1024, 8
    W = _grouped_weights(N, K, G, 3)
    X = workloads.acts_normal(4, K, 4)
    ref = oracle.bitlinear_groups(X, W, G)
    Pg, bg = bl.quantize_weights_scale_groups(dev(W), G)
    Xq, xs = bl.quantize_acts(dev(X))
    for k in ("skinny", "prefill", "generic"):
        Y, acc = bl.forward_scale_groups(Xq, xs, Pg, bg, with_acc=True, kernel=k)
        assert np.array_equal(host(acc), ref["acc"]), k
        assert_y_close(host(Y), ref["Y"], k)
    entries, refs, groups = [], [], []
    for i, (n, k, g) in enumerate([(512, 4096, 8), (96, 4096, 3), (1024, 14336, 2)]):
        Wi = _grouped_weights(n, k, g, 10 + i)
        Xi = workloads.acts_normal(1, k, 20 + i)
        ri = oracle.bitlinear_groups(Xi, Wi, g)
        Pi, bi = bl.quantize_weights_scale_groups(dev(Wi), g)
        Xqi, xsi = bl.quantize_acts(dev(Xi))
        Yi = torch.empty((1, n), dtype=torch.float32, device=DEV)
        ai = torch.empty((1, n), dtype=torch.int32, device=DEV)
        entries.append((Xqi, xsi, Pi, bi, Yi, ai))
        refs.append(ri)
        groups.append(g)
    bl.bitlinear_forward_grouped_scale_groups(entries, groups, 1)
    for (_, _, _, _, Yi, ai), ri in zip(entries, refs):
        assert np.array_equal(host(ai), ri["acc"])
        assert_y_close(host(Yi), ri["Y"], "grouped call")


@pytest.mark.parametrize("T", [1, 16, 24, 32, 48])
def test_fused_layer_layout_prepared(bl, T):
    # The decode layer in one allocation (reading L1): q|k|v and gate|up each quantized
    # per projection into consecutive rows, one scale per segment (rows per group = gcd
    # of the parts' rows), launched as one prepared grouped call with per-entry scale
    # groups. Every output must equal, bit for bit, the separate product of its
    # projection with its own scale; acc against the oracle.
    shapes = {"q": (192, 512), "k": (64, 512), "v": (64, 512), "o": (128, 512),
              "gate": (320, 512), "up": (320, 512), "down": (128, 1280)}
    fused = (("qkv", ("q", "k", "v"), 0), ("o", ("o",), 1), ("gateup", ("gate", "up"), 0),
             ("down", ("down",), 2))
    inputs = [workloads.acts_normal(T, 512, 40 + T), workloads.acts_normal(T, 512, 41 + T),
              workloads.acts_normal(T, 1280, 42 + T)]
    acts = [bl.quantize_acts(dev(X)) for X in inputs]
    total = sum(n * k // 4 for (n, k) in shapes.values())
    buf = torch.empty(total, dtype=torch.uint8, device=DEV)
    ws = torch.empty(max(bl.bitlinear_weight_workspace_bytes(*s) for s in shapes.values()),
                     dtype=torch.uint8, device=DEV)
    views, betas, Ws, off = {}, {}, {}, 0
    for p, (n, k) in shapes.items():
        Ws[p] = workloads.weights(n, k, 50 + n + k) * np.float32(1.0 + 0.3 * len(p))
        views[p] = buf[off: off + n * k // 4].view(n, k // 4)
        betas[p] = torch.empty(1, dtype=torch.float32, device=DEV)
        bl.bitlinear_quantize_weights(dev(Ws[p]), views[p], betas[p], None, ws)
        off += n * k // 4
    entries, groups, outs, base = [], [], [], 0
    for name, parts, inp in fused:
        rows = [shapes[p][0] for p in parts]
        k = shapes[parts[0]][1]
        rpg = int(np.gcd.reduce(rows))
        scale = torch.cat([betas[p].repeat(shapes[p][0] // rpg) for p in parts])
        n = sum(rows)
        Wf = buf[base: base + n * k // 4].view(n, k // 4)
        base += n * k // 4
        Y = torch.empty((T, n), dtype=torch.float32, device=DEV)
        A = torch.empty((T, n), dtype=torch.int32, device=DEV)
        entries.append((acts[inp][0], acts[inp][1], Wf, scale, Y, A))
        groups.append(n // rpg)
        outs.append((parts, inp, Y, A))
    call = bl.prepare_forward_grouped_scale_groups(entries, groups, T)
    call()
    call()  # a second launch of the same prepared call gives the same bits
    for parts, inp, Y, A in outs:
        r0 = 0
        for p in parts:
            n, k = shapes[p]
            Ys = torch.empty((T, n), dtype=torch.float32, device=DEV)
            As = torch.empty((T, n), dtype=torch.int32, device=DEV)
            bl.bitlinear_forward(acts[inp][0], acts[inp][1], views[p], betas[p], Ys, As)
            assert torch.equal(A[:, r0:r0 + n], As), p
            assert torch.equal(Y[:, r0:r0 + n], Ys), p
            acc_o = oracle.product(host(acts[inp][0]), host(views[p]), k)
            assert np.array_equal(host(As), acc_o), p
            r0 += n
