"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed weights, beta, gamma, int8 activations, token scales and int32
accumulators bit-exact; fp32 outputs within 1e-5 relative per element (an output the
oracle computes as 0 must be exactly 0). Inputs are the seeded workloads of
workloads.py. Small cases span several tiles and ragged tails on every kernel; the
full-size Llama-3-8B / 70B shapes run in the launch configuration the benchmark times
and are compared in full where the oracle is fast, on sampled rows otherwise.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import workloads  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RTOL = 1e-5


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_quantized_linear_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_y_close(Yh, Yo, what=""):
    bad = ~(np.abs(Yh.astype(np.float64) - Yo.astype(np.float64)) <= RTOL * np.abs(Yo.astype(np.float64)))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d outputs differ; first at %s: gpu %r oracle %r"
                             % (what, int(bad.sum()), tuple(i), Yh[tuple(i)], Yo[tuple(i)]))


def assert_codes_equal(qh, qo, Xref=None, what=""):
    if np.array_equal(qh, qo):
        return
    i = np.argwhere(qh != qo)[0]
    raise AssertionError("%s: %d int8 codes differ; first at %s: gpu %d oracle %d"
                         % (what, int((qh != qo).sum()), tuple(i), qh[tuple(i)], qo[tuple(i)]))


def random_product_inputs(T, N, K, seed):
    r = np.random.default_rng(seed)
    Xq = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    q = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    xs = r.uniform(1.0, 300.0, T).astype(np.float32)
    beta = np.float32(r.uniform(0.005, 0.05))
    return Xq, oracle.pack(q), xs, beta


# ---------------------------------------------------------------- weights

@pytest.mark.parametrize("N,K,seed", [(256, 1024, 0), (256, 1024, 1), (256, 1024, 2),
                                      (37, 68, 3), (1, 4, 4), (1024, 4096, 5), (3, 4100, 6)])
def test_quantize_weights_parity(bl, N, K, seed):
    W = workloads.weights(N, K, seed)
    P, beta, gamma = oracle.quantize_weights(W)
    for _ in range(2):  # run twice: bit-identical every time
        Pg, bg, gg = bl.quantize_weights(dev(W), with_gamma=True)
        assert host(gg)[0] == gamma
        assert host(bg)[0] == beta
        assert np.array_equal(host(Pg), P)


@pytest.mark.parametrize("seed", range(3))
def test_quantize_weights_exact_sum_wide_range(bl, seed):
    # magnitudes over ~250 binades: a floating-point tree sum would not be exact
    W = workloads.wide_range(64 * 4096, seed, lo_exp=-149, hi_exp=60).reshape(64, 4096)
    P, beta, gamma = oracle.quantize_weights(W)
    Pg, bg, gg = bl.quantize_weights(dev(W), with_gamma=True)
    assert host(gg)[0] == gamma
    assert host(bg)[0] == beta
    assert np.array_equal(host(Pg), P)


def test_quantize_weights_special_cases(bl):
    cases = [np.zeros((4, 8), np.float32), np.full((2, 8), 1e-40, np.float32),
             np.full((3, 12), 0.37, np.float32)]
    W = np.zeros((2, 16), np.float32)
    W[1, 3] = -100.0
    W[0, 7] = 0.01
    cases.append(W)
    for W in cases:
        P, beta, gamma = oracle.quantize_weights(W)
        Pg, bg, gg = bl.quantize_weights(dev(W), with_gamma=True)
        assert host(gg)[0] == gamma and host(bg)[0] == beta
        assert np.array_equal(host(Pg), P)


# ---------------------------------------------------------------- activations

@pytest.mark.parametrize("T,K,dist", [(8, 1024, "n"), (3, 4100, "n"), (1, 4096, "n"),
                                      (1, 14336, "n"), (16, 4096, "t"), (5, 28672, "n"),
                                      (2, 40000, "n"), (64, 8192, "t"), (7, 132104, "t"),
                                      (66, 14336, "t"), (130, 2052, "n"), (200, 28672, "n"),
                                      (4, 2000, "n"), (1, 28000, "t"), (2, 6000, "t")])
def test_quantize_acts_parity(bl, T, K, dist):
    X = (workloads.acts_normal if dist == "n" else workloads.acts_student_t)(T, K, T + K)
    q, s = oracle.quantize_acts(X)
    qg, sg = bl.quantize_acts(dev(X))
    assert np.array_equal(host(sg), s)
    assert_codes_equal(host(qg), q, X, "Xq")


@pytest.mark.parametrize("T,K", [(6, 2048), (1, 14336), (2, 40000), (70, 4100), (65, 36000),
                                 (67, 12000)])
def test_quantize_acts_gain_noNorm_eps(bl, T, K):
    # register-resident rows (few and many tokens) and the streaming variant
    X = workloads.acts_student_t(T, K, 3)
    g = (1 + 0.3 * np.random.default_rng(1).standard_normal(K)).astype(np.float32)
    for kw in ({"gain": g}, {"flags": oracle.NO_NORM}, {"eps": 0.0}, {"eps": 0.5},
               {"gain": g, "flags": oracle.NO_NORM}):
        q, s = oracle.quantize_acts(X, **kw)
        gk = dict(kw)
        if "gain" in gk:
            gk["gain"] = dev(gk["gain"])
        qg, sg = bl.quantize_acts(dev(X), **gk)
        assert np.array_equal(host(sg), s), kw
        assert_codes_equal(host(qg), q, X, str(kw))


def test_quantize_acts_special_rows(bl):
    K = 256
    X = np.zeros((5, K), np.float32)
    X[0] = 0.3
    X[1, 5] = -2.0
    X[3] = -1e3
    X[4, :4] = [127.0, 2.5, -3.5, 0.5]
    for flags in (0, oracle.NO_NORM):
        q, s = oracle.quantize_acts(X, flags=flags)
        qg, sg = bl.quantize_acts(dev(X), flags=flags)
        assert np.array_equal(host(sg), s)
        assert np.array_equal(host(qg), q)


def test_quantize_acts_grouped_equals_single(bl):
    Xs = [workloads.acts_normal(4, K, K) for K in (4096, 14336, 1024)]
    outs = []
    for X in Xs:
        outs.append((torch.empty(X.shape, dtype=torch.int8, device=DEV),
                     torch.empty(X.shape[0], dtype=torch.float32, device=DEV)))
    entries = [(dev(X), None, q, s) for X, (q, s) in zip(Xs, outs)]
    bl.bitlinear_quantize_acts_grouped(entries, 4, 1e-6, 0)
    for X, (q, s) in zip(Xs, outs):
        qo, so = oracle.quantize_acts(X)
        assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)


# ---------------------------------------------------------------- the product

PRODUCT_CASES = [
    # kernel, T, N, K
    ("gemv", 1, 4096, 4096), ("gemv", 1, 300, 4096), ("gemv", 1, 1000, 14336),
    ("gemv", 1, 97, 8192), ("gemv", 1, 64, 28672), ("gemv", 1, 33, 1024), ("gemv", 1, 70, 2048),
    ("gemv", 1, 50, 1088), ("gemv", 1, 3, 4096), ("gemv", 1, 20000, 4096), ("gemv", 1, 7, 14336),
    ("gemv", 1, 5, 64), ("gemv", 1, 130, 32768), ("gemv", 1, 9, 4160), ("gemv", 1, 611, 16384),
    ("skinny", 2, 300, 4096),
    ("skinny", 1, 300, 4096), ("skinny", 3, 129, 4096), ("skinny", 16, 1000, 14336),
    ("skinny", 17, 257, 8192), ("skinny", 32, 130, 1024), ("skinny", 31, 200, 28672),
    ("skinny", 9, 77, 4352), ("prefill", 33, 130, 1024), ("prefill", 64, 200, 28672),
    ("skinny", 33, 130, 1024), ("skinny", 100, 200, 4096), ("skinny", 128, 64, 8192),
    ("skinny", 8, 64, 256),
    # every segment length of the LDS regroup (64*MPW bytes per row, MPW = 1, 2, 4, 7),
    # one and two token blocks, several passes over K, ragged rows
    ("skinny", 12, 45, 512), ("skinny", 20, 45, 512), ("skinny", 16, 77, 28672),
    ("skinny", 7, 19, 4096), ("skinny", 2, 1001, 14336),
    # four token blocks (33..64 tokens in one pass; segments of 256 and 512 codes),
    # ragged tokens and rows, several passes over K, and more than one 64-token pass
    ("skinny", 64, 300, 8192), ("skinny", 48, 1001, 28672), ("skinny", 40, 77, 512),
    ("skinny", 64, 4097, 14336), ("skinny", 57, 16, 256), ("skinny", 65, 130, 4096),
    ("prefill", 1, 130, 1024), ("prefill", 100, 300, 4096), ("prefill", 129, 129, 1280),
    ("prefill", 263, 520, 14336), ("prefill", 256, 256, 128),
    # large-tile kernels (chosen by tile count): 128 x 256 tiles, then 256 x 256 tiles,
    # ragged in tokens and rows
    ("prefill", 130, 32845, 256), ("prefill", 300, 49102, 384), ("prefill", 513, 32668, 256),
    # up to 128 tokens with few row tiles: K cut into slices (int32 partials, then a
    # summing and rescaling kernel); one token block of 32, 64 (ragged) and 128 rows
    ("prefill", 17, 6500, 16384), ("prefill", 40, 12288, 4096), ("prefill", 100, 9000, 8192),
    ("prefill", 33, 6501, 16384),  # N % 4 != 0: the summing kernel's scalar path
    ("generic", 3, 77, 68), ("generic", 5, 300, 4100), ("generic", 1, 16, 4),
]


@pytest.mark.parametrize("kernel,T,N,K", PRODUCT_CASES)
def test_product_parity(bl, kernel, T, N, K):
    Xq, P, xs, beta = random_product_inputs(T, N, K, T * 1000 + N + K)
    acc_o = oracle.product(Xq, P, K)
    Y_o = oracle.rescale(acc_o, xs, beta)
    Yg, accg = bl.forward(dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)),
                          with_acc=True, kernel=kernel)
    assert np.array_equal(host(accg), acc_o), "%s T=%d N=%d K=%d accumulators" % (kernel, T, N, K)
    assert_y_close(host(Yg), Y_o, kernel)


@pytest.mark.parametrize("kernel,T", [("gemv", 1), ("skinny", 5), ("prefill", 70), ("generic", 2)])
def test_product_extreme_accumulators(bl, kernel, T):
    # |acc| = 127 * K at K = 28672 on every token: no int32 or fp32-conversion loss
    K, N = 28672, 64
    Xq = np.full((T, K), 127, np.int8)
    Xq[::2] = -127
    q = np.ones((N, K), np.int8)
    q[1::2] = -1
    P = oracle.pack(q)
    xs = np.full(T, 3.0, np.float32)
    beta = np.float32(0.02)
    acc_o = oracle.product(Xq, P, K)
    Yg, accg = bl.forward(dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)),
                          with_acc=True, kernel=kernel)
    assert np.array_equal(host(accg), acc_o)
    assert np.abs(acc_o).max() == 127 * K
    assert_y_close(host(Yg), oracle.rescale(acc_o, xs, beta), kernel)


def test_splitk_workspace_and_graph_capture(bl):
    # split K: the slices' int32 partials go to the caller's workspace. With no or too
    # small a workspace the product runs unsplit; either way it matches the oracle, also
    # as a captured graph replayed several times with eager work in between.
    T, N, K = 40, 12288, 4096
    Xq, P, xs, beta = random_product_inputs(T, N, K, 77)
    acc_o = oracle.product(Xq, P, K)
    Y_o = oracle.rescale(acc_o, xs, beta)
    dXq, dxs, dP = dev(Xq), dev(xs), dev(P)
    db = dev(np.array([beta], np.float32))
    nb = bl.bitlinear_forward_workspace_bytes(T, N, K)
    assert nb > 0
    Y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")

    def check(what):
        assert np.array_equal(host(acc), acc_o), what
        assert_y_close(host(Y), Y_o, what)

    for ws in (torch.empty(nb, dtype=torch.uint8, device="cuda"), None,
               torch.empty(nb - 16, dtype=torch.uint8, device="cuda")):
        acc.fill_(-1)
        bl.bitlinear_forward_ws(dXq, dxs, dP, db, Y, acc, "prefill", ws)
        torch.cuda.synchronize()
        check("eager, workspace %s" % (None if ws is None else ws.numel()))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bl.bitlinear_forward_ws(dXq, dxs, dP, db, Y, acc, "prefill", ws)
    for rep in range(3):
        Y.fill_(7.0)
        acc.fill_(-1)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check("graph replay %d" % rep)
    del g


def test_kernels_agree_bitwise(bl):
    # every kernel computes the same rescale from the same exact accumulator
    T, N, K = 1, 512, 4096
    Xq, P, xs, beta = random_product_inputs(T, N, K, 9)
    outs = [host(bl.forward(dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)), kernel=k))
            for k in ("gemv", "skinny", "prefill", "generic")]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_forward_grouped_mixed_shapes(bl):
    # seven projections with two different K in one grouped call, T = 1 and T = 16
    for T in (1, 16):
        entries, refs = [], []
        for i, (N, K) in enumerate([(300, 4096), (64, 4096), (1000, 14336), (128, 1024)]):
            Xq, P, xs, beta = random_product_inputs(T, N, K, 50 + i)
            Y = torch.empty((T, N), dtype=torch.float32, device=DEV)
            acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
            entries.append((dev(Xq), dev(xs), dev(P), dev(np.array([beta], np.float32)), Y, acc))
            refs.append((oracle.product(Xq, P, K), xs, beta))
        bl.bitlinear_forward_grouped(entries, T)
        for (_, _, _, _, Y, acc), (acc_o, xs, beta) in zip(entries, refs):
            assert np.array_equal(host(acc), acc_o)
            assert_y_close(host(Y), oracle.rescale(acc_o, xs, beta), "grouped")


# ---------------------------------------------------------------- whole forward

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_config_end_to_end(bl, seed):
    N, K = workloads.TINY_W
    W = workloads.weights(N, K, seed)
    X = workloads.acts_normal(workloads.TINY_T, K, seed + 100)
    ref = oracle.bitlinear(X, W)
    packed, beta = bl.quantize_weights(dev(W))
    Xq, xs = bl.quantize_acts(dev(X))
    assert np.array_equal(host(packed), ref["packed"]) and host(beta)[0] == ref["beta"]
    assert np.array_equal(host(Xq), ref["Xq"]) and np.array_equal(host(xs), ref["x_scale"])
    for k in ("auto", "skinny", "prefill", "generic"):
        Y, acc = bl.forward(Xq, xs, packed, beta, with_acc=True, kernel=k)
        assert np.array_equal(host(acc), ref["acc"]), k
        assert_y_close(host(Y), ref["Y"], k)
    module = bl.BitLinear(dev(W))
    assert_y_close(host(module(dev(X))), ref["Y"], "BitLinear module")


def _quantize_layer(bl, layer_seed):
    Ws = workloads.decode8b_layer(layer_seed)
    out = {}
    for name, W in Ws.items():
        P, beta, _ = oracle.quantize_weights(W)
        Pg, bg = bl.quantize_weights(dev(W))
        assert host(bg)[0] == beta, name
        assert np.array_equal(host(Pg), P), name
        out[name] = (Pg, bg, P, beta)
    return out


def _layer_forward_check(bl, layer, T, seed):
    inputs = workloads.decode8b_inputs(T, seed)
    acts = {}
    entries = []
    for name, X in inputs.items():
        Xg = dev(X)
        Xq = torch.empty(X.shape, dtype=torch.int8, device=DEV)
        xs = torch.empty(T, dtype=torch.float32, device=DEV)
        entries.append((Xg, None, Xq, xs))
        acts[name] = (Xq, xs, X)
    bl.bitlinear_quantize_acts_grouped(entries, T, 1e-6, 0)
    projs = []
    for name, ps in workloads.LLAMA3_8B_INPUTS.items():
        Xq, xs, X = acts[name]
        qo, so = oracle.quantize_acts(X)
        assert np.array_equal(host(xs), so) and np.array_equal(host(Xq), qo), name
        for p in ps:
            Pg, bg, P, beta = layer[p]
            N = P.shape[0]
            Y = torch.empty((T, N), dtype=torch.float32, device=DEV)
            acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
            projs.append((p, (Xq, xs, Pg, bg, Y, acc), (qo, so, P, beta)))
    bl.bitlinear_forward_grouped([e for _, e, _ in projs], T)
    for p, (_, _, _, _, Y, acc), (qo, so, P, beta) in projs:
        acc_o = oracle.product(qo, P, qo.shape[1])
        assert np.array_equal(host(acc), acc_o), p
        assert_y_close(host(Y), oracle.rescale(acc_o, so, beta), p)


def test_decode8b_layer_full(bl):
    # one Llama-3-8B layer at T = 1, seven projections in the grouped launch the
    # benchmark times; every output checked
    oracle.set_threads(0)
    layer = _quantize_layer(bl, 0)
    _layer_forward_check(bl, layer, 1, 100)


def test_fullpass_layers_t16(bl):
    # the full-pass workload runs each layer at T = 16 (skinny MFMA); layers 0 and 31
    for layer_seed in (0, 31):
        layer = _quantize_layer(bl, layer_seed)
        _layer_forward_check(bl, layer, workloads.FULLPASS_T, 200 + layer_seed)


@pytest.mark.parametrize("N,K", workloads.PREFILL_SHAPES)
def test_prefill_full_size_sampled(bl, N, K):
    T = workloads.PREFILL_T
    W = workloads.weights(N, K, 7)
    X = workloads.acts_student_t(T, K, 8)
    P, beta, _ = oracle.quantize_weights(W)
    Pg, bg = bl.quantize_weights(dev(W))
    assert host(bg)[0] == beta and np.array_equal(host(Pg), P)
    qo, so = oracle.quantize_acts(X)
    Xq, xs = bl.quantize_acts(dev(X))
    assert np.array_equal(host(xs), so)
    assert_codes_equal(host(Xq), qo, X, "prefill Xq")
    assert bl.bitlinear_forward_choice(T, N, K) == "prefill"
    Y, acc = bl.forward(Xq, xs, Pg, bg, with_acc=True)
    Yh, acch = host(Y), host(acc)
    r = np.random.default_rng(0)
    rows = np.unique(np.concatenate([r.choice(N, 48, replace=False), [0, N - 1]]))
    acc_o = oracle.product(qo, P[rows], K)
    assert np.array_equal(acch[:, rows], acc_o)
    assert_y_close(Yh[:, rows], oracle.rescale(acc_o, so, beta), "prefill")
    toks = np.unique(np.concatenate([r.choice(T, 8, replace=False), [0, T - 1]]))
    acc_t = oracle.product(qo[toks], P, K)
    assert np.array_equal(acch[toks], acc_t)


# 17..64 tokens run as token slices of 16 or 32 (entries of one grouped launch over the
# same weights, the last slice ragged) or as one slice, by shape: each way at full size,
# all tokens on sampled rows and all rows on sampled tokens
@pytest.mark.parametrize("T,N,K", [(50, 28672, 8192), (48, 28672, 4096), (24, 28672, 8192),
                                   (61, 4096, 14336), (40, 6144, 4096), (26, 4096, 14336),
                                   (17, 4096, 14336)])
def test_skinny_token_slices_sampled(bl, T, N, K):
    print("skinny slices T=%d N=%d K=%d" % (T, N, K), flush=True)
    r = np.random.default_rng(T + N + K)
    Xq = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    q = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    P = oracle.pack(q)
    del q
    xs = r.uniform(1.0, 300.0, T).astype(np.float32)
    beta = np.float32(0.02)
    Y = torch.empty((T, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    bl.bitlinear_forward_ex(dev(Xq), dev(xs), dev(P), dev(np.array([beta])), Y, acc, kernel="skinny")
    Yh, acch = host(Y), host(acc)
    rows = np.unique(np.concatenate([r.choice(N, 64, replace=False), [0, N - 1]]))
    acc_o = oracle.product(Xq, P[rows], K)
    assert np.array_equal(acch[:, rows], acc_o)
    assert_y_close(Yh[:, rows], oracle.rescale(acc_o, xs, beta), "slices")
    toks = np.unique(np.array([0, 15, 16, 31, 32, 47, 48, T - 1]).clip(0, T - 1))
    acc_t = oracle.product(Xq[toks], P, K)
    assert np.array_equal(acch[toks], acc_t)


@pytest.mark.parametrize("which", ["down", "gate"])
def test_sweep70b_full_size_sampled(bl, which):
    N, K = workloads.LLAMA_70B_SWEEP[which]
    W = workloads.weights(N, K, 70)
    P, beta, _ = oracle.quantize_weights(W)
    Pg, bg = bl.quantize_weights(dev(W))
    assert host(bg)[0] == beta and np.array_equal(host(Pg), P)
    del W
    r = np.random.default_rng(1)
    rows = np.unique(np.concatenate([r.choice(N, 96, replace=False), [0, N - 1]]))
    # 16 tokens on the down matrix: the most the streaming kernel takes at K = 28672
    for T in workloads.SWEEP_TOKENS + ((16,) if which == "down" else ()):
        X = workloads.acts_normal(T, K, 1000 + T)
        qo, so = oracle.quantize_acts(X)
        Xq, xs = bl.quantize_acts(dev(X))
        assert np.array_equal(host(Xq), qo) and np.array_equal(host(xs), so)
        Y, acc = bl.forward(Xq, xs, Pg, bg, with_acc=True)
        acc_o = oracle.product(qo, P[rows], K)
        assert np.array_equal(host(acc)[:, rows], acc_o), "T=%d" % T
        assert_y_close(host(Y)[:, rows], oracle.rescale(acc_o, so, beta), "T=%d" % T)
