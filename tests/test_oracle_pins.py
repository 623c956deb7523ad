"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against exact-rational or 60-digit brute force, a library
routine (math.fsum, a float64 BLAS matmul), a closed form, an invariant that the
definitions fix, or a hand-worked fixture under tests/golden/. The tests are chosen
so that a plausible slip in the oracle -- a wrong rounding mode, a per-row instead of
a per-tensor scale, a sum instead of a mean, a misplaced epsilon, 128 in place of 127,
a transposed operand, a flipped code sign, an inverted rescale -- fails at least one.
"""
import math
import os
import sys
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import workloads  # noqa: E402
from golden.load import load  # noqa: E402

F32 = np.float32


def ulp32(x):
    x = abs(float(x))
    if x < 2.0 ** -126:
        return 2.0 ** -149
    return 2.0 ** (math.floor(math.log2(x)) - 23)


# ---------------------------------------------------------------- exact sums (gamma)

def _fraction_abs_sum(a):
    return sum((Fraction(float(v)) for v in np.abs(a.astype(np.float64)).ravel()), Fraction(0))


@pytest.mark.parametrize("seed", range(6))
def test_abs_sum_equals_exact_rational(seed):
    # values over ~250 binades, denormals included: naive float sums lose them
    a = workloads.wide_range(2000, seed)
    exact = _fraction_abs_sum(a)
    assert oracle.abs_sum(a) == float(exact)  # float(Fraction) rounds correctly


def test_abs_sum_equals_math_fsum_large():
    r = np.random.default_rng(7)
    a = (r.standard_normal(3_000_000) * np.exp(r.uniform(-30, 30, 3_000_000))).astype(np.float32)
    assert oracle.abs_sum(a) == math.fsum(np.abs(a.astype(np.float64)).tolist())


def test_abs_sum_rounding_ties():
    # 1 + 2^-53 is a midpoint between 1 and 1 + 2^-52: ties to even gives 1;
    # a further 2^-80 puts the exact sum above the midpoint: the result must round up.
    assert oracle.abs_sum(np.array([1.0, 2.0 ** -53], np.float32)) == 1.0
    assert oracle.abs_sum(np.array([1.0, 2.0 ** -53, 2.0 ** -80], np.float32)) == 1.0 + 2.0 ** -52
    assert oracle.abs_sum(np.array([2.0 ** -80, 2.0 ** -53, 1.0], np.float32)) == 1.0 + 2.0 ** -52
    # 2^-110 lies more than 53 binades below 2^-53, so no two parts can merge: the sum
    # is held as 1 + 2^-53 (an exact midpoint) plus 2^-110, and must still round up
    assert oracle.abs_sum(np.array([1.0, 2.0 ** -53, 2.0 ** -110], np.float32)) == 1.0 + 2.0 ** -52
    # 1 + 3*2^-53 is a midpoint between 1+2^-52 and 1+2^-51: even is 1+2^-51
    v = np.array([1.0, 2.0 ** -52, 2.0 ** -53], np.float32)
    assert oracle.abs_sum(v) == 1.0 + 2.0 ** -51


def test_abs_sum_order_and_thread_independent():
    a = workloads.weights(512, 4096, 3).ravel()
    perm = np.random.default_rng(1).permutation(a.size)
    oracle.set_threads(1)
    one = oracle.abs_sum(a)
    oracle.set_threads(os.cpu_count() or 1)
    assert oracle.abs_sum(a[perm]) == one
    assert oracle.abs_sum(a[::-1].copy()) == one


@pytest.mark.parametrize("seed", range(3))
def test_sum_sq_equals_exact_rational(seed):
    a = workloads.wide_range(1000, seed, lo_exp=-60, hi_exp=60)
    exact = sum((Fraction(float(v)) ** 2 for v in a.astype(np.float64)), Fraction(0))
    assert oracle.sum_sq(a) == float(exact)


def test_oracle_rejects_nonfinite():
    for bad in (np.inf, -np.inf, np.nan):
        with pytest.raises(oracle.OracleError):
            oracle.abs_sum(np.array([1.0, bad], np.float32))
        with pytest.raises(oracle.OracleError):
            oracle.quantize_acts(np.array([[1.0, bad, 0.0, 0.0]], np.float32))


# ---------------------------------------------------------------- weight scale / codes

@pytest.mark.parametrize("shape", [(3, 8), (7, 12), (16, 64)])
def test_weight_scale_equals_exact_rational(shape):
    N, K = shape
    W = workloads.wide_range(N * K, N, lo_exp=-40, hi_exp=5).reshape(N, K)
    gamma, beta = oracle.weight_scale(W)
    S = float(_fraction_abs_sum(W))          # exact sum, one rounding to fp64
    g = S / float(N * K)                     # fp64 division
    assert gamma == g
    assert beta == F32(g)


def test_weight_scale_is_mean_over_gaussian():
    # closed form: E|w| = sigma * sqrt(2/pi) for w ~ N(0, sigma^2)
    W = workloads.weights(1024, 4096, 11)
    gamma, _ = oracle.weight_scale(W)
    n = W.size
    ratio = gamma / workloads.WEIGHT_SIGMA
    se = math.sqrt(1 - 2 / math.pi) / math.sqrt(n)  # std error of mean|z|
    assert abs(ratio - math.sqrt(2 / math.pi)) < 5 * se


def test_weight_scale_power_of_two_equivariance():
    W = workloads.weights(64, 256, 2)
    g0, b0 = oracle.weight_scale(W)
    for k in (-7, 3, 20):
        gk, bk = oracle.weight_scale((W * F32(2.0 ** k)).astype(np.float32))
        assert gk == g0 * 2.0 ** k and bk == b0 * F32(2.0 ** k)


def test_golden_weights_ties():
    g = load("weights_ties.txt")
    W = np.array(g["W"], np.float32)
    P, beta, gamma = oracle.quantize_weights(W)
    assert gamma == g["gamma"] and beta == g["beta"]
    q = oracle.ternarize(W, beta)
    assert q.tolist() == g["codes"]
    assert P.tolist() == g["packed"]


def test_golden_per_tensor_scale():
    g = load("weights_per_tensor.txt")
    W = np.array(g["W"], np.float32)
    P, beta, gamma = oracle.quantize_weights(W)
    assert gamma == g["gamma"]
    assert oracle.unpack(P, W.shape[1]).tolist() == g["codes"]


def test_codes_invariants_and_gaussian_zero_fraction():
    # closed form: q = 0 iff |w| <= gamma/2 with gamma = sigma*sqrt(2/pi), so the
    # zero fraction is 2*Phi(sqrt(2/pi)/2) - 1 = 0.31006 and each sign 0.34497.
    W = workloads.weights(1024, 2048, 5)
    P, beta, _ = oracle.quantize_weights(W)
    q = oracle.unpack(P, 2048)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    z = math.sqrt(2 / math.pi) / 2
    p0 = math.erf(z / math.sqrt(2))
    frac0 = float(np.mean(q == 0))
    assert abs(p0 - 0.31006) < 1e-4
    assert abs(frac0 - p0) < 0.002
    assert abs(float(np.mean(q == 1)) - (1 - p0) / 2) < 0.002
    assert abs(float(np.mean(q == -1)) - (1 - p0) / 2) < 0.002
    # the sign of every non-zero code is the sign of its weight
    nz = q != 0
    assert np.all(np.sign(W[nz]) == q[nz])


def test_codes_special_cases():
    # constant matrix: scale 1/c maps every weight to exactly 1
    W = np.full((4, 8), 0.37, np.float32)
    P, beta, _ = oracle.quantize_weights(W)
    assert beta == F32(0.37) and np.all(oracle.unpack(P, 8) == 1)
    # all zero: beta = 0 and every code 0
    P, beta, _ = oracle.quantize_weights(np.zeros((2, 4), np.float32))
    assert beta == 0 and np.all(oracle.unpack(P, 4) == 0)
    # denormal-only weights: beta below FLT_MIN gives all codes 0
    W = np.full((2, 4), 1e-40, np.float32)
    P, beta, _ = oracle.quantize_weights(W)
    assert beta < np.finfo(np.float32).tiny and np.all(oracle.unpack(P, 4) == 0)
    # one outlier dominates the mean: the others round to 0, the outlier clamps to 1
    W = np.zeros((1, 8), np.float32)
    W[0, 3] = -100.0
    W[0, 5] = 0.01
    P, beta, _ = oracle.quantize_weights(W)
    assert oracle.unpack(P, 8).tolist() == [[0, 0, 0, -1, 0, 0, 0, 0]]


# ---------------------------------------------------------------- packing

def test_pack_roundtrip_and_layout():
    r = np.random.default_rng(3)
    q = r.integers(-1, 2, size=(37, 64)).astype(np.int8)
    P = oracle.pack(q)
    assert P.shape == (37, 16) and P.nbytes == 37 * 64 // 4
    assert np.array_equal(oracle.unpack(P, 64), q)
    # independent decode: code k = 4j+i sits in bits [2i+1:2i] of byte j, as q+1
    dec = np.stack([((P >> (2 * i)) & 3).astype(np.int8) - 1 for i in range(4)], axis=-1)
    assert np.array_equal(dec.reshape(37, 64), q)


def test_unpack_rejects_unused_pattern():
    with pytest.raises(oracle.OracleError):
        oracle.unpack(np.array([[0b11000000]], np.uint8), 4)


def test_pack_density_matches_page_counts():
    g = load("page_counts.txt")
    n_proj = sum(N * K for (N, K) in workloads.LLAMA3_8B.values()) * workloads.LLAMA3_8B_LAYERS
    packed_elems = n_proj // 4             # four 2-bit codes per int8 element
    assert n_proj == 6_979_321_856 and packed_elems == 1_744_830_464
    # the rest of the 8B model (embeddings, head, norms) stays unpacked
    rest = 8.03e9 - n_proj
    assert abs((packed_elems + rest) - g["params_after"]) < 0.05e9
    # 2 bits per weight is 87.5% below 16; the entropy figure log2(3) is the page's ~90%
    assert abs(math.log2(3) - g["bits_ternary"]) < 0.005
    assert abs((1 - g["bits_ternary"] / g["bits_fp16"]) - g["memory_saving_approx"]) < 0.01
    assert 1 - 2 / 16 == 0.875


# ---------------------------------------------------------------- activations

def test_golden_acts_ties():
    g = load("acts_ties.txt")
    X = np.array(g["X"], np.float32)
    q, s = oracle.quantize_acts(X, flags=oracle.NO_NORM)
    assert q.tolist() == g["codes"] and s.tolist() == g["x_scale"]


def _decimal_rmsnorm(x, eps, gain=None):
    getcontext().prec = 60
    d = [Decimal(float(v)) for v in x]
    ms = sum(v * v for v in d) / len(d)
    r = 1 / (ms + Decimal(float(F32(eps)))).sqrt()
    if gain is None:
        return [v * r for v in d]
    return [v * r * Decimal(float(gv)) for v, gv in zip(d, gain)]


@pytest.mark.parametrize("seed,gain", [(0, False), (1, True), (2, False)])
def test_rmsnorm_and_codes_against_decimal(seed, gain):
    K = 96
    X = workloads.acts_student_t(3, K, seed)
    X[1] *= F32(1e-3)  # a token whose mean square is near eps
    g = (1 + 0.5 * np.random.default_rng(seed).standard_normal(K)).astype(np.float32) if gain else None
    Y = oracle.rmsnorm(X, g, 1e-6)
    q, s = oracle.quantize_acts(X, g, 1e-6)
    for t in range(X.shape[0]):
        ye = _decimal_rmsnorm(X[t], 1e-6, g)
        for k in range(K):
            err = abs(Decimal(float(Y[t, k])) - ye[k])
            assert err <= Decimal(0.5000001) * Decimal(ulp32(float(ye[k])))
        m = max(abs(float(v)) for v in Y[t])
        se = Decimal(127) / Decimal(max(m, float(F32(1e-5))))
        assert abs(Decimal(float(s[t])) - se) <= Decimal(0.5) * Decimal(ulp32(float(se)))
        for k in range(K):
            v = Decimal(float(Y[t, k])) * Decimal(float(s[t]))
            frac = abs(v - v.to_integral_value(rounding="ROUND_FLOOR") - Decimal("0.5"))
            if frac > Decimal("1e-4"):  # away from a tie, fp32 rounding cannot matter
                assert int(q[t, k]) == int(v.to_integral_value(rounding="ROUND_HALF_EVEN"))


def test_rmsnorm_mean_square_closed_form():
    # mean(y^2) = ms / (ms + eps) before rounding: a token with ms = eps gives 1/2
    r = np.random.default_rng(4)
    x = r.standard_normal(4096)
    x = x / np.sqrt(np.mean(x * x)) * 1e-3          # ms = 1e-6 = eps (up to rounding)
    X = x.astype(np.float32)[None, :]
    ms = float(np.mean(X.astype(np.float64) ** 2))
    Y = oracle.rmsnorm(X, None, 1e-6).astype(np.float64)
    expect = ms / (ms + float(F32(1e-6)))
    assert abs(float(np.mean(Y * Y)) - expect) < 1e-6
    assert abs(expect - 0.5) < 1e-3
    # and a unit-scale token is normalized to mean square ~1
    X = workloads.acts_normal(1, 4096, 9)
    Y = oracle.rmsnorm(X, None, 1e-6).astype(np.float64)
    assert abs(float(np.mean(Y * Y)) - 1.0) < 1e-5


def test_act_codes_invariants():
    X = np.concatenate([workloads.acts_normal(8, 1024, 1), workloads.acts_student_t(8, 1024, 2)])
    q, s = oracle.quantize_acts(X)
    assert q.min() >= -127 and q.max() <= 127          # -128 never appears with 127
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    Y = oracle.rmsnorm(X)
    assert np.all(np.sign(q) == np.where(q == 0, 0, np.sign(Y)))


def test_act_special_rows():
    K = 64
    X = np.zeros((4, K), np.float32)
    X[0] = 0.3                    # constant row -> all +127
    X[1, 5] = -2.0                # one-hot row -> one -127, the rest 0
    X[3] = -1e3                   # constant negative row -> all -127
    q, s = oracle.quantize_acts(X)
    assert np.all(q[0] == 127) and np.all(q[3] == -127)
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1
    assert np.all(q[2] == 0) and s[2] == F32(127.0) / F32(1e-5)   # zero row: floor 1e-5


def _decimal_rms_inv(x, eps):
    # r = 1 / sqrt(mean(x^2) + eps), every step in 60 digits from the exact fp32 inputs
    getcontext().prec = 60
    d = [Decimal(float(v)) for v in x]
    return 1 / (sum(v * v for v in d) / len(d) + Decimal(float(F32(eps)))).sqrt()


def test_rms_inv_exact_cases():
    # x = [3, 4], eps = 0: mean square 25/2, so r = 1/sqrt(12.5) = sqrt(2)/5
    getcontext().prec = 60
    r = oracle.rms_inv(np.array([[3.0, 4.0], [2.0, -2.0]], np.float32), eps=0.0)
    assert r.dtype == np.float64 and r.shape == (2,)
    exact = Decimal(2).sqrt() / 5
    assert abs(Decimal(float(r[0])) - exact) <= Decimal(2.0 ** -53) * exact
    assert r[1] == 0.5                                  # mean square 4: r = 1/2 exactly
    # the norm switched off: r = 1 for every token, whatever the values
    X = workloads.acts_normal(3, 64, 5)
    assert np.array_equal(oracle.rms_inv(X, flags=oracle.NO_NORM), np.ones(3))


@pytest.mark.parametrize("K", [4, 96, 4096])
def test_rms_inv_against_decimal(K):
    # the fp64 factor is within a few roundings (sum once, /K, +eps, sqrt, 1/) of the
    # 60-digit value: a K-1 for K, eps outside the square root, eps dropped or taken as
    # the double 1e-6 instead of fp32(1e-6), or an fp32 square root each miss by far more
    X = workloads.acts_normal(4, K, 40 + K)
    X[1] *= F32(1e-3)          # mean square near eps: eps is half of the radicand
    X[2] *= F32(3e-5)          # mean square far below eps: eps dominates
    X[3] *= F32(1e4)           # large values
    r = oracle.rms_inv(X, eps=1e-6)
    for t in range(X.shape[0]):
        re = _decimal_rms_inv(X[t], 1e-6)
        assert abs(Decimal(float(r[t])) - re) <= Decimal(4 * 2.0 ** -53) * re


def test_rms_inv_matches_the_rmsnorm_output():
    # the C RMSNorm forms y = fp32(fp64(x * r)) (unit gain): the same r, bit for bit
    X = np.concatenate([workloads.acts_normal(4, 1024, 6), workloads.acts_student_t(4, 1024, 7)])
    r = oracle.rms_inv(X, eps=1e-6)
    y = (X.astype(np.float64) * r[:, None]).astype(np.float32)
    assert np.array_equal(y, oracle.rmsnorm(X, None, 1e-6))


def test_act_quant_scale_invariance_without_eps():
    # with eps = 0, RMSNorm is invariant under x -> 2^k x, bit for bit
    X = workloads.acts_normal(4, 512, 3)
    q0, s0 = oracle.quantize_acts(X, eps=0.0)
    for k in (-20, 5):
        qk, sk = oracle.quantize_acts((X * F32(2.0 ** k)).astype(np.float32), eps=0.0)
        assert np.array_equal(q0, qk) and np.array_equal(s0, sk)


# ---------------------------------------------------------------- product and rescale

def test_golden_forward():
    gw, ga, gf = load("weights_ties.txt"), load("acts_ties.txt"), load("forward_small.txt")
    out = oracle.bitlinear(np.array(ga["X"], np.float32), np.array(gw["W"], np.float32),
                           flags=oracle.NO_NORM)
    assert out["acc"].tolist() == gf["acc"]
    assert out["Y"].tolist() == gf["Y"]


@pytest.mark.parametrize("T,N,K", [(1, 7, 16), (5, 33, 100), (16, 64, 1024)])
def test_product_add_sub_and_blas(T, N, K):
    r = np.random.default_rng(T * N + K)
    Xq = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    q = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = oracle.product(Xq, oracle.pack(q), K)
    x = Xq.astype(np.int64)
    # add/subtract form: only additions of +x and -x, no multiplications
    addsub = np.stack([(x * (q[o] == 1)).sum(1) - (x * (q[o] == -1)).sum(1) for o in range(N)], 1)
    assert np.array_equal(acc, addsub)
    # a float64 BLAS matmul of the integer matrices is exact here (|acc| < 2^53)
    assert np.array_equal(acc, (Xq.astype(np.float64) @ q.astype(np.float64).T).astype(np.int64))


def test_product_python_int_bruteforce():
    r = np.random.default_rng(0)
    Xq = r.integers(-127, 128, size=(3, 12)).astype(np.int8)
    q = r.integers(-1, 2, size=(5, 12)).astype(np.int8)
    acc = oracle.product(Xq, oracle.pack(q), 12)
    for t in range(3):
        for o in range(5):
            assert acc[t, o] == sum(int(Xq[t, k]) * int(q[o, k]) for k in range(12))


def test_product_extreme_magnitude():
    K = 28672
    Xq = np.full((1, K), 127, np.int8)
    q = np.ones((2, K), np.int8)
    q[1] = -1
    acc = oracle.product(Xq, oracle.pack(q), K)
    assert acc.tolist() == [[127 * K, -127 * K]]


def test_rescale_against_exact_rational():
    r = np.random.default_rng(5)
    acc = r.integers(-300000, 300000, size=(4, 50)).astype(np.int32)
    acc[0, 0] = 0
    s = (r.uniform(0.5, 200, 4)).astype(np.float32)
    beta = F32(0.0159)
    Y = oracle.rescale(acc, s, beta)
    assert Y[0, 0] == 0.0
    for t in range(4):
        for o in range(50):
            e = Fraction(int(acc[t, o])) * Fraction(float(beta)) / Fraction(float(s[t]))
            assert abs(Fraction(float(Y[t, o])) - e) <= Fraction(0.5000001) * Fraction(ulp32(float(e)))


def test_forward_equals_dequantized_matmul():
    # y = (Xq / s) (beta * q)^T: dequantized activations times dequantized weights
    W = workloads.weights(*workloads.TINY_W, seed=0)
    X = workloads.acts_normal(workloads.TINY_T, workloads.TINY_W[1], seed=1)
    out = oracle.bitlinear(X, W)
    q = oracle.unpack(out["packed"], W.shape[1]).astype(np.float64)
    xd = out["Xq"].astype(np.float64) / out["x_scale"].astype(np.float64)[:, None]
    ref = xd @ (float(out["beta"]) * q).T
    assert np.allclose(out["Y"], ref, rtol=1e-6, atol=1e-30)
    # closed form of the agreement with the unquantized RMSNorm(X) W^T: for Gaussian w
    # and q = sign(w) [|w| > c sigma], c = sqrt(2/pi)/2, corr(w, q) = 2 phi(c) / sqrt(P(|z| > c))
    c = math.sqrt(2 / math.pi) / 2
    phi = math.exp(-c * c / 2) / math.sqrt(2 * math.pi)
    corr = 2 * phi / math.sqrt(1 - math.erf(c / math.sqrt(2)))
    assert abs(corr - 0.8866) < 1e-3
    full = oracle.rmsnorm(X).astype(np.float64) @ W.astype(np.float64).T
    cos = np.sum(full * out["Y"]) / np.linalg.norm(full) / np.linalg.norm(out["Y"])
    assert abs(cos - corr) < 0.01


# ---------------------------------------------------------------- 1-bit sign variant

@pytest.mark.parametrize("seed", range(4))
def test_signed_sum_equals_exact_rational(seed):
    a = workloads.wide_range(2000, seed)
    exact = sum((Fraction(float(v)) for v in a.astype(np.float64).ravel()), Fraction(0))
    assert oracle.exact_sum(a) == float(exact)


def test_signed_sum_cancellation():
    # the large terms cancel exactly; what is left is far below their ulp
    a = np.array([2.0 ** 100, 3.0, -(2.0 ** 100), 2.0 ** -60], np.float32)
    assert oracle.exact_sum(a) == 3.0 + 2.0 ** -60
    assert oracle.exact_sum(-a) == -(3.0 + 2.0 ** -60)


def test_golden_sign_weights():
    g = load("sign_weights.txt")
    for k in ("A", "B"):
        W = np.array(g[k + "_W"], np.float32)
        c, alpha, gamma, beta = oracle.sign_weights(W)
        assert alpha == g[k + "_alpha"] and beta == g[k + "_beta"]
        assert c.tolist() == g[k + "_codes"]
        assert oracle.pack1(c).tolist() == g[k + "_packed"]
        assert oracle.unpack1(oracle.pack1(c), W.shape[1]).tolist() == g[k + "_codes"]


def test_golden_sign_forward():
    g = load("sign_weights.txt")
    P = np.array(g["A_packed"], np.uint8)
    Y, acc = oracle.forward_sign(np.array(g["C_Xq"], np.int8), np.array(g["C_s"], np.float32),
                                 P, np.float32(g["A_beta"]))
    assert acc.tolist() == g["C_acc"] and Y.tolist() == g["C_Y"]


def test_sign_alpha_is_exact_mean_and_codes_threshold():
    r = np.random.default_rng(3)
    W = (r.standard_normal((37, 64)) * 0.02 + 0.003).astype(np.float32)
    c, alpha, gamma, beta = oracle.sign_weights(W)
    exact = sum((Fraction(float(v)) for v in W.astype(np.float64).ravel()), Fraction(0))
    assert alpha == float(exact) / W.size  # the exact sum rounded once, then one division
    # the code is the sign of the exact difference, -1 on a tie
    w64 = W.astype(np.float64)
    assert np.array_equal(c, np.where(w64 > alpha, 1, -1).astype(np.int8))
    # a weight placed exactly on alpha goes to -1, one ulp above goes to +1
    W2 = np.array([[1.0, 2.0, 3.0, 4.0, 2.5, 2.5, 2.5, 2.5]], np.float32)  # mean 2.5
    c2, a2, _, _ = oracle.sign_weights(W2)
    assert a2 == 2.5 and c2.tolist() == [[-1, -1, 1, 1, -1, -1, -1, -1]]
    W3 = W2.copy()
    W3[0, 4] = np.nextafter(np.float32(2.5), np.float32(3.0))
    c3, a3, _, _ = oracle.sign_weights(W3)
    # sum = 20 + 2^-22 (one fp32 ulp of 2.5), alpha = 2.5 + 2^-25 < 2.5 + 2^-22
    assert a3 == 2.5 + 2.0 ** -25
    assert c3.tolist() == [[-1, -1, 1, 1, 1, -1, -1, -1]]


def test_sign_codes_invariants_gaussian():
    # codes are +-1 only; about half are +1 for a symmetric distribution about its mean;
    # beta = mean |W| -> sigma * sqrt(2/pi) for zero-mean Gaussian weights
    r = np.random.default_rng(11)
    W = (r.standard_normal((512, 2048)) * 0.02).astype(np.float32)
    c, alpha, gamma, beta = oracle.sign_weights(W)
    assert set(np.unique(c).tolist()) <= {-1, 1}
    assert abs(float((c == 1).mean()) - 0.5) < 0.003
    assert abs(gamma / (0.02 * math.sqrt(2.0 / math.pi)) - 1.0) < 0.003
    assert beta == F32(gamma)


def test_sign_scale_minimizes_l2_error():
    # [BitDelta] Eq. (3)-(4): for a sign code S = Sign(W) the error ||W - b S||^2 is
    # smallest at b = mean |W|. Zero-mean W (each value with its negative) makes
    # alpha = 0, so the oracle's codes are Sign(W) itself.
    r = np.random.default_rng(5)
    half = (r.standard_normal(4096) * 0.02).astype(np.float32)
    W = np.concatenate([half, -half]).reshape(8, 1024)
    c, alpha, gamma, beta = oracle.sign_weights(W)
    assert alpha == 0.0
    w = W.astype(np.float64).ravel()
    s = c.astype(np.float64).ravel()

    def err(b):
        return float(np.sum((w - b * s) ** 2))

    e0 = err(gamma)
    for d in (1e-3, 1e-5, 1e-7):
        assert e0 <= err(gamma * (1 + d)) and e0 <= err(gamma * (1 - d))
    # the closed-form minimizer sum(W*S)/sum(S*S) equals mean |W|
    assert abs(float(np.dot(w, s) / np.dot(s, s)) - gamma) <= 1e-12 * gamma


def test_pack1_layout_roundtrip_and_density():
    r = np.random.default_rng(2)
    c = np.where(r.random((13, 64)) < 0.5, -1, 1).astype(np.int8)
    P = oracle.pack1(c)
    assert P.shape == (13, 8)
    for o in range(13):
        for k in range(64):
            assert ((int(P[o, k // 8]) >> (k % 8)) & 1) == (1 if c[o, k] == 1 else 0)
    assert np.array_equal(oracle.unpack1(P, 64), c)
    with pytest.raises(oracle.OracleError):
        oracle.pack1(np.zeros((1, 8), np.int8))  # 0 is not a sign code
    # one bit per weight: an 8B-parameter model packs into 1e9 bytes
    assert 8_000_000_000 // 8 == 1_000_000_000


def test_sign_product_bruteforce_and_identity():
    r = np.random.default_rng(9)
    T, N, K = 3, 7, 96
    Xq = r.integers(-128, 128, (T, K), dtype=np.int64).astype(np.int8)
    c = np.where(r.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    acc = oracle.product_sign(Xq, oracle.pack1(c), K)
    for t in range(T):
        for o in range(N):
            assert int(acc[t, o]) == sum(int(Xq[t, k]) * int(c[o, k]) for k in range(K))
    # sum c*x = 2 * sum_{c=+1} x - sum x
    pos = (c == 1).astype(np.int64)
    assert np.array_equal(acc, 2 * (Xq.astype(np.int64) @ pos.T) - Xq.astype(np.int64).sum(1)[:, None])


def test_sign_forward_equals_dequantized_matmul():
    r = np.random.default_rng(4)
    X = r.standard_normal((5, 256)).astype(np.float32)
    W = (r.standard_normal((33, 256)) * 0.02).astype(np.float32)
    out = oracle.bitlinear_sign(X, W)
    deq = (out["Xq"].astype(np.float64) / out["x_scale"].astype(np.float64)[:, None]) @ \
          (out["codes"].astype(np.float64) * float(out["beta"])).T
    assert np.allclose(out["Y"].astype(np.float64), deq, rtol=1e-6, atol=1e-6 * np.abs(deq).max())


# ---------------------------------------------------------------- group quantization

def test_golden_weight_groups():
    g = load("weight_groups.txt")
    W = np.array(g["W"], np.float32)
    P, beta, gamma = oracle.quantize_weights_groups(W, g["G"])
    assert beta.tolist() == g["beta"] and P.tolist() == g["packed"]
    acc = oracle.product(np.array(g["Xq"], np.int8), P, W.shape[1])
    assert acc.tolist() == g["acc"]
    s = np.array(g["s"], np.float32)
    assert oracle.rescale_groups(acc, s, beta).tolist() == g["Y"]
    P1, b1, _ = oracle.quantize_weights(W)
    assert oracle.rescale(oracle.product(np.array(g["Xq"], np.int8), P1, 4), s, b1).tolist() == \
        g["Y_one_scale"]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_weight_groups_are_independent_blocks(G):
    # each block's scale and codes are those of the block quantized alone; G = 1 is the
    # per-tensor quantizer; scaling one block by 2^k changes only that block's scale
    r = np.random.default_rng(G)
    W = (r.standard_normal((64, 256)) * np.repeat(r.uniform(0.005, 0.05, G), 64 // G)[:, None]
         ).astype(np.float32)
    P, beta, gamma = oracle.quantize_weights_groups(W, G)
    rows = 64 // G
    for g in range(G):
        Pg, bg, gg = oracle.quantize_weights(W[g * rows:(g + 1) * rows])
        assert beta[g] == bg and gamma[g] == gg
        assert np.array_equal(P[g * rows:(g + 1) * rows], Pg)
    if G == 1:
        P1, b1, g1 = oracle.quantize_weights(W)
        assert np.array_equal(P, P1) and beta[0] == b1
    W2 = W.copy()
    W2[:rows] *= np.float32(8.0)
    P2, beta2, _ = oracle.quantize_weights_groups(W2, G)
    assert beta2[0] == beta[0] * np.float32(8.0) and np.array_equal(P2, P)
    assert np.array_equal(beta2[1:], beta[1:])


def test_weight_groups_rescale_exact():
    r = np.random.default_rng(3)
    acc = r.integers(-2 ** 20, 2 ** 20, (3, 12)).astype(np.int32)
    s = r.uniform(1.0, 300.0, 3).astype(np.float32)
    beta = r.uniform(0.005, 0.05, 4).astype(np.float32)
    Y = oracle.rescale_groups(acc, s, beta)
    for t in range(3):
        for o in range(12):
            exact = Fraction(int(acc[t, o])) * Fraction(float(beta[o // 3])) / Fraction(float(s[t]))
            assert Y[t, o] == np.float32(float(exact))


# ---------------------------------------------------------------- training side

def test_golden_train_fake_quant():
    g = load("train_fake_quant.txt")
    Wl = oracle.fake_quant_weights(np.array(g["W"], np.float32), g["W_lam"])
    assert oracle.bf16_to_f32(Wl).tolist() == g["W_out"]
    Xl, Xq, s, r = oracle.fake_quant_acts(np.array(g["X"], np.float32), flags=oracle.NO_NORM,
                                          lam=g["X_lam"])
    assert oracle.bf16_to_f32(Xl).tolist() == g["X_out"]
    assert [oracle.warmup_lambda(t, 1000) for t in g["lam_steps"]] == g["lam_values"]


def _bf16_brute(v):
    # the two bf16 values around v, the nearer by exact comparison, ties to the even one
    b = np.float32(v).view(np.uint32)
    lo = (int(b) >> 16) & 0xFFFF
    cand = [lo, lo + 1]
    vals = [Fraction(float(np.array([c << 16], np.uint32).view(np.float32)[0])) for c in cand]
    x = Fraction(float(v))
    d0, d1 = abs(x - vals[0]), abs(x - vals[1])
    if d0 < d1 or (d0 == d1 and lo % 2 == 0):
        return lo
    return lo + 1


def test_bf16_rounding_against_brute_force():
    r = np.random.default_rng(8)
    v = (r.standard_normal(3000) * np.exp(r.uniform(-20, 20, 3000))).astype(np.float32)
    # ties and near-ties: patterns with low half exactly 0x8000 and 0x8000 +- 1
    u = r.integers(0, 2 ** 31, 300, dtype=np.int64).astype(np.uint32) & np.uint32(0x7F7F0000)
    ties = np.concatenate([(u | 0x8000), (u | 0x8001), (u | 0x7FFF)]).view(np.float32)
    v = np.concatenate([v, ties, np.array([0.0, -0.0, 1.0, -1.0], np.float32)])
    got = oracle.bf16_bits(v)
    for x, b in zip(v, got):
        assert int(b) == _bf16_brute(x), x
    assert oracle.bf16_bits(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7F80, 0xFF80]
    assert np.isnan(oracle.bf16_to_f32(oracle.bf16_bits(np.array([np.nan], np.float32))))[0]


def test_fake_quant_lambda_limits():
    # lambda = 0: the original values (bf16-rounded); lambda = 1: the dequantized values,
    # exactly where the difference is exact (Sterbenz: within a factor 2), else within one
    # fp32 rounding before the bf16 one
    r = np.random.default_rng(12)
    W = (r.standard_normal((64, 256)) * 0.02).astype(np.float32)
    assert np.array_equal(oracle.fake_quant_weights(W, 0.0), oracle.bf16_bits(W))
    _, beta, _ = oracle.quantize_weights(W)
    deq = (oracle.ternarize(W, beta).astype(np.float32) * beta).astype(np.float32)
    w1 = oracle.bf16_to_f32(oracle.fake_quant_weights(W, 1.0)).astype(np.float64)
    ref = oracle.bf16_to_f32(oracle.bf16_bits(deq)).astype(np.float64)
    tol = 2.0 ** -7 * np.maximum(np.abs(W), np.abs(deq)).astype(np.float64)
    assert np.all(np.abs(w1 - ref) <= tol)
    sterbenz = (deq != 0) & (np.abs(W) <= 2 * np.abs(deq)) & (np.abs(deq) <= 2 * np.abs(W))
    assert np.array_equal(w1[sterbenz], ref[sterbenz])
    X = r.standard_normal((4, 512)).astype(np.float32)
    xl0, Xq, s, _ = oracle.fake_quant_acts(X, lam=0.0)
    assert np.array_equal(xl0, oracle.bf16_bits(oracle.rmsnorm(X)))


def _rmsnorm64(X, g, eps):
    X = np.asarray(X, np.float64)
    r = 1.0 / np.sqrt((X * X).mean(axis=1) + eps)
    return X * r[:, None] * g[None, :]


@pytest.mark.parametrize("with_gain", [False, True])
def test_rmsnorm_backward_finite_differences(with_gain):
    # central differences of the fp64 forward: the loss sum(dY * y(X))
    r = np.random.default_rng(21)
    T, K, eps = 3, 16, 1e-6
    X = r.standard_normal((T, K))
    g = r.uniform(0.5, 1.5, K) if with_gain else np.ones(K)
    dY = r.standard_normal((T, K))
    rr = 1.0 / np.sqrt((X * X).mean(axis=1) + eps)
    dX, dg = oracle.rmsnorm_backward(X, g if with_gain else None, rr, dY)
    h = 1e-6
    for t in range(T):
        for k in range(K):
            Xp, Xm = X.copy(), X.copy()
            Xp[t, k] += h
            Xm[t, k] -= h
            num = (np.sum(dY * _rmsnorm64(Xp, g, eps)) - np.sum(dY * _rmsnorm64(Xm, g, eps))) / (2 * h)
            assert abs(num - dX[t, k]) <= 1e-5 * max(1.0, abs(num))
    if with_gain:
        for k in range(K):
            gp, gm = g.copy(), g.copy()
            gp[k] += h
            gm[k] -= h
            num = (np.sum(dY * _rmsnorm64(X, gp, eps)) - np.sum(dY * _rmsnorm64(X, gm, eps))) / (2 * h)
            assert abs(num - dg[k]) <= 1e-5 * max(1.0, abs(num))


def test_rmsnorm_backward_against_autograd():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(22)
    T, K, eps = 5, 64, 1e-6
    X = r.standard_normal((T, K))
    g = r.uniform(0.5, 1.5, K)
    dY = r.standard_normal((T, K))
    xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    y = xt * torch.rsqrt((xt * xt).mean(dim=1, keepdim=True) + eps) * gt
    y.backward(torch.tensor(dY, dtype=torch.float64))
    rr = 1.0 / np.sqrt((X * X).mean(axis=1) + eps)
    dX, dg = oracle.rmsnorm_backward(X, g, rr, dY)
    assert np.allclose(dX, xt.grad.numpy(), rtol=1e-6, atol=1e-7)
    assert np.allclose(dg, gt.grad.numpy(), rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- BitDelta

def test_golden_bitdelta():
    g = load("bitdelta.txt")
    base = oracle.bf16_bits(np.array(g["W_base"], np.float32))
    bits, alpha, codes = oracle.bitdelta_compress(np.array(g["W_fine"], np.float32), base)
    assert alpha == g["alpha"] and codes.tolist() == g["codes"] and bits.tolist() == g["bits"]
    y = oracle.bitdelta_forward(base, [codes], [alpha], np.array(g["x"], np.float32))
    assert y.tolist() == g["y"]


def test_bitdelta_alpha_is_l2_optimal():
    # [BitDelta] Eq. (3)-(4): with S = Sign(delta), ||delta - a S||^2 is smallest at
    # a = mean |delta| (closed form sum(delta * S) / sum(S * S), and a numerical check)
    r = np.random.default_rng(31)
    base = oracle.bf16_bits((r.standard_normal((64, 256)) * 0.02).astype(np.float32))
    fine = (oracle.bf16_to_f32(base) + r.standard_normal((64, 256)).astype(np.float32) * 0.001
            ).astype(np.float32)
    bits, alpha, codes = oracle.bitdelta_compress(fine, base)
    delta = (fine - oracle.bf16_to_f32(base)).astype(np.float64).ravel()
    s = codes.astype(np.float64).ravel()
    a_star = float(np.dot(delta, s) / np.dot(s, s))
    assert abs(a_star - float(alpha)) <= 2.0 ** -23 * float(alpha)

    def err(a):
        return float(np.sum((delta - a * s) ** 2))

    for d in (1e-2, 1e-4):
        assert err(float(alpha)) <= err(float(alpha) * (1 + d))
        assert err(float(alpha)) <= err(float(alpha) * (1 - d))


def test_bitdelta_interleave_and_forward_dense():
    # the batched layout holds each model's 2-byte groups side by side; the forward
    # equals the dense fp64 product with the dequantized fine-tuned matrices
    r = np.random.default_rng(33)
    B, N, M = 3, 20, 64
    base = oracle.bf16_bits((r.standard_normal((N, M)) * 0.02).astype(np.float32))
    bits, alphas, codes = [], [], []
    for i in range(B):
        fine = (oracle.bf16_to_f32(base) + r.standard_normal((N, M)).astype(np.float32) * 0.002
                ).astype(np.float32)
        b, a, c = oracle.bitdelta_compress(fine, base)
        bits.append(b)
        alphas.append(a)
        codes.append(c)
    inter = oracle.bitdelta_interleave(bits)
    assert inter.shape == (N, M)
    for i in range(8):
        for n in range(N):
            for j in range(M // 16):
                lo, hi = (bits[i][n, 2 * j], bits[i][n, 2 * j + 1]) if i < B else (0, 0)
                assert inter[n, (j * 8 + i) * 2] == lo and inter[n, (j * 8 + i) * 2 + 1] == hi
    X = r.standard_normal((B, M)).astype(np.float32)
    Y = oracle.bitdelta_forward(base, codes, alphas, X)
    for i in range(B):
        dense = oracle.bf16_to_f32(base).astype(np.float64) + float(alphas[i]) * \
            oracle.unpack1(bits[i], M).astype(np.float64)
        assert np.allclose(Y[i].astype(np.float64), dense @ X[i].astype(np.float64),
                           rtol=1e-6, atol=1e-7)
