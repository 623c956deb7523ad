"""CPU oracle of the BitNet b1.58 BitLinear forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package. The HIP product path (``ternary_quantized_linear_amd``)
neither imports it nor shares any code with it.

The arithmetic lives in ``bitlinear_oracle.c`` (plain C loops, built with gcc
``-O2 -ffp-contract=off -fno-fast-math -fopenmp``); this module compiles it on demand
and wraps it with numpy arrays in and out. The header of the C file states, for each
step, the passage of the pages it follows and the precision of every rounding:

  1. gamma = exact sum |W| / (N*K) in fp64, beta = fp32(gamma)
  2. codes = clamp(round_half_even(w * fp32(1/beta)), -1, 1)
  3. four 2-bit codes per byte, u = q + 1, code k = 4j+i in bits [2i+1:2i] of byte j
  4. RMSNorm: r = 1/sqrt(exact sum x^2 / K + eps) in fp64, y = fp32(x * r * g)
  5. s_t = 127 / max(max|y|, 1e-5) in fp32, Xq = clamp(rint(y * s_t), -128, 127)
  6. acc = Xq . codes^T in integers
  7. Y = fp32(acc * beta / s_t) computed in fp64

and the 1-bit sign variant (the original BitNet weight binarization):

  S1. alpha = exact sum W / (N*K) in fp64
  S2. codes = +1 where fp64(w) > alpha, else -1 (Sign(0) = -1)
  S3. beta = fp32(mean |W|) (step 1's scale)
  S4. eight codes per byte, code k = 8j+i in bit i of byte j, set for +1
  S5. acc = Xq . codes^T in integers, Y = fp32(acc * beta / s_t)

and group quantization: G blocks of N/G output rows, each quantized alone (beta_g);
Y[t, o] = fp32(acc * beta_{o // (N/G)} / s_t).

and the training side (fake quantization with the warm-up lambda and the straight-
through estimator), in numpy with the roundings written out:

  T1. lambda = min(step / total, 1)
  T2. W_lam = bf16(W + lam * (beta * q - W)), every operation one fp32 rounding
  T3. x_lam = bf16(y + lam * (Xq / s - y)) with y the RMSNorm output, Xq / s one fp32
      division; r = 1/rms per token kept for the backward
  T4. STE: the gradient of the quantizer output is passed to its input unchanged; the
      RMSNorm backward in fp64: dx = r g dy - x r^3 (sum g dy x) / K, dg = sum_t r dy x

and BitDelta (a base model plus per-model 1-bit deltas, numpy):

  D1. delta = fp32(W_fine - W_base); alpha = fp32(exact sum |delta| / (N*M))
  D2. codes = +1 where delta > 0, else -1; eight per byte as in S4; a batch of up to 8
      models interleaves the codes per 16-code group (2 bytes per model slot, 8 slots)
  D3. Y[i, n] = sum_k base[n,k] x[i,k] + alpha_i sum_k c_i[n,k] x[i,k], in fp64

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute force in exact rationals, library routines, closed forms, invariants and the
worked examples under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

NO_NORM = 0x1

_ERRORS = {
    -1: "non-finite input",
    -2: "bad dimensions",
    -3: "out of memory",
    -4: "invalid packed code (0b11) or code outside {-1,0,1}",
    -5: "accumulator outside int32",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            sig = {
                "orc_set_threads": [ctypes.c_int],
                "orc_abs_sum": [P, I64, P],
                "orc_sum_sq": [P, I64, P],
                "orc_weight_scale": [P, I64, I64, P, P],
                "orc_ternarize": [P, I64, ctypes.c_float, P],
                "orc_pack": [P, I64, I64, P],
                "orc_unpack": [P, I64, I64, P],
                "orc_quantize_weights": [P, I64, I64, P, P, P],
                "orc_rmsnorm": [P, P, I64, I64, ctypes.c_float, P],
                "orc_absmax_quant": [P, I64, I64, P, P],
                "orc_quantize_acts": [P, P, I64, I64, ctypes.c_float, ctypes.c_uint32, P, P],
                "orc_product": [P, P, I64, I64, I64, P],
                "orc_rescale": [P, P, ctypes.c_float, I64, I64, P],
                "orc_forward": [P, P, I64, I64, P, ctypes.c_float, I64, P, P],
                "orc_quantize_weights_groups": [P, I64, I64, I64, P, P, P],
                "orc_rescale_groups": [P, P, P, I64, I64, I64, P],
                "orc_sum": [P, I64, P],
                "orc_sign_codes": [P, I64, ctypes.c_double, P],
                "orc_sign_weights": [P, I64, I64, P, P, P, P],
                "orc_pack1": [P, I64, I64, P],
                "orc_unpack1": [P, I64, I64, P],
                "orc_product_sign": [P, P, I64, I64, I64, P],
                "orc_forward_sign": [P, P, I64, I64, P, ctypes.c_float, I64, P, P],
            }
            for name, args in sig.items():
                f = getattr(lib, name)
                f.argtypes = args
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(st):
    if st != 0:
        raise OracleError(_ERRORS.get(st, "oracle error %d" % st))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (0 keeps it); returns the count in effect."""
    return _load().orc_set_threads(int(n))


def abs_sum(w) -> float:
    """Exact sum of |w| rounded once to fp64."""
    w = _f32(w)
    out = ctypes.c_double()
    _check(_load().orc_abs_sum(_ptr(w), w.size, ctypes.addressof(out)))
    return out.value


def sum_sq(x) -> float:
    """Exact sum of x^2 rounded once to fp64."""
    x = _f32(x)
    out = ctypes.c_double()
    _check(_load().orc_sum_sq(_ptr(x), x.size, ctypes.addressof(out)))
    return out.value


def weight_scale(W):
    """Returns (gamma64, beta32) of W [N, K]."""
    W = _f32(W)
    N, K = W.shape
    g = ctypes.c_double()
    b = ctypes.c_float()
    _check(_load().orc_weight_scale(_ptr(W), N, K, ctypes.addressof(g), ctypes.addressof(b)))
    return g.value, np.float32(b.value)


def ternarize(W, beta):
    W = _f32(W)
    q = np.empty(W.shape, dtype=np.int8)
    _check(_load().orc_ternarize(_ptr(W), W.size, float(np.float32(beta)), _ptr(q)))
    return q


def pack(q):
    q = np.ascontiguousarray(q, dtype=np.int8)
    N, K = q.shape
    P = np.empty((N, K // 4), dtype=np.uint8)
    _check(_load().orc_pack(_ptr(q), N, K, _ptr(P)))
    return P


def unpack(P, K):
    P = np.ascontiguousarray(P, dtype=np.uint8)
    N = P.shape[0]
    q = np.empty((N, K), dtype=np.int8)
    _check(_load().orc_unpack(_ptr(P), N, K, _ptr(q)))
    return q


def quantize_weights(W):
    """W [N, K] fp32 -> (packed uint8 [N, K/4], beta fp32, gamma fp64)."""
    W = _f32(W)
    N, K = W.shape
    P = np.empty((N, K // 4), dtype=np.uint8)
    b = ctypes.c_float()
    g = ctypes.c_double()
    _check(_load().orc_quantize_weights(_ptr(W), N, K, _ptr(P), ctypes.addressof(b),
                                        ctypes.addressof(g)))
    return P, np.float32(b.value), g.value


def rmsnorm(X, gain=None, eps=1e-6):
    X = _f32(X)
    T, K = X.shape
    g = None if gain is None else _f32(gain)
    Y = np.empty_like(X)
    _check(_load().orc_rmsnorm(_ptr(X), _ptr(g), T, K, float(np.float32(eps)), _ptr(Y)))
    return Y


def absmax_quant(Y):
    Y = _f32(Y)
    T, K = Y.shape
    q = np.empty((T, K), dtype=np.int8)
    s = np.empty(T, dtype=np.float32)
    _check(_load().orc_absmax_quant(_ptr(Y), T, K, _ptr(q), _ptr(s)))
    return q, s


def quantize_acts(X, gain=None, eps=1e-6, flags=0):
    """X [T, K] fp32 -> (Xq int8 [T, K], x_scale fp32 [T])."""
    X = _f32(X)
    T, K = X.shape
    g = None if gain is None else _f32(gain)
    q = np.empty((T, K), dtype=np.int8)
    s = np.empty(T, dtype=np.float32)
    _check(_load().orc_quantize_acts(_ptr(X), _ptr(g), T, K, float(np.float32(eps)),
                                     int(flags), _ptr(q), _ptr(s)))
    return q, s


def product(Xq, P, K):
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    T = Xq.shape[0]
    N = P.shape[0]
    acc = np.empty((T, N), dtype=np.int32)
    _check(_load().orc_product(_ptr(Xq), _ptr(P), T, N, K, _ptr(acc)))
    return acc


def rescale(acc, s, beta):
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s = _f32(s)
    T, N = acc.shape
    Y = np.empty((T, N), dtype=np.float32)
    _check(_load().orc_rescale(_ptr(acc), _ptr(s), float(np.float32(beta)), T, N, _ptr(Y)))
    return Y


def forward(Xq, s, P, beta):
    """(Xq [T,K], s [T], packed [N,K/4], beta) -> (Y fp32 [T,N], acc int32 [T,N])."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    s = _f32(s)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    T, K = Xq.shape
    N = P.shape[0]
    Y = np.empty((T, N), dtype=np.float32)
    acc = np.empty((T, N), dtype=np.int32)
    _check(_load().orc_forward(_ptr(Xq), _ptr(s), T, K, _ptr(P), float(np.float32(beta)), N,
                               _ptr(Y), _ptr(acc)))
    return Y, acc


def bitlinear(X, W, gain=None, eps=1e-6, flags=0):
    """The whole forward from fp32 X [T,K] and fp32 W [N,K]; returns a dict of stages."""
    P, beta, gamma = quantize_weights(W)
    Xq, s = quantize_acts(X, gain, eps, flags)
    Y, acc = forward(Xq, s, P, beta)
    return {"packed": P, "beta": beta, "gamma": gamma, "Xq": Xq, "x_scale": s,
            "acc": acc, "Y": Y}


# ---------------------------------------------------------------- sign variant

def exact_sum(w) -> float:
    """Exact signed sum rounded once to fp64."""
    w = _f32(w)
    out = ctypes.c_double()
    _check(_load().orc_sum(_ptr(w), w.size, ctypes.addressof(out)))
    return out.value


def sign_codes(W, alpha):
    W = _f32(W)
    c = np.empty(W.shape, dtype=np.int8)
    _check(_load().orc_sign_codes(_ptr(W), W.size, float(alpha), _ptr(c)))
    return c


def sign_weights(W):
    """W [N, K] fp32 -> (codes int8 [N, K] in {-1, +1}, alpha fp64, gamma fp64, beta fp32)."""
    W = _f32(W)
    N, K = W.shape
    c = np.empty((N, K), dtype=np.int8)
    a = ctypes.c_double()
    g = ctypes.c_double()
    b = ctypes.c_float()
    _check(_load().orc_sign_weights(_ptr(W), N, K, _ptr(c), ctypes.addressof(a),
                                    ctypes.addressof(g), ctypes.addressof(b)))
    return c, a.value, g.value, np.float32(b.value)


def pack1(c):
    c = np.ascontiguousarray(c, dtype=np.int8)
    N, K = c.shape
    P = np.empty((N, K // 8), dtype=np.uint8)
    _check(_load().orc_pack1(_ptr(c), N, K, _ptr(P)))
    return P


def unpack1(P, K):
    P = np.ascontiguousarray(P, dtype=np.uint8)
    N = P.shape[0]
    c = np.empty((N, K), dtype=np.int8)
    _check(_load().orc_unpack1(_ptr(P), N, K, _ptr(c)))
    return c


def product_sign(Xq, P, K):
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    T = Xq.shape[0]
    N = P.shape[0]
    acc = np.empty((T, N), dtype=np.int32)
    _check(_load().orc_product_sign(_ptr(Xq), _ptr(P), T, N, K, _ptr(acc)))
    return acc


def forward_sign(Xq, s, P, beta):
    """(Xq [T,K], s [T], packed bits [N,K/8], beta) -> (Y fp32 [T,N], acc int32 [T,N])."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    s = _f32(s)
    P = np.ascontiguousarray(P, dtype=np.uint8)
    T, K = Xq.shape
    N = P.shape[0]
    Y = np.empty((T, N), dtype=np.float32)
    acc = np.empty((T, N), dtype=np.int32)
    _check(_load().orc_forward_sign(_ptr(Xq), _ptr(s), T, K, _ptr(P), float(np.float32(beta)),
                                    N, _ptr(Y), _ptr(acc)))
    return Y, acc


def bitlinear_sign(X, W, gain=None, eps=1e-6, flags=0):
    """The 1-bit sign forward from fp32 X [T,K] and W [N,K]; returns a dict of stages."""
    c, alpha, gamma, beta = sign_weights(W)
    P = pack1(c)
    Xq, s = quantize_acts(X, gain, eps, flags)
    Y, acc = forward_sign(Xq, s, P, beta)
    return {"packed": P, "codes": c, "alpha": alpha, "beta": beta, "gamma": gamma, "Xq": Xq,
            "x_scale": s, "acc": acc, "Y": Y}


# ---------------------------------------------------------------- group quantization

def quantize_weights_groups(W, G):
    """W [N, K] fp32, G | N -> (packed [N, K/4], beta fp32 [G], gamma fp64 [G])."""
    W = _f32(W)
    N, K = W.shape
    P = np.empty((N, K // 4), dtype=np.uint8)
    b = np.empty(G, dtype=np.float32)
    g = np.empty(G, dtype=np.float64)
    _check(_load().orc_quantize_weights_groups(_ptr(W), N, K, int(G), _ptr(P), _ptr(b), _ptr(g)))
    return P, b, g


def rescale_groups(acc, s, beta):
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s = _f32(s)
    beta = _f32(beta)
    T, N = acc.shape
    Y = np.empty((T, N), dtype=np.float32)
    _check(_load().orc_rescale_groups(_ptr(acc), _ptr(s), _ptr(beta), T, N, beta.size, _ptr(Y)))
    return Y


def bitlinear_groups(X, W, G, gain=None, eps=1e-6, flags=0):
    """The forward with G weight scale groups; returns a dict of stages."""
    P, beta, gamma = quantize_weights_groups(W, G)
    Xq, s = quantize_acts(X, gain, eps, flags)
    acc = product(Xq, P, W.shape[1])
    return {"packed": P, "beta": beta, "gamma": gamma, "Xq": Xq, "x_scale": s, "acc": acc,
            "Y": rescale_groups(acc, s, beta)}


# ---------------------------------------------------------------- training side (numpy)
# [HF-1.58] "Training with the straight-through estimator (STE)": round() has no useful
# gradient, so its gradient is taken as 1 and gradients flow as through the identity.
# [HF-1.58] "Dynamic warm-up quantization": lambda = min(step / total_steps, 1) scales
# the difference between the quantized and the original values (0: full precision,
# 1: fully quantized). [HF-1.58] "How quantization works": the quantized weights and
# activations are rescaled back (dequantized) after rounding.

def warmup_lambda(step, total):
    """T1: min(step / total, 1), in fp64."""
    if total <= 0:
        raise OracleError("bad dimensions")
    return min(float(step) / float(total), 1.0)


def bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even (the top 16
    bits of the fp32 pattern, plus one unit where the dropped 16 bits exceed half, or
    equal half with an odd kept part). NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & np.uint64(1)) == 1))
    out = (keep + up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(x)
    out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint32)
    return out.astype(np.uint16)


def bf16_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def fake_quant_weights(W, lam):
    """T2: W [N, K] fp32, lam -> bf16 bits [N, K] of W + lam * (beta * q - W)."""
    W = _f32(W)
    N, K = W.shape
    _, beta, _ = quantize_weights(W)
    q = ternarize(W, beta)
    wq = (q.astype(np.float32) * np.float32(beta)).astype(np.float32)  # exact: q in {-1,0,1}
    d = (wq - W).astype(np.float32)
    m = (W + (np.float32(lam) * d).astype(np.float32)).astype(np.float32)
    return bf16_bits(m)


def rms_inv(X, eps=1e-6, flags=0):
    """1 / sqrt(exact sum x^2 / K + eps) per token in fp64 (1 with NO_NORM)."""
    X = _f32(X)
    T, K = X.shape
    if flags & NO_NORM:
        return np.ones(T, np.float64)
    return np.array([1.0 / np.sqrt(sum_sq(X[t]) / K + float(np.float32(eps))) for t in range(T)])


def fake_quant_acts(X, gain=None, eps=1e-6, flags=0, lam=1.0):
    """T3: -> (bf16 bits [T, K] of y + lam * (Xq / s - y), Xq, s, r)."""
    X = _f32(X)
    y = X.copy() if flags & NO_NORM else rmsnorm(X, gain, eps)
    Xq, s = absmax_quant(y)
    xd = (Xq.astype(np.float32) / s[:, None]).astype(np.float32)  # one fp32 division
    d = (xd - y).astype(np.float32)
    m = (y + (np.float32(lam) * d).astype(np.float32)).astype(np.float32)
    return bf16_bits(m), Xq, s, rms_inv(X, eps, flags)


def rmsnorm_backward(X, gain, r, dY):
    """T4 (the norm part; the quantizers pass gradients through): dX [T, K] fp32 and
    dgain [K] fp32 (None without gain), all arithmetic in fp64, one rounding each."""
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    r = np.asarray(r, np.float64)
    T, K = X.shape
    g = np.ones(K) if gain is None else np.asarray(gain, np.float64)
    gdy = dY * g[None, :]
    c = np.array([math_fsum(gdy[t] * X[t]) for t in range(T)])
    dX = r[:, None] * gdy - X * (r ** 3 * c / K)[:, None]
    dg = None if gain is None else np.array([math_fsum(dY[:, k] * X[:, k] * r) for k in range(K)])
    return dX.astype(np.float32), (None if dg is None else dg.astype(np.float32))


def math_fsum(v):
    import math
    return math.fsum(np.asarray(v, np.float64).tolist())


# ---------------------------------------------------------------- BitDelta (numpy)
# [BitDelta] "BitDelta: Your Fine-Tune May Only Be Worth One Bit": Eq. (1) the delta of
# a fine-tuned model is approximated by alpha times its sign; Eq. (2) Sign(W) = +1 for
# W > 0 and -1 otherwise; Eq. (4) alpha = the mean of |delta| over all n*m entries, the
# minimizer of the L2 error of Eq. (3); Eq. (6) the fine-tuned product is the base
# product plus the 1-bit delta product.

def bitdelta_compress(W_fine, W_base_bf16):
    """W_fine fp32 [N, M], base as bf16 bits [N, M] -> (sign bits [N, M/8] (S4 layout),
    alpha fp32, codes int8 [N, M])."""
    W_fine = _f32(W_fine)
    base = bf16_to_f32(W_base_bf16)
    delta = (W_fine - base).astype(np.float32)
    codes = np.where(delta > 0, 1, -1).astype(np.int8)
    alpha = np.float32(abs_sum(delta) / float(delta.size))
    return pack1(codes), alpha, codes


def bitdelta_interleave(bits_list):
    """Per-model sign bits [N, M/8] (B <= 8 of them) -> the batched layout [N, M/16, 8, 2]
    (slots past B zero)."""
    N, mb = bits_list[0].shape
    out = np.zeros((N, mb // 2, 8, 2), np.uint8)
    for i, b in enumerate(bits_list):
        out[:, :, i, :] = np.asarray(b, np.uint8).reshape(N, mb // 2, 2)
    return out.reshape(N, -1)


def bitdelta_forward(W_base_bf16, codes_list, alphas, X):
    """Y [B, N] fp32 = base . x_i + alpha_i * codes_i . x_i, computed in fp64."""
    base = bf16_to_f32(W_base_bf16).astype(np.float64)
    X = np.asarray(X, np.float64)
    B = X.shape[0]
    Y = np.empty((B, base.shape[0]), np.float64)
    for i in range(B):
        Y[i] = base @ X[i] + float(alphas[i]) * (np.asarray(codes_list[i], np.float64) @ X[i])
    return Y.astype(np.float32)
