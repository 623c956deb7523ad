"""Argument checks of the Python binding, without a GPU.

The binding hands raw pointers and sizes to the C ABI, which cannot see dtypes, strides
or buffer lengths. Every mirror of an ABI call must therefore reject a wrong dtype, a
non-contiguous view, a shape that disagrees with the sizes it passes, or a tensor off
the GPU with ValueError, before any call into the library. Here the library's entry
points are replaced by recorders, so a check that let a bad argument through shows up
as a recorded call (CPU tensors are used throughout; the last check every call makes is
that its tensors sit on one GPU).
"""
import os

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "ternary_quantized_linear_amd", "libbitlinear.so")


@pytest.fixture(scope="module")
def bl():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    import ternary_quantized_linear_amd as m
    return m


@pytest.fixture
def calls(bl, monkeypatch):
    made = []
    for name in dir(bl):
        if name.startswith("_c_") and name not in ("_c_str", "_c_err", "_c_ver", "_c_fw_wsb",
                                                   "_c_ws_bytes", "_c_choice", "_c_choice_ws",
                                                   "_c_lam"):
            monkeypatch.setattr(bl, name, lambda *a, _n=name: made.append(_n) or 0)
    return made


def proj(T=2, N=8, K=64, cpb=4):
    return dict(Xq=torch.zeros((T, K), dtype=torch.int8), x_scale=torch.ones(T),
                W_packed=torch.zeros((N, K // cpb), dtype=torch.uint8), w_scale=torch.ones(1),
                Y=torch.empty((T, N)), acc=torch.empty((T, N), dtype=torch.int32))


def fwd(bl, p):
    bl.bitlinear_forward(p["Xq"], p["x_scale"], p["W_packed"], p["w_scale"], p["Y"], p["acc"])


def test_consistent_cpu_tensors_are_refused_as_off_gpu(bl, calls):
    with pytest.raises(ValueError, match="GPU"):
        fwd(bl, proj())
    assert calls == []


@pytest.mark.parametrize("field,bad,msg", [
    ("Xq", torch.zeros((2, 64), dtype=torch.uint8), "dtype"),
    ("Xq", torch.zeros((2, 64), dtype=torch.float32), "dtype"),
    ("x_scale", torch.ones(2, dtype=torch.float64), "dtype"),
    ("x_scale", torch.ones(1), "elements"),
    ("W_packed", torch.zeros((8, 15), dtype=torch.uint8), "bytes per row"),
    ("W_packed", torch.zeros((8, 16), dtype=torch.int8), "dtype"),
    ("W_packed", torch.zeros(128, dtype=torch.uint8), "dimensions"),
    ("w_scale", torch.ones(0), "elements"),
    ("Y", torch.empty((2, 7)), "elements"),
    ("Y", torch.empty((2, 8), dtype=torch.float16), "dtype"),
    ("acc", torch.empty((2, 8), dtype=torch.int64), "dtype"),
    ("acc", torch.empty((1, 8), dtype=torch.int32), "elements"),
])
def test_forward_rejects_mismatched_arguments(bl, calls, field, bad, msg):
    p = proj()
    p[field] = bad
    with pytest.raises(ValueError, match=msg):
        fwd(bl, p)
    assert calls == []


def test_forward_rejects_strided_views(bl, calls):
    p = proj()
    p["Xq"] = torch.zeros((2, 128), dtype=torch.int8)[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        fwd(bl, p)
    p = proj()
    p["Y"] = torch.empty((8, 2)).t()
    with pytest.raises(ValueError, match="contiguous"):
        fwd(bl, p)
    p = proj()
    p["W_packed"] = torch.zeros((16, 16), dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        fwd(bl, p)
    assert calls == []


def test_every_forward_variant_checks(bl, calls):
    p = proj()
    p["Y"] = torch.empty((2, 4))
    args = (p["Xq"], p["x_scale"], p["W_packed"], p["w_scale"], p["Y"], None)
    for f in (lambda: bl.bitlinear_forward_ex(*args, kernel="skinny"),
              lambda: bl.bitlinear_forward_ws(*args, workspace=None),
              lambda: bl.bitlinear_forward_grouped([args], 2),
              lambda: bl.bitlinear_forward_grouped_ws([args], 2, None),
              lambda: bl.prepare_forward_grouped([args], 2),
              lambda: bl.bitlinear_forward_scale_groups(*args[:4], 1, p["Y"]),
              lambda: bl.bitlinear_forward_grouped_scale_groups([args], [1], 2)):
        with pytest.raises(ValueError):
            f()
    # a grouped call whose T disagrees with an entry's token count
    q = proj(T=3)
    with pytest.raises(ValueError, match="tokens"):
        bl.bitlinear_forward_grouped([(q["Xq"], q["x_scale"], q["W_packed"], q["w_scale"],
                                       q["Y"], None)], 2)
    # scale groups: w_scale must hold one scale per group
    q = proj(N=8)
    with pytest.raises(ValueError, match="elements"):
        bl.bitlinear_forward_scale_groups(q["Xq"], q["x_scale"], q["W_packed"], q["w_scale"], 4,
                                          q["Y"])
    with pytest.raises(ValueError, match="one scale-group count"):
        bl.bitlinear_forward_grouped_scale_groups(
            [(q["Xq"], q["x_scale"], q["W_packed"], q["w_scale"], q["Y"], None)], [1, 2], 2)
    # grouped calls: 1..8 entries
    with pytest.raises(ValueError, match="1..8"):
        bl.bitlinear_forward_grouped([], 2)
    assert calls == []


def test_sign_products_need_eight_codes_per_byte(bl, calls):
    p = proj(cpb=4)   # K / 4 bytes per row: the 2-bit layout, not the 1-bit one
    with pytest.raises(ValueError, match="bytes per row"):
        bl.bitlinear_forward_sign(p["Xq"], p["x_scale"], p["W_packed"], p["w_scale"], p["Y"])
    with pytest.raises(ValueError, match="bytes per row"):
        bl.prepare_forward_sign_grouped([(p["Xq"], p["x_scale"], p["W_packed"], p["w_scale"],
                                          p["Y"], None)], 2)
    assert calls == []


def test_activation_quantizer_checks(bl, calls):
    X = torch.zeros((4, 64))
    Xq = torch.zeros((4, 64), dtype=torch.int8)
    xs = torch.ones(4)
    for bad in [dict(X=torch.zeros((4, 64), dtype=torch.float64)),
                dict(X=torch.zeros((4, 128))[:, ::2]),
                dict(Xq=torch.zeros((4, 60), dtype=torch.int8)),
                dict(Xq=torch.zeros((4, 64), dtype=torch.uint8)),
                dict(xs=torch.ones(3)),
                dict(gain=torch.ones(63))]:
        a = dict(X=X, gain=None, Xq=Xq, xs=xs)
        a.update(bad)
        with pytest.raises(ValueError):
            bl.bitlinear_quantize_acts(a["X"], a["gain"], 1e-6, 0, a["Xq"], a["xs"])
        with pytest.raises(ValueError):
            bl.prepare_quantize_acts_grouped([(a["X"], a["gain"], a["Xq"], a["xs"])], 4)
    with pytest.raises(ValueError, match="tokens"):
        bl.bitlinear_quantize_acts_grouped([(X, None, Xq, xs)], 2, 1e-6, 0)
    assert calls == []


def test_weight_quantizer_checks(bl, calls):
    W = torch.zeros((8, 64))
    P = torch.zeros((8, 16), dtype=torch.uint8)
    b = torch.ones(1)
    ws = torch.zeros(1024, dtype=torch.uint8)
    for args, msg in [((W, torch.zeros((8, 15), dtype=torch.uint8), b, None, ws), "shape"),
                      ((W.double(), P, b, None, ws), "dtype"),
                      ((W, P, torch.ones(0), None, ws), "elements"),
                      ((W, P, b, torch.ones(1), ws), "dtype"),      # gamma must be fp64
                      ((W, P, b, None, None), "required"),
                      ((W, P, b, None, torch.zeros(256, dtype=torch.int32)), "dtype"),
                      ((torch.zeros((8, 62)), P, b, None, ws), "multiple")]:
        with pytest.raises(ValueError, match=msg):
            bl.bitlinear_quantize_weights(*args)
    with pytest.raises(ValueError, match="shape"):
        bl.bitlinear_quantize_weights_sign(W, P, b, None, ws)      # needs [N, K / 8]
    with pytest.raises(ValueError, match="elements"):
        bl.bitlinear_quantize_weights_scale_groups(W, 4, P, b, None, ws)
    assert calls == []


def test_training_and_bitdelta_checks(bl, calls):
    W = torch.zeros((8, 64))
    with pytest.raises(ValueError, match="shape"):
        bl.bitlinear_fake_quant_weights(W, torch.ones(1), 0.5,
                                        torch.empty((8, 32), dtype=torch.bfloat16))
    X = torch.zeros((4, 64))
    with pytest.raises(ValueError, match="dtype"):
        bl.bitlinear_fake_quant_acts(X, None, 1e-6, 0, 0.5, torch.zeros((4, 64), dtype=torch.int8),
                                     torch.ones(4), torch.empty((4, 64)), None)
    with pytest.raises(ValueError, match="elements"):
        bl.bitlinear_rmsnorm_backward(X, None, torch.ones(3, dtype=torch.float64), X, X.clone())
    base = torch.zeros((8, 64), dtype=torch.int16)
    D = torch.zeros((8, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="features"):
        bl.bitlinear_bitdelta_forward(base, D, torch.ones(2), torch.zeros((2, 32)),
                                      torch.empty((2, 8)))
    with pytest.raises(ValueError, match="elements"):
        bl.bitlinear_bitdelta_forward(base, D, torch.ones(1), torch.zeros((2, 64)),
                                      torch.empty((2, 8)))
    with pytest.raises(ValueError, match="shape"):
        bl.bitlinear_bitdelta_compress(torch.zeros((8, 64)), base, 2, 0,
                                       torch.zeros((8, 8), dtype=torch.uint8), torch.ones(2),
                                       torch.zeros(64, dtype=torch.uint8))
    assert calls == []
