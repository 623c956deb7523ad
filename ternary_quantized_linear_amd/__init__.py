"""Python binding of libbitlinear.so, the BitNet b1.58 BitLinear forward on MI355X.

Argument marshalling only: every step runs in the library's HIP kernels. torch
provides device memory and the current stream; no computation happens here. The
functions named ``bitlinear_*`` mirror the C ABI of include/bitlinear.h one to one
(tensors in place of pointers); ``quantize_weights``, ``quantize_acts``, ``forward``
and ``BitLinear`` allocate their outputs and call them.

If the shared library is missing, importing this package raises ImportError: there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BitLinearError", "lib_path", "bitlinear_weight_workspace_bytes",
    "bitlinear_quantize_weights", "bitlinear_quantize_acts",
    "bitlinear_quantize_acts_grouped", "bitlinear_forward", "bitlinear_forward_ex",
    "bitlinear_forward_choice", "bitlinear_forward_grouped", "bitlinear_status_str",
    "bitlinear_forward_workspace_bytes", "bitlinear_forward_ws", "bitlinear_forward_grouped_ws",
    "bitlinear_last_hip_error", "bitlinear_abi_version", "quantize_weights",
    "quantize_acts", "forward", "BitLinear", "KERNELS", "NO_NORM", "MAX_K", "MAX_GROUP",
    "prepare_forward_grouped", "prepare_quantize_acts_grouped",
    "bitlinear_forward_grouped_noalloc", "NOALLOC_SCRATCH_BYTES",
    "bitlinear_roof_read", "bitlinear_roof_mfma_i8", "ROOF_READ_SINK_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libbitlinear.so")

NO_NORM = 0x1
MAX_K = 132104
MAX_GROUP = 8
ABI_VERSION = 1
KERNELS = {"auto": 0, "gemv": 1, "skinny": 2, "prefill": 3, "generic": 4}
_KERNEL_NAMES = {v: k for k, v in KERNELS.items()}

if not os.path.exists(lib_path):
    raise ImportError(
        "libbitlinear.so is not built (%s); run ternary_quantized_linear_amd/build.py or "
        "__graft_entry__.build()" % lib_path)

_lib = ctypes.CDLL(lib_path)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class _ActDesc(ctypes.Structure):
    _fields_ = [("X", _P), ("gain", _P), ("Xq", _P), ("x_scale", _P), ("K", _I64)]


class _ProjDesc(ctypes.Structure):
    _fields_ = [("Xq", _P), ("x_scale", _P), ("W_packed", _P), ("w_scale", _P),
                ("Y", _P), ("acc", _P), ("N", _I64), ("K", _I64)]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_c_ws_bytes = _sig("bitlinear_weight_workspace_bytes", [_I64, _I64], ctypes.c_size_t)
_c_qw = _sig("bitlinear_quantize_weights", [_P, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P])
_c_qa = _sig("bitlinear_quantize_acts",
             [_P, _P, _I64, _I64, ctypes.c_float, ctypes.c_uint32, _P, _P, _P])
_c_qag = _sig("bitlinear_quantize_acts_grouped",
              [ctypes.POINTER(_ActDesc), ctypes.c_int, _I64, ctypes.c_float, ctypes.c_uint32, _P])
_c_fw = _sig("bitlinear_forward", [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P])
_c_fwx = _sig("bitlinear_forward_ex",
              [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, ctypes.c_int, _P])
_c_choice = _sig("bitlinear_forward_choice", [_I64, _I64, _I64])
_c_fw_wsb = _sig("bitlinear_forward_workspace_bytes", [_I64, _I64, _I64], ctypes.c_size_t)
_c_fw_ws = _sig("bitlinear_forward_ws", [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, ctypes.c_int,
                                         _P, ctypes.c_size_t, _P])
_c_fwg_na = _sig("bitlinear_forward_grouped_noalloc",
                 [ctypes.POINTER(_ProjDesc), ctypes.c_int, _I64, _P])
_c_choice_ws = _sig("bitlinear_forward_choice_ws", [_I64, _I64, _I64, ctypes.c_size_t])
_c_fwg = _sig("bitlinear_forward_grouped", [ctypes.POINTER(_ProjDesc), ctypes.c_int, _I64, _P])
_c_fwg_ws = _sig("bitlinear_forward_grouped_ws",
                 [ctypes.POINTER(_ProjDesc), ctypes.c_int, _I64, _P, ctypes.c_size_t, _P])
_c_qws = _sig("bitlinear_quantize_weights_sign",
              [_P, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P])
_c_fws = _sig("bitlinear_forward_sign", [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P])
_c_fwsg = _sig("bitlinear_forward_sign_grouped",
               [ctypes.POINTER(_ProjDesc), ctypes.c_int, _I64, _P])
_c_qwsg = _sig("bitlinear_quantize_weights_scale_groups",
               [_P, _I64, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P])
_c_fwsg_scale = _sig("bitlinear_forward_scale_groups",
                     [_P, _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, ctypes.c_int, _P])
_c_fwg_scale = _sig("bitlinear_forward_grouped_scale_groups",
                    [ctypes.POINTER(_ProjDesc), ctypes.POINTER(_I64), ctypes.c_int, _I64, _P])
_c_lam = _sig("bitlinear_warmup_lambda", [_I64, _I64], ctypes.c_float)
_c_fqw = _sig("bitlinear_fake_quant_weights", [_P, _I64, _I64, _P, ctypes.c_float, _P, _P])
_c_fqa = _sig("bitlinear_fake_quant_acts",
              [_P, _P, _I64, _I64, ctypes.c_float, ctypes.c_uint32, ctypes.c_float, _P, _P, _P,
               _P, _P])
_c_rbw = _sig("bitlinear_rmsnorm_backward", [_P, _P, _P, _P, _I64, _I64, _P, _P, _P])
_c_bdc = _sig("bitlinear_bitdelta_compress",
              [_P, _P, _I64, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P])
_c_bdf = _sig("bitlinear_bitdelta_forward",
              [_P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P, _P])
_c_roof_read = _sig("bitlinear_roof_read",
                    [ctypes.POINTER(_P), ctypes.POINTER(_I64), ctypes.c_int, ctypes.c_int, _P, _P])
_c_roof_mfma = _sig("bitlinear_roof_mfma_i8", [ctypes.c_int, ctypes.c_int, _P, _P, _P])
_c_str = _sig("bitlinear_status_str", [ctypes.c_int], ctypes.c_char_p)
_c_err = _sig("bitlinear_last_hip_error", [], ctypes.c_char_p)
_c_ver = _sig("bitlinear_abi_version", [])


class BitLinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = "%s: %s" % (where, _c_str(status).decode())
        if status == 6:
            msg += " (%s)" % _c_err().decode()
        super().__init__(msg)
        self.status = status


def _check(status, where):
    if status != 0:
        raise BitLinearError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ---------------------------------------------------------------- argument checks
# The C ABI sees raw pointers and sizes; the sizes it gets are taken from these tensors.
# So before any call, every tensor must have the dtype the ABI reads through its pointer,
# be contiguous (the ABI assumes dense row-major arrays), sit on the same GPU, and agree
# with the sizes passed: a short or strided buffer would otherwise be read or written
# past its end on the device.

_U8, _I8, _I16, _I32 = torch.uint8, torch.int8, torch.int16, torch.int32
_F32, _F64, _BF16 = torch.float32, torch.float64, torch.bfloat16


def _arg(t, name, dtypes, shape=None, numel=None, optional=False, min_numel=None):
    """Checks one tensor argument (None is allowed only when optional); numel: exactly
    that many elements, min_numel: at least that many (a table read by index)."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected %s"
                         % (name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (got strides %s for shape %s)"
                         % (name, tuple(t.stride()), tuple(t.shape)))
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if numel is not None and t.numel() != int(numel):
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), int(numel)))
    if min_numel is not None and t.numel() < int(min_numel):
        raise ValueError("%s has %d elements, expected at least %d"
                         % (name, t.numel(), int(min_numel)))


def _dims(t, name, nd):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.dim() != nd:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, nd, tuple(t.shape)))
    return tuple(int(v) for v in t.shape)


def _same_gpu(*tensors):
    """Every given tensor on one GPU (checked after dtypes and shapes)."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU, got device %s" % dev)
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check_proj(Xq, x_scale, W, w_scale, Y, acc, codes_per_byte=4, n_scales=1, T=None):
    """A product's arguments: Xq int8 [T, K], x_scale fp32 [T], W uint8 [N, K/cpb],
    w_scale fp32 [n_scales], Y fp32 [T, N], acc int32 [T, N] or None -> (T, N, K)."""
    T0, K = _dims(Xq, "Xq", 2)
    if T is not None and T0 != T:
        raise ValueError("Xq has %d tokens, the call is for %d" % (T0, T))
    N, kb = _dims(W, "W_packed", 2)
    _arg(Xq, "Xq", _I8)
    if K % codes_per_byte or kb != K // codes_per_byte:
        raise ValueError("W_packed has %d bytes per row; K = %d needs %s"
                         % (kb, K, "K / %d" % codes_per_byte))
    _arg(W, "W_packed", _U8)
    _arg(x_scale, "x_scale", _F32, min_numel=T0)
    _arg(w_scale, "w_scale", _F32, min_numel=n_scales)   # scale g read at index g
    _arg(Y, "Y", _F32, numel=T0 * N)
    _arg(acc, "acc", _I32, numel=T0 * N, optional=True)
    _same_gpu(Xq, x_scale, W, w_scale, Y, acc)
    return T0, N, K


def _check_entries(entries, T, codes_per_byte=4, groups=None):
    if len(entries) < 1 or len(entries) > MAX_GROUP:
        raise ValueError("a grouped call takes 1..%d entries, got %d" % (MAX_GROUP, len(entries)))
    dev = None
    for i, (Xq, xs, Wp, ws, Y, acc) in enumerate(entries):
        n_scales = 1 if groups is None else int(groups[i])
        _check_proj(Xq, xs, Wp, ws, Y, acc, codes_per_byte, n_scales, T)
        dev = Xq.device if dev is None else dev
        if Xq.device != dev:
            raise ValueError("grouped entries on different devices: %s and %s" % (dev, Xq.device))


def _check_act_entries(entries, T):
    if len(entries) < 1 or len(entries) > MAX_GROUP:
        raise ValueError("a grouped call takes 1..%d entries, got %d" % (MAX_GROUP, len(entries)))
    dev = None
    for X, gain, Xq, xs in entries:
        T0, K = _dims(X, "X", 2)
        if T0 != T:
            raise ValueError("X has %d tokens, the call is for %d" % (T0, T))
        _arg(X, "X", _F32)
        _arg(gain, "gain", _F32, numel=K, optional=True)
        _arg(Xq, "Xq", _I8, shape=(T, K))
        _arg(xs, "x_scale", _F32, min_numel=T)
        _same_gpu(X, gain, Xq, xs)
        dev = X.device if dev is None else dev
        if X.device != dev:
            raise ValueError("grouped entries on different devices: %s and %s" % (dev, X.device))


def _check_weights(W, out, codes_per_byte, scales, scale_name, gamma, workspace):
    N, K = _dims(W, "W", 2)
    _arg(W, "W", _F32)
    if K % codes_per_byte:
        raise ValueError("K = %d is not a multiple of %d" % (K, codes_per_byte))
    _arg(out, "W_packed", _U8, shape=(N, K // codes_per_byte))
    _arg(scales[0], scale_name, _F32, min_numel=scales[1])
    _arg(gamma, "w_gamma", _F64, min_numel=scales[1], optional=True)
    _arg(workspace, "workspace", _U8)
    _same_gpu(W, out, scales[0], gamma, workspace)
    return N, K


# ---------------------------------------------------------------- C ABI mirror

def bitlinear_status_str(status: int) -> str:
    return _c_str(status).decode()


def bitlinear_last_hip_error() -> str:
    return _c_err().decode()


def bitlinear_abi_version() -> int:
    return _c_ver()


def bitlinear_weight_workspace_bytes(N: int, K: int) -> int:
    return int(_c_ws_bytes(N, K))


def bitlinear_quantize_weights(W, W_packed, w_scale, w_gamma, workspace, stream=None):
    N, K = _check_weights(W, W_packed, 4, (w_scale, 1), "w_scale", w_gamma, workspace)
    _check(_c_qw(_ptr(W), N, K, _ptr(W_packed), _ptr(w_scale), _ptr(w_gamma), _ptr(workspace),
                 _nbytes(workspace), _stream(W, stream)), "bitlinear_quantize_weights")


def bitlinear_quantize_acts(X, gain, eps, flags, Xq, x_scale, stream=None):
    T, K = _dims(X, "X", 2)
    _check_act_entries([(X, gain, Xq, x_scale)], T)
    _check(_c_qa(_ptr(X), _ptr(gain), T, K, float(eps), int(flags), _ptr(Xq), _ptr(x_scale),
                 _stream(X, stream)), "bitlinear_quantize_acts")


def bitlinear_quantize_acts_grouped(entries, T, eps, flags, stream=None):
    """entries: list of (X, gain, Xq, x_scale)."""
    _check_act_entries(entries, T)
    arr = (_ActDesc * len(entries))()
    for i, (X, gain, Xq, xs) in enumerate(entries):
        arr[i] = _ActDesc(X.data_ptr(), None if gain is None else gain.data_ptr(), Xq.data_ptr(),
                          xs.data_ptr(), X.shape[-1])
    _check(_c_qag(arr, len(entries), T, float(eps), int(flags), _stream(entries[0][0], stream)),
           "bitlinear_quantize_acts_grouped")


def bitlinear_forward(Xq, x_scale, W_packed, w_scale, Y, acc=None, stream=None):
    T, N, K = _check_proj(Xq, x_scale, W_packed, w_scale, Y, acc)
    _check(_c_fw(_ptr(Xq), _ptr(x_scale), T, K, _ptr(W_packed), _ptr(w_scale), N, _ptr(Y),
                 _ptr(acc), _stream(Xq, stream)), "bitlinear_forward")


def bitlinear_forward_ex(Xq, x_scale, W_packed, w_scale, Y, acc=None, kernel="auto",
                         stream=None):
    T, N, K = _check_proj(Xq, x_scale, W_packed, w_scale, Y, acc)
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(_c_fwx(_ptr(Xq), _ptr(x_scale), T, K, _ptr(W_packed), _ptr(w_scale), N, _ptr(Y),
                  _ptr(acc), k, _stream(Xq, stream)), "bitlinear_forward_ex")


def bitlinear_forward_workspace_bytes(T: int, N: int, K: int) -> int:
    return int(_c_fw_wsb(T, N, K))


def _workspace(nbytes, like):
    """Split-K workspace from torch's allocator (graph-capture safe), or None."""
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device) if nbytes else None


def bitlinear_forward_ws(Xq, x_scale, W_packed, w_scale, Y, acc=None, kernel="auto",
                         workspace=None, stream=None):
    T, N, K = _check_proj(Xq, x_scale, W_packed, w_scale, Y, acc)
    _arg(workspace, "workspace", _U8, optional=True)
    _same_gpu(Xq, workspace)
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    nb = _nbytes(workspace)
    _check(_c_fw_ws(_ptr(Xq), _ptr(x_scale), T, K, _ptr(W_packed), _ptr(w_scale), N, _ptr(Y),
                    _ptr(acc), k, _ptr(workspace), nb, _stream(Xq, stream)),
           "bitlinear_forward_ws")


def bitlinear_forward_choice(T: int, N: int, K: int, workspace: bool = True) -> str:
    """The kernel the product runs: by default as this binding calls it (forward,
    prepare_forward_grouped: with the split-K workspace the shape asks for), with
    workspace=False as the plain C call bitlinear_forward does."""
    if not workspace:
        return _KERNEL_NAMES[_c_choice(T, N, K)]
    return _KERNEL_NAMES[_c_choice_ws(T, N, K, _c_fw_wsb(T, N, K))]


def bitlinear_forward_grouped(entries, T, stream=None):
    """entries: list of (Xq, x_scale, W_packed, w_scale, Y, acc_or_None)."""
    _check_entries(entries, T)
    _check(_c_fwg(_proj_array(entries), len(entries), T, _stream(entries[0][0], stream)),
           "bitlinear_forward_grouped")


def bitlinear_forward_grouped_ws(entries, T, workspace, stream=None):
    """bitlinear_forward_grouped with a split-K workspace (a uint8 tensor or None)."""
    _check_entries(entries, T)
    _arg(workspace, "workspace", _U8, optional=True)
    _same_gpu(entries[0][0], workspace)
    nb = _nbytes(workspace)
    _check(_c_fwg_ws(_proj_array(entries), len(entries), T, _ptr(workspace), nb,
                     _stream(entries[0][0], stream)), "bitlinear_forward_grouped_ws")


def bitlinear_forward_grouped_noalloc(entries, T, stream=None):
    """bitlinear_forward_grouped_ws with the library's static split-K scratch (64 MiB per
    GPU) in place of a workspace: nothing is allocated. Calls that overlap on one GPU
    race on that scratch."""
    _check_entries(entries, T)
    _check(_c_fwg_na(_proj_array(entries), len(entries), T, _stream(entries[0][0], stream)),
           "bitlinear_forward_grouped_noalloc")


NOALLOC_SCRATCH_BYTES = 64 << 20


def bitlinear_quantize_weights_sign(W, W_bits, w_scale, w_alpha, workspace, stream=None):
    N, K = _check_weights(W, W_bits, 8, (w_scale, 1), "w_scale", w_alpha, workspace)
    _check(_c_qws(_ptr(W), N, K, _ptr(W_bits), _ptr(w_scale), _ptr(w_alpha), _ptr(workspace),
                  _nbytes(workspace), _stream(W, stream)), "bitlinear_quantize_weights_sign")


def bitlinear_forward_sign(Xq, x_scale, W_bits, w_scale, Y, acc=None, stream=None):
    T, N, K = _check_proj(Xq, x_scale, W_bits, w_scale, Y, acc, codes_per_byte=8)
    _check(_c_fws(_ptr(Xq), _ptr(x_scale), T, K, _ptr(W_bits), _ptr(w_scale), N, _ptr(Y),
                  _ptr(acc), _stream(Xq, stream)), "bitlinear_forward_sign")


def _proj_array(entries):
    arr = (_ProjDesc * len(entries))()
    for i, (Xq, xs, Wp, ws, Y, acc) in enumerate(entries):
        arr[i] = _ProjDesc(Xq.data_ptr(), xs.data_ptr(), Wp.data_ptr(), ws.data_ptr(),
                           Y.data_ptr(), None if acc is None else acc.data_ptr(),
                           Wp.shape[0], Xq.shape[-1])
    return arr


def bitlinear_forward_sign_grouped(entries, T, stream=None):
    """entries: list of (Xq, x_scale, W_bits, w_scale, Y, acc_or_None)."""
    _check_entries(entries, T, codes_per_byte=8)
    _check(_c_fwsg(_proj_array(entries), len(entries), T, _stream(entries[0][0], stream)),
           "bitlinear_forward_sign_grouped")


def bitlinear_quantize_weights_scale_groups(W, G, W_packed, w_scale, w_gamma, workspace,
                                            stream=None):
    N, K = _check_weights(W, W_packed, 4, (w_scale, int(G)), "w_scale", w_gamma, workspace)
    _check(_c_qwsg(_ptr(W), N, K, int(G), _ptr(W_packed), _ptr(w_scale), _ptr(w_gamma),
                   _ptr(workspace), _nbytes(workspace), _stream(W, stream)),
           "bitlinear_quantize_weights_scale_groups")


def bitlinear_forward_scale_groups(Xq, x_scale, W_packed, w_scale, G, Y, acc=None, kernel="auto",
                                   stream=None):
    T, N, K = _check_proj(Xq, x_scale, W_packed, w_scale, Y, acc, n_scales=int(G))
    k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(_c_fwsg_scale(_ptr(Xq), _ptr(x_scale), T, K, _ptr(W_packed), _ptr(w_scale), N, int(G),
                         _ptr(Y), _ptr(acc), k, _stream(Xq, stream)),
           "bitlinear_forward_scale_groups")


def bitlinear_forward_grouped_scale_groups(entries, groups, T, stream=None):
    """entries as for bitlinear_forward_grouped; groups[i] = scale groups of entry i."""
    if len(groups) != len(entries):
        raise ValueError("one scale-group count per entry: %d for %d" % (len(groups), len(entries)))
    _check_entries(entries, T, groups=groups)
    g = (_I64 * len(groups))(*[int(x) for x in groups])
    _check(_c_fwg_scale(_proj_array(entries), g, len(entries), T, _stream(entries[0][0], stream)),
           "bitlinear_forward_grouped_scale_groups")


def prepare_forward_grouped_scale_groups(entries, groups, T):
    if len(groups) != len(entries):
        raise ValueError("one scale-group count per entry: %d for %d" % (len(groups), len(entries)))
    _check_entries(entries, T, groups=groups)
    g = (_I64 * len(groups))(*[int(x) for x in groups])
    return PreparedCall(_c_fwg_scale, _proj_array(entries), len(entries), T, (),
                        "bitlinear_forward_grouped_scale_groups", _keep(entries), pre=(g,))


def bitlinear_warmup_lambda(step: int, total: int) -> float:
    return float(_c_lam(int(step), int(total)))


def bitlinear_fake_quant_weights(W, w_scale, lam, W_out, stream=None):
    N, K = _dims(W, "W", 2)
    _arg(W, "W", _F32)
    _arg(w_scale, "w_scale", _F32, min_numel=1)
    _arg(W_out, "W_out", (_BF16, _I16), shape=(N, K))
    _same_gpu(W, w_scale, W_out)
    _check(_c_fqw(_ptr(W), N, K, _ptr(w_scale), float(lam), _ptr(W_out), _stream(W, stream)),
           "bitlinear_fake_quant_weights")


def bitlinear_fake_quant_acts(X, gain, eps, flags, lam, Xq, x_scale, X_out, x_rinv, stream=None):
    T, K = _dims(X, "X", 2)
    _arg(X_out, "X_out", (_BF16, _I16), shape=(T, K))
    _arg(x_rinv, "x_rinv", _F64, min_numel=T, optional=True)
    _check_act_entries([(X, gain, Xq, x_scale)], T)
    _same_gpu(X, X_out, x_rinv)
    _check(_c_fqa(_ptr(X), _ptr(gain), T, K, float(eps), int(flags), float(lam), _ptr(Xq),
                  _ptr(x_scale), _ptr(X_out), _ptr(x_rinv), _stream(X, stream)),
           "bitlinear_fake_quant_acts")


def bitlinear_rmsnorm_backward(X, gain, x_rinv, dY, dX, dgain=None, stream=None):
    T, K = _dims(X, "X", 2)
    _arg(X, "X", _F32)
    _arg(gain, "gain", _F32, numel=K, optional=True)
    _arg(x_rinv, "x_rinv", _F64, min_numel=T)
    _arg(dY, "dY", _F32, shape=(T, K))
    _arg(dX, "dX", _F32, shape=(T, K))
    _arg(dgain, "dgain", _F32, numel=K, optional=True)
    _same_gpu(X, gain, x_rinv, dY, dX, dgain)
    _check(_c_rbw(_ptr(X), _ptr(gain), _ptr(x_rinv), _ptr(dY), T, K, _ptr(dX), _ptr(dgain),
                  _stream(X, stream)), "bitlinear_rmsnorm_backward")


def bitlinear_bitdelta_compress(W_fine, W_base, B, model, D, alpha, workspace, stream=None):
    N, M = _dims(W_fine, "W_fine", 2)
    _arg(W_fine, "W_fine", _F32)
    _arg(W_base, "W_base", (_I16, _BF16), shape=(N, M))
    _arg(D, "D", _U8, shape=(N, M))
    _arg(alpha, "alpha", _F32, min_numel=int(B))
    _arg(workspace, "workspace", _U8)
    _same_gpu(W_fine, W_base, D, alpha, workspace)
    _check(_c_bdc(_ptr(W_fine), _ptr(W_base), N, M, int(B), int(model), _ptr(D), _ptr(alpha),
                  _ptr(workspace), _nbytes(workspace), _stream(W_fine, stream)),
           "bitlinear_bitdelta_compress")


def bitlinear_bitdelta_forward(W_base, D, alpha, X, Y, stream=None):
    N, M = _dims(W_base, "W_base", 2)
    B, M2 = _dims(X, "X", 2)
    if M2 != M:
        raise ValueError("X has %d features, W_base %d" % (M2, M))
    _arg(W_base, "W_base", (_I16, _BF16))
    _arg(D, "D", _U8, shape=(N, M))
    _arg(alpha, "alpha", _F32, min_numel=B)
    _arg(X, "X", _F32)
    _arg(Y, "Y", _F32, numel=B * N)
    _same_gpu(W_base, D, alpha, X, Y)
    _check(_c_bdf(_ptr(W_base), _ptr(D), _ptr(alpha), _ptr(X), N, M, int(B), _ptr(Y),
                  _stream(X, stream)), "bitlinear_bitdelta_forward")


ROOF_READ_SINK_BYTES = 65536


def bitlinear_roof_read(bufs, sink, schedule=0, stream=None):
    """Reads every tensor in bufs once (the HBM read roof of those bytes) in block
    schedule 0..3; sink: a uint8 tensor of ROOF_READ_SINK_BYTES on the same GPU."""
    if len(bufs) < 1 or len(bufs) > MAX_GROUP:
        raise ValueError("1..%d buffers, got %d" % (MAX_GROUP, len(bufs)))
    for i, b in enumerate(bufs):
        _arg(b, "bufs[%d]" % i, (b.dtype,))
        if _nbytes(b) % 16:
            raise ValueError("bufs[%d] holds %d bytes, not a multiple of 16" % (i, _nbytes(b)))
    _arg(sink, "sink", _U8, numel=ROOF_READ_SINK_BYTES)
    _same_gpu(*bufs, sink)
    ptrs = (_P * len(bufs))(*[b.data_ptr() for b in bufs])
    sizes = (_I64 * len(bufs))(*[_nbytes(b) for b in bufs])
    _check(_c_roof_read(ptrs, sizes, len(bufs), int(schedule), _ptr(sink), _stream(sink, stream)),
           "bitlinear_roof_read")


def bitlinear_roof_mfma_i8(iters, workgroups, sink, clocks, stream=None):
    """workgroups x 4 waves, each 8 * iters int8 MFMAs of 65536 ops; sink int32
    [workgroups * 256], clocks int64 [workgroups * 4, 4] (shader clock start/end,
    100 MHz clock start/end per wave)."""
    _arg(sink, "sink", _I32, numel=int(workgroups) * 256)
    _arg(clocks, "clocks", torch.int64, numel=int(workgroups) * 16)
    _same_gpu(sink, clocks)
    _check(_c_roof_mfma(int(iters), int(workgroups), _ptr(sink), _ptr(clocks),
                        _stream(sink, stream)), "bitlinear_roof_mfma_i8")


class PreparedCall:
    """A grouped ABI call with its descriptor array marshalled once:
    fn(arr, *pre, count, T, *extra, stream). Calling it launches on the current stream at
    call time (so it can be captured into a graph); keep holds the tensors it points to."""

    def __init__(self, fn, arr, count, T, extra, where, keep, pre=()):
        self._fn, self._arr, self._count, self._T = fn, arr, count, T
        self._extra, self._where, self._keep, self._pre = extra, where, keep, pre

    def __call__(self, stream=None):
        s = _stream(self._keep[0], stream)
        _check(self._fn(self._arr, *self._pre, self._count, self._T, *self._extra, s), self._where)


def _keep(entries):
    return [t for e in entries for t in e if t is not None]


def prepare_quantize_acts_grouped(entries, T, eps=1e-6, flags=0):
    _check_act_entries(entries, T)
    arr = (_ActDesc * len(entries))()
    for i, (X, gain, Xq, xs) in enumerate(entries):
        arr[i] = _ActDesc(X.data_ptr(), None if gain is None else gain.data_ptr(), Xq.data_ptr(),
                          xs.data_ptr(), X.shape[-1])
    return PreparedCall(_c_qag, arr, len(entries), T, (ctypes.c_float(eps), ctypes.c_uint32(flags)),
                        "bitlinear_quantize_acts_grouped", _keep(entries))


def prepare_forward_grouped(entries, T):
    _check_entries(entries, T)
    arr = _proj_array(entries)
    keep = _keep(entries)
    # one split-K workspace for the call (its projections run one after another), owned
    # by the prepared call
    nb = max(_c_fw_wsb(T, Wp.shape[0], Xq.shape[-1]) for (Xq, _, Wp, _, _, _) in entries)
    ws = _workspace(nb, entries[0][0])
    if ws is not None:
        keep.append(ws)
    return PreparedCall(_c_fwg_ws, arr, len(entries), T,
                        (_ptr(ws), ctypes.c_size_t(nb)), "bitlinear_forward_grouped_ws", keep)


def prepare_forward_sign_grouped(entries, T):
    _check_entries(entries, T, codes_per_byte=8)
    return PreparedCall(_c_fwsg, _proj_array(entries), len(entries), T, (),
                        "bitlinear_forward_sign_grouped", _keep(entries))


# ---------------------------------------------------------------- allocating wrappers

def quantize_weights(W: torch.Tensor, with_gamma: bool = False):
    """W fp32 [N, K] on the GPU -> (packed uint8 [N, K/4], beta fp32 [1][, gamma fp64 [1]])."""
    N, K = W.shape
    dev = W.device
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    gamma = torch.empty(1, dtype=torch.float64, device=dev) if with_gamma else None
    ws = torch.empty(bitlinear_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    bitlinear_quantize_weights(W, packed, beta, gamma, ws)
    return (packed, beta, gamma) if with_gamma else (packed, beta)


def quantize_weights_scale_groups(W: torch.Tensor, G: int, with_gamma: bool = False):
    """W fp32 [N, K], G | N -> (packed uint8 [N, K/4], beta fp32 [G][, gamma fp64 [G]])."""
    N, K = W.shape
    dev = W.device
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    beta = torch.empty(G, dtype=torch.float32, device=dev)
    gamma = torch.empty(G, dtype=torch.float64, device=dev) if with_gamma else None
    ws = torch.empty(bitlinear_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    bitlinear_quantize_weights_scale_groups(W, G, packed, beta, gamma, ws)
    return (packed, beta, gamma) if with_gamma else (packed, beta)


def forward_scale_groups(Xq, x_scale, packed, beta, with_acc: bool = False, kernel="auto"):
    """As forward(), with beta fp32 [G] (G | N): row o uses beta[o // (N / G)]."""
    T = Xq.shape[0]
    N = packed.shape[0]
    Y = torch.empty((T, N), dtype=torch.float32, device=Xq.device)
    acc = torch.empty((T, N), dtype=torch.int32, device=Xq.device) if with_acc else None
    bitlinear_forward_scale_groups(Xq, x_scale, packed, beta, beta.numel(), Y, acc, kernel)
    return (Y, acc) if with_acc else Y


def fake_quant_weights(W: torch.Tensor, beta: torch.Tensor, lam: float) -> torch.Tensor:
    """W fp32 [N, K] and its beta [1] -> bf16 [N, K] of W + lam * (beta * q - W)."""
    out = torch.empty(W.shape, dtype=torch.bfloat16, device=W.device)
    bitlinear_fake_quant_weights(W, beta, lam, out)
    return out


def fake_quant_acts(X: torch.Tensor, lam: float, gain=None, eps: float = 1e-6, flags: int = 0):
    """X fp32 [T, K] -> (bf16 [T, K] of y + lam * (Xq / s - y), Xq, x_scale, r fp64 [T])."""
    T, K = X.shape
    Xq = torch.empty((T, K), dtype=torch.int8, device=X.device)
    xs = torch.empty(T, dtype=torch.float32, device=X.device)
    out = torch.empty((T, K), dtype=torch.bfloat16, device=X.device)
    r = torch.empty(T, dtype=torch.float64, device=X.device)
    bitlinear_fake_quant_acts(X, gain, eps, flags, lam, Xq, xs, out, r)
    return out, Xq, xs, r


def rmsnorm_backward(X: torch.Tensor, r: torch.Tensor, dY: torch.Tensor, gain=None):
    """-> (dX fp32 [T, K], dgain fp32 [K] or None)."""
    dX = torch.empty_like(X)
    dg = torch.empty(X.shape[1], dtype=torch.float32, device=X.device) if gain is not None else None
    bitlinear_rmsnorm_backward(X, gain, r, dY, dX, dg)
    return dX, dg


def bitdelta_compress(W_fines, W_base: torch.Tensor):
    """B (<= 8) fine-tuned fp32 [N, M] matrices and the base (bf16 [N, M]) -> (batched sign
    bits uint8 [N, M], alpha fp32 [B])."""
    B = len(W_fines)
    N, M = W_base.shape
    dev = W_base.device
    D = torch.zeros((N, M), dtype=torch.uint8, device=dev)
    alpha = torch.empty(B, dtype=torch.float32, device=dev)
    ws = torch.empty(bitlinear_weight_workspace_bytes(N, M), dtype=torch.uint8, device=dev)
    for i, Wf in enumerate(W_fines):
        bitlinear_bitdelta_compress(Wf, W_base.view(torch.int16), B, i, D, alpha, ws)
    return D, alpha


def bitdelta_forward(W_base: torch.Tensor, D, alpha, X: torch.Tensor) -> torch.Tensor:
    """Y fp32 [B, N] = W_base x_i + alpha_i Sign(delta_i) x_i for X fp32 [B, M]."""
    Y = torch.empty((X.shape[0], W_base.shape[0]), dtype=torch.float32, device=X.device)
    bitlinear_bitdelta_forward(W_base.view(torch.int16), D, alpha, X, Y)
    return Y


def quantize_weights_sign(W: torch.Tensor):
    """W fp32 [N, K] (K % 8 == 0) on the GPU -> (sign bits uint8 [N, K/8], beta fp32 [1],
    alpha fp64 [1])."""
    N, K = W.shape
    dev = W.device
    bits = torch.empty((N, K // 8), dtype=torch.uint8, device=dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    alpha = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(bitlinear_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    bitlinear_quantize_weights_sign(W, bits, beta, alpha, ws)
    return bits, beta, alpha


def forward_sign(Xq, x_scale, bits, beta, with_acc: bool = False):
    """(Xq [T, K], x_scale [T], sign bits [N, K/8], beta [1]) -> Y fp32 [T, N] (and acc)."""
    T = Xq.shape[0]
    N = bits.shape[0]
    Y = torch.empty((T, N), dtype=torch.float32, device=Xq.device)
    acc = torch.empty((T, N), dtype=torch.int32, device=Xq.device) if with_acc else None
    bitlinear_forward_sign(Xq, x_scale, bits, beta, Y, acc)
    return (Y, acc) if with_acc else Y


def quantize_acts(X: torch.Tensor, gain=None, eps: float = 1e-6, flags: int = 0):
    """X fp32 [T, K] -> (Xq int8 [T, K], x_scale fp32 [T])."""
    T, K = X.shape
    Xq = torch.empty((T, K), dtype=torch.int8, device=X.device)
    xs = torch.empty(T, dtype=torch.float32, device=X.device)
    bitlinear_quantize_acts(X, gain, eps, flags, Xq, xs)
    return Xq, xs


def forward(Xq, x_scale, packed, beta, with_acc: bool = False, kernel="auto"):
    """(Xq [T, K], x_scale [T], packed [N, K/4], beta [1]) -> Y fp32 [T, N] (and acc).
    Passes the split-K workspace the shape asks for (from torch's allocator)."""
    T, K = Xq.shape
    N = packed.shape[0]
    Y = torch.empty((T, N), dtype=torch.float32, device=Xq.device)
    acc = torch.empty((T, N), dtype=torch.int32, device=Xq.device) if with_acc else None
    ws = _workspace(bitlinear_forward_workspace_bytes(T, N, K), Xq)
    bitlinear_forward_ws(Xq, x_scale, packed, beta, Y, acc, kernel, ws)
    return (Y, acc) if with_acc else Y


class BitLinear(torch.nn.Module):
    """A drop-in inference replacement of nn.Linear (no bias): weights quantized once
    to packed ternary codes, activations RMSNorm'd and int8-quantized per call."""

    def __init__(self, weight: torch.Tensor, eps: float = 1e-6, gain=None):
        super().__init__()
        packed, beta = quantize_weights(weight.detach().to(torch.float32).contiguous())
        self.register_buffer("packed", packed)
        self.register_buffer("beta", beta)
        self.register_buffer("gain", None if gain is None else gain.to(torch.float32).contiguous())
        self.eps = eps
        self.in_features = weight.shape[1]
        self.out_features = weight.shape[0]

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        shape = x.shape
        x2 = x.reshape(-1, shape[-1]).to(torch.float32).contiguous()
        Xq, xs = quantize_acts(x2, self.gain, self.eps)
        y = forward(Xq, xs, self.packed, self.beta)
        return y.reshape(*shape[:-1], self.out_features)
