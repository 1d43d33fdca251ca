"""Python binding of libkq, the KronQ per-layer quantization engine for MI355X.

Thin ctypes marshalling over the C ABI declared in include/kq.h: each
function takes PyTorch tensors (device memory) or numpy arrays (host memory),
checks dtypes, devices and sizes, and passes raw pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels; this
module computes nothing itself and has no fallback: if libkq.so is missing or
fails to load, importing the engine raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkq.so")

KQ_OK, KQ_EINVAL, KQ_ESHAPE, KQ_ENOTSPD, KQ_EWORKSPACE, KQ_ENOTIMPL, KQ_EHIP = range(7)
KQ_BIIP_FULL, KQ_BIIP_NO_RESCALE, KQ_BIIP_IN_ONLY, KQ_BIIP_OUT_ONLY = range(4)
STATUS_NAMES = {0: "KQ_OK", 1: "KQ_EINVAL", 2: "KQ_ESHAPE", 3: "KQ_ENOTSPD", 4: "KQ_EWORKSPACE",
                5: "KQ_ENOTIMPL", 6: "KQ_EHIP"}

EXPORTED = ("kq_version", "kq_last_error", "kq_accumulate_hessian", "kq_sensitivity",
            "kq_sensitivity_async",
            "kq_biip_rotate", "kq_quantize_layer_workspace", "kq_quantize_layer",
            "kq_quantize_layer_noalloc", "kq_quantize_layer_async",
            "kq_allocate_bits", "kq_deploy_linear", "kq_deploy_linear_group",
            "kq_flipflop_workspace", "kq_flipflop", "kq_quantize_two_sided_workspace",
            "kq_quantize_two_sided", "kq_testing_select")


class KQError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class NotSPDError(KQError):
    pass


class DeployLayer(ctypes.Structure):
    """kq_deploy_layer (include/kq.h)."""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("bits", ctypes.c_int), ("group", ctypes.c_int), ("out", ctypes.c_int64),
                ("d_in", ctypes.c_void_p), ("d_out", ctypes.c_void_p), ("sign_in", ctypes.c_void_p),
                ("sign_out", ctypes.c_void_p), ("had_in", ctypes.c_int64), ("had_out", ctypes.c_int64),
                ("y", ctypes.c_void_p)]


class QuantParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int), ("group", ctypes.c_int), ("block", ctypes.c_int),
                ("damp", ctypes.c_float), ("asym", ctypes.c_int), ("act_order", ctypes.c_int),
                ("w_clip", ctypes.c_int)]


_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "kq_version": ([], ctypes.c_int),
    "kq_last_error": ([], ctypes.c_char_p),
    "kq_accumulate_hessian": ([_vp, _i64, _i64, _i64, _vp, _i64, _int, _vp], _int),
    "kq_sensitivity": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp], _int),
    "kq_sensitivity_async": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp], _int),
    "kq_biip_rotate": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int,
                        _vp, _vp, _vp], _int),
    "kq_quantize_layer_workspace": ([ctypes.POINTER(QuantParams), _i64, _i64, _int,
                                     ctypes.POINTER(_sz)], _int),
    "kq_quantize_layer": ([ctypes.POINTER(QuantParams), _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                           _vp, _vp, _sz, _vp], _int),
    "kq_quantize_layer_async": ([ctypes.POINTER(QuantParams), _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "kq_quantize_layer_noalloc": ([ctypes.POINTER(QuantParams), _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                                   _vp, _vp, _vp, _vp], _int),
    "kq_allocate_bits": ([_vp, _vp, _i64, _vp, _int, _i64, _i64, _vp], _int),
    "kq_deploy_linear": ([_vp, _vp, _vp, _int, _int, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                          _vp, _vp, _vp], _int),
    "kq_deploy_linear_group": ([ctypes.POINTER(DeployLayer), _int, _i64, _vp, _vp], _int),
    "kq_flipflop_workspace": ([_i64, _i64, _i64, ctypes.POINTER(_sz)], _int),
    "kq_quantize_two_sided_workspace": ([ctypes.POINTER(QuantParams), _i64, _i64, ctypes.POINTER(_sz)], _int),
    "kq_quantize_two_sided": ([ctypes.POINTER(QuantParams), _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                               _sz, _vp, _vp], _int),
    "kq_flipflop": ([_vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _sz,
                     ctypes.POINTER(ctypes.c_double), _vp], _int),
    "kq_testing_select": ([_int, _i64], _int),
}

# include/kq_testing.h: implementation selection for tests
KQ_TESTING_SYRK_KERNEL, KQ_TESTING_FACTOR_SUPERBLOCK, KQ_TESTING_ROW_LDS_BYTES = range(3)

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkq.so (raises OSError/ImportError if it is missing)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


class testing_select:
    """Context manager over kq_testing_select: forces one implementation path for the calls
    made inside the block, then restores the default."""

    def __init__(self, knob: int, value: int):
        self.knob, self.value = knob, value

    def __enter__(self):
        _check(load_library().kq_testing_select(self.knob, self.value), "kq_testing_select")
        return self

    def __exit__(self, *exc):
        _check(load_library().kq_testing_select(self.knob, -1), "kq_testing_select")
        return False


def _check(status: int, fn: str) -> None:
    if status != KQ_OK:
        msg = _lib.kq_last_error().decode(errors="replace")
        if status == KQ_ENOTSPD:
            raise NotSPDError(status, fn, msg)
        raise KQError(status, fn, msg)


def _torch():
    import torch
    return torch


def _dev_ptr(t, name: str, dtypes=None, allow_none: bool = False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda/hip) tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def version() -> int:
    return load_library().kq_version()


def kq_accumulate_hessian(A, H, accumulate: bool = False, stream=None) -> None:
    """H = A^T A (or H += A^T A): A bf16 [T x n] (token-major), H fp32 [n x n]."""
    torch = _torch()
    lib = load_library()
    T, n = A.shape
    if H.shape != (n, n):
        raise ValueError("H must be n x n")
    st = lib.kq_accumulate_hessian(_dev_ptr(A, "A", (torch.bfloat16, torch.int16, torch.uint16)),
                                   T, n, _ld(A, "A"), _dev_ptr(H, "H", (torch.float32,)), _ld(H, "H"),
                                   1 if accumulate else 0, _stream(stream))
    _check(st, "kq_accumulate_hessian")


def kq_sensitivity(HX, HG, stream=None) -> tuple[float, float, float]:
    """(tr H_X, tr H_G, tr H_G * tr H_X); synchronizes the stream."""
    torch = _torch()
    lib = load_library()
    out = (ctypes.c_double * 3)()
    st = lib.kq_sensitivity(_dev_ptr(HX, "HX", (torch.float32,)), HX.shape[0], _ld(HX, "HX"),
                            _dev_ptr(HG, "HG", (torch.float32,)), HG.shape[0], _ld(HG, "HG"),
                            ctypes.cast(out, ctypes.c_void_p), _stream(stream))
    _check(st, "kq_sensitivity")
    return out[0], out[1], out[2]


def kq_sensitivity_async(HX, HG, out, stream=None) -> None:
    """Traces and sensitivity into `out` (device float64, 3 entries); does not synchronize."""
    torch = _torch()
    lib = load_library()
    if out.numel() < 3:
        raise ValueError("kq_sensitivity_async: out needs 3 entries")
    st = lib.kq_sensitivity_async(_dev_ptr(HX, "HX", (torch.float32,)), HX.shape[0], _ld(HX, "HX"),
                                  _dev_ptr(HG, "HG", (torch.float32,)), HG.shape[0], _ld(HG, "HG"),
                                  _dev_ptr(out, "out", (torch.float64,)), _stream(stream))
    _check(st, "kq_sensitivity_async")


def kq_biip_rotate(W_src, W_dst, HX_src, HX_dst, HG_src, HG_dst, sign_in, sign_out, d_in, d_out,
                   alpha: float = 0.25, mode: int = KQ_BIIP_FULL, had_block_in: int = 0,
                   had_block_out: int = 0, stream=None) -> None:
    """Bidirectional incoherence processing (rescale + randomized Hadamard, both sides)."""
    torch = _torch()
    lib = load_library()
    out_n, in_n = W_src.shape
    f32 = (torch.float32,)
    i8 = (torch.int8,)
    st = lib.kq_biip_rotate(
        _dev_ptr(W_src, "W_src", f32), _dev_ptr(W_dst, "W_dst", f32), out_n, in_n,
        _dev_ptr(HX_src, "HX_src", f32), _dev_ptr(HX_dst, "HX_dst", f32),
        _dev_ptr(HG_src, "HG_src", f32, True), _dev_ptr(HG_dst, "HG_dst", f32, True),
        _dev_ptr(sign_in, "sign_in", i8, True), _dev_ptr(sign_out, "sign_out", i8, True),
        had_block_in, had_block_out, alpha, mode, _dev_ptr(d_in, "d_in", f32),
        _dev_ptr(d_out, "d_out", f32), _stream(stream))
    _check(st, "kq_biip_rotate")


def make_params(bits: int = 2, group: int = 128, block: int = 128, damp: float = 0.01,
                asym: int = 1, act_order: int = 0, w_clip: int = 0) -> QuantParams:
    return QuantParams(bits, group, block, damp, asym, act_order, w_clip)


def kq_quantize_layer_workspace(p: QuantParams, out_n: int, in_n: int, with_loss: bool) -> int:
    lib = load_library()
    sz = ctypes.c_size_t(0)
    st = lib.kq_quantize_layer_workspace(ctypes.byref(p), out_n, in_n, 1 if with_loss else 0,
                                         ctypes.byref(sz))
    _check(st, "kq_quantize_layer_workspace")
    return sz.value


def kq_quantize_layer(p: QuantParams, W_rot, HX_rot, HG_rot, packed, scales, zeros, ws,
                      codes=None, want_loss: bool = False, stream=None):
    """GPTQ to packed codes; returns (loss_direct, loss_pred) if want_loss else None."""
    torch = _torch()
    lib = load_library()
    out_n, in_n = W_rot.shape
    loss = (ctypes.c_double * 2)() if want_loss else None
    st = lib.kq_quantize_layer(
        ctypes.byref(p), _dev_ptr(W_rot, "W_rot", (torch.float32,)),
        _dev_ptr(HX_rot, "HX_rot", (torch.float32,)),
        _dev_ptr(HG_rot, "HG_rot", (torch.float32,), True), out_n, in_n,
        _dev_ptr(packed, "packed", (torch.int32, torch.uint32)),
        _dev_ptr(scales, "scales", (torch.float32,)), _dev_ptr(zeros, "zeros", (torch.uint8,)),
        _dev_ptr(codes, "codes", (torch.uint8,), True),
        ctypes.cast(loss, ctypes.c_void_p) if loss is not None else None,
        _dev_ptr(ws, "ws", (torch.uint8,)), ws.numel(), _stream(stream))
    _check(st, "kq_quantize_layer")
    return (loss[0], loss[1]) if want_loss else None


def kq_quantize_layer_async(p: QuantParams, W_rot, HX_rot, HG_rot, packed, scales, zeros, ws,
                            status, codes=None, loss=None, stream=None) -> None:
    """kq_quantize_layer without waiting: `status` (device int32, 1 entry) receives KQ_OK or
    KQ_ENOTSPD and `loss` (device float64, 2 entries, optional) the two losses, when the work
    has run."""
    torch = _torch()
    lib = load_library()
    out_n, in_n = W_rot.shape
    st = lib.kq_quantize_layer_async(
        ctypes.byref(p), _dev_ptr(W_rot, "W_rot", (torch.float32,)),
        _dev_ptr(HX_rot, "HX_rot", (torch.float32,)),
        _dev_ptr(HG_rot, "HG_rot", (torch.float32,), True), out_n, in_n,
        _dev_ptr(packed, "packed", (torch.int32, torch.uint32)),
        _dev_ptr(scales, "scales", (torch.float32,)), _dev_ptr(zeros, "zeros", (torch.uint8,)),
        _dev_ptr(codes, "codes", (torch.uint8,), True), _dev_ptr(loss, "loss", (torch.float64,), True),
        _dev_ptr(status, "status", (torch.int32,)), _dev_ptr(ws, "ws", (torch.uint8,)), ws.numel(),
        _stream(stream))
    _check(st, "kq_quantize_layer_async")


KQ_NOALLOC_WORKSPACE_BYTES = 64 << 20


def kq_quantize_layer_noalloc(p: QuantParams, W_rot, HX_rot, HG_rot, packed, scales, zeros,
                              codes=None, want_loss: bool = False, stream=None):
    """kq_quantize_layer on the library's fixed per-GPU workspace (no allocation); returns
    (loss_direct, loss_pred) if want_loss else None."""
    torch = _torch()
    lib = load_library()
    out_n, in_n = W_rot.shape
    loss = (ctypes.c_double * 2)() if want_loss else None
    st = lib.kq_quantize_layer_noalloc(
        ctypes.byref(p), _dev_ptr(W_rot, "W_rot", (torch.float32,)),
        _dev_ptr(HX_rot, "HX_rot", (torch.float32,)),
        _dev_ptr(HG_rot, "HG_rot", (torch.float32,), True), out_n, in_n,
        _dev_ptr(packed, "packed", (torch.int32, torch.uint32)),
        _dev_ptr(scales, "scales", (torch.float32,)), _dev_ptr(zeros, "zeros", (torch.uint8,)),
        _dev_ptr(codes, "codes", (torch.uint8,), True),
        ctypes.cast(loss, ctypes.c_void_p) if loss is not None else None, _stream(stream))
    _check(st, "kq_quantize_layer_noalloc")
    return (loss[0], loss[1]) if want_loss else None


def kq_allocate_bits(sens, numel, allowed=(2, 3, 4), target_num: int = 5, target_den: int = 2):
    """Per-sublayer bit widths (host computation inside the library)."""
    lib = load_library()
    s = np.ascontiguousarray(sens, dtype=np.float64)
    n = np.ascontiguousarray(numel, dtype=np.int64)
    a = np.ascontiguousarray(allowed, dtype=np.int32)
    if s.shape != n.shape or s.ndim != 1:
        raise ValueError("sens and numel must be 1-D of equal length")
    out = np.zeros(s.shape[0], dtype=np.int32)
    st = lib.kq_allocate_bits(s.ctypes.data_as(ctypes.c_void_p), n.ctypes.data_as(ctypes.c_void_p),
                              s.shape[0], a.ctypes.data_as(ctypes.c_void_p), a.shape[0], target_num,
                              target_den, out.ctypes.data_as(ctypes.c_void_p))
    _check(st, "kq_allocate_bits")
    return out.tolist()


def kq_deploy_linear(packed, scales, zeros, bits: int, group: int, d_in, d_out, sign_in, sign_out,
                     had_in: int, had_out: int, x, y, stream=None) -> None:
    """y = D_out^-1 P_out^T Qhat P_in D_in^-1 x for one quantized layer (batch 1)."""
    torch = _torch()
    lib = load_library()
    out_n = packed.shape[0]
    in_n = x.shape[-1]
    st = lib.kq_deploy_linear(
        _dev_ptr(packed, "packed", (torch.int32, torch.uint32)),
        _dev_ptr(scales, "scales", (torch.float32,)), _dev_ptr(zeros, "zeros", (torch.uint8,)),
        bits, group, out_n, in_n,
        _dev_ptr(d_in, "d_in", (torch.float32,), True), _dev_ptr(d_out, "d_out", (torch.float32,), True),
        _dev_ptr(sign_in, "sign_in", (torch.int8,), True),
        _dev_ptr(sign_out, "sign_out", (torch.int8,), True), had_in, had_out,
        _dev_ptr(x, "x", (torch.float32,)), _dev_ptr(y, "y", (torch.float32,)), _stream(stream))
    _check(st, "kq_deploy_linear")


def kq_deploy_linear_group(layers, x, stream=None) -> None:
    """kq_deploy_linear for several layers reading the same x, in one launch.

    layers: sequence of dicts with the keyword arguments of kq_deploy_linear other than x
    (packed, scales, zeros, bits, group, d_in, d_out, sign_in, sign_out, had_in, had_out, y)."""
    torch = _torch()
    lib = load_library()
    arr = (DeployLayer * max(1, len(layers)))()
    for i, L in enumerate(layers):
        arr[i] = DeployLayer(
            _dev_ptr(L["packed"], "packed", (torch.int32, torch.uint32)),
            _dev_ptr(L["scales"], "scales", (torch.float32,)),
            _dev_ptr(L["zeros"], "zeros", (torch.uint8,)), L["bits"], L["group"], L["packed"].shape[0],
            _dev_ptr(L.get("d_in"), "d_in", (torch.float32,), True),
            _dev_ptr(L.get("d_out"), "d_out", (torch.float32,), True),
            _dev_ptr(L.get("sign_in"), "sign_in", (torch.int8,), True),
            _dev_ptr(L.get("sign_out"), "sign_out", (torch.int8,), True),
            L.get("had_in", 0), L.get("had_out", 0), _dev_ptr(L["y"], "y", (torch.float32,)))
    st = lib.kq_deploy_linear_group(arr, len(layers), x.shape[-1], _dev_ptr(x, "x", (torch.float32,)),
                                    _stream(stream))
    _check(st, "kq_deploy_linear_group")


def kq_flipflop_workspace(T: int, n: int, m: int) -> int:
    lib = load_library()
    b = ctypes.c_size_t(0)
    _check(lib.kq_flipflop_workspace(T, n, m, ctypes.byref(b)), "kq_flipflop_workspace")
    return b.value


def kq_flipflop(X, G, iters: int, A, B, ws=None, stream=None, phases: bool = False):
    """FlipFlop factors A (n x n) and B (m x m) from bf16 streams X (T x n) and G (T x m),
    given as int16/uint16/bfloat16 tensors of bit patterns, after `iters` iterations.
    With phases=True, returns the summed HIP-event milliseconds of {factor, quadratic
    forms, scaling, syrk}."""
    torch = _torch()
    lib = load_library()
    T, n = X.shape
    m = G.shape[1]
    if G.shape[0] != T:
        raise ValueError("X and G need the same token count")
    if ws is None:
        ws = torch.empty(kq_flipflop_workspace(T, n, m), dtype=torch.uint8, device=X.device)
    bf = (torch.int16, torch.uint16, torch.bfloat16)
    ph = (ctypes.c_double * 4)() if phases else None
    st = lib.kq_flipflop(_dev_ptr(X, "X", bf), _ld(X, "X"), _dev_ptr(G, "G", bf), _ld(G, "G"), T, n, m,
                         iters, _dev_ptr(A, "A", (torch.float32,)), _dev_ptr(B, "B", (torch.float32,)),
                         _dev_ptr(ws, "ws", (torch.uint8,)), ws.numel(), ph, _stream(stream))
    _check(st, "kq_flipflop")
    if phases:
        return dict(zip(("factor", "quadratic_forms", "scale", "syrk"), list(ph)))
    return None


def kq_quantize_two_sided_workspace(p: QuantParams, out_n: int, in_n: int) -> int:
    lib = load_library()
    b = ctypes.c_size_t(0)
    _check(lib.kq_quantize_two_sided_workspace(ctypes.byref(p), out_n, in_n, ctypes.byref(b)),
           "kq_quantize_two_sided_workspace")
    return b.value


def kq_quantize_two_sided(p: QuantParams, W, HX, HG, packed, scales, zeros, ws=None, codes=None,
                          stream=None) -> None:
    """Two-sided rounding of W (out x in) under H_X (x) H_G into packed codes, scales and
    zero points (the layout of kq_quantize_layer)."""
    torch = _torch()
    lib = load_library()
    out_n, in_n = W.shape
    if ws is None:
        ws = torch.empty(kq_quantize_two_sided_workspace(p, out_n, in_n), dtype=torch.uint8,
                         device=W.device)
    f32 = (torch.float32,)
    st = lib.kq_quantize_two_sided(
        ctypes.byref(p), _dev_ptr(W, "W", f32), _dev_ptr(HX, "HX", f32), _dev_ptr(HG, "HG", f32),
        out_n, in_n, _dev_ptr(packed, "packed", (torch.int32, torch.uint32)),
        _dev_ptr(scales, "scales", f32), _dev_ptr(zeros, "zeros", (torch.uint8,)),
        _dev_ptr(ws, "ws", (torch.uint8,)), ws.numel(), _dev_ptr(codes, "codes", (torch.uint8,), True),
        _stream(stream))
    _check(st, "kq_quantize_two_sided")
