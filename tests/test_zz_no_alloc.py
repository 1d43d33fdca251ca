"""kq_quantize_layer_noalloc, the quantizer entry point that allocates nothing: its workspace
is the library's fixed per-GPU array.  Two calls in a row (the second on a smaller layer, so
the array still holds the first call's contents) must give what kq_quantize_layer gives with
a workspace of the caller's, through the C ABI."""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import announce, torch_cuda

pytestmark = pytest.mark.gpu


def _spd(rng, n):
    sc = np.exp(rng.standard_normal(n))
    A = rng.standard_normal((2 * n, n)) * sc
    return (A.T @ A).astype(np.float32)


def _run(torch, kq, lib, p, W, HX, HG, use_ws):
    out_n, in_n = W.shape
    dev = "cuda"
    Wd = torch.from_numpy(W).to(dev)
    HXd = torch.from_numpy(HX).to(dev)
    HGd = None if HG is None else torch.from_numpy(HG).to(dev)
    packed = torch.full((out_n, in_n * p.bits // 32), -1, dtype=torch.int32, device=dev)
    scales = torch.full((out_n, in_n // p.group), -1.0, device=dev)
    zeros = torch.full((out_n, in_n // p.group), 255, dtype=torch.uint8, device=dev)
    codes = torch.full((out_n, in_n), 255, dtype=torch.uint8, device=dev)
    loss = (ctypes.c_double * 2)()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hg = None if HGd is None else ctypes.c_void_p(HGd.data_ptr())
    args = (ctypes.byref(p), ctypes.c_void_p(Wd.data_ptr()), ctypes.c_void_p(HXd.data_ptr()), hg,
            out_n, in_n, ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
            ctypes.c_void_p(zeros.data_ptr()), ctypes.c_void_p(codes.data_ptr()),
            ctypes.cast(loss, ctypes.c_void_p))
    if use_ws:
        need = kq.kq_quantize_layer_workspace(p, out_n, in_n, True)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        st = lib.kq_quantize_layer(*args, ctypes.c_void_p(ws.data_ptr()), need, stream)
    else:
        st = lib.kq_quantize_layer_noalloc(*args, stream)
    assert st == kq.KQ_OK, lib.kq_last_error()
    torch.cuda.synchronize()
    return dict(E=Wd.cpu().numpy(), packed=packed.cpu().numpy(), scales=scales.cpu().numpy(),
                zeros=zeros.cpu().numpy(), codes=codes.cpu().numpy(), loss=(loss[0], loss[1]))


def test_noalloc_matches_workspace_call_twice():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    lib = kq.load_library()
    rng = np.random.default_rng(123)
    cases = [(384, 512, 3, 128, 128, True),    # larger first: 384 x 512, W3, with H_G
             (96, 256, 2, 64, 64, False)]       # then smaller, W2, H_G = identity
    for out_n, in_n, bits, group, block, with_hg in cases:
        announce(f"noalloc: {out_n} x {in_n} W{bits} g{group} B{block} H_G={'yes' if with_hg else 'I'}")
        p = kq.make_params(bits, group, block, 0.01)
        W = (rng.standard_normal((out_n, in_n)) * 0.02).astype(np.float32)
        HX = _spd(rng, in_n)
        HG = _spd(rng, out_n) if with_hg else None
        ref = _run(torch, kq, lib, p, W, HX, HG, use_ws=True)
        got = _run(torch, kq, lib, p, W, HX, HG, use_ws=False)
        for k in ("packed", "scales", "zeros", "codes", "E"):
            assert np.array_equal(got[k], ref[k]), k
        for a, b in zip(got["loss"], ref["loss"]):
            assert a == pytest.approx(b, rel=1e-9)


def test_noalloc_refuses_a_layer_beyond_its_array():
    torch_cuda()
    import post_quantization_syrk_amd as kq
    lib = kq.load_library()
    p = kq.make_params(2, 128, 128, 0.01)
    buf = ctypes.c_void_p(0x1000)
    # 8192 x 8192: the factor alone is 256 MiB, beyond the fixed array
    st = lib.kq_quantize_layer_noalloc(ctypes.byref(p), buf, buf, None, 8192, 8192, buf, buf, buf,
                                       None, None, None)
    assert st == kq.KQ_EWORKSPACE
    assert b"workspace" in lib.kq_last_error()
