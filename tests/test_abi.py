"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, rejects bad arguments before touching a GPU, and its host-only bit
allocator matches the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as o
import post_quantization_syrk_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    import glob
    src = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_five_engine_calls():
    syms = declared_symbols()
    for name in ("kq_accumulate_hessian", "kq_biip_rotate", "kq_quantize_layer", "kq_sensitivity",
                 "kq_allocate_bits"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = kq.load_library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(kq.EXPORTED)
    assert kq.version() >= 100


def _raw():
    return kq.load_library()


def test_hessian_rejects_bad_arguments_on_host():
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    assert lib.kq_accumulate_hessian(buf, 16, 8, 8, None, 8, 0, None) == kq.KQ_EINVAL
    assert lib.kq_accumulate_hessian(None, 16, 8, 8, buf, 8, 0, None) == kq.KQ_EINVAL
    assert lib.kq_accumulate_hessian(buf, 16, 8, 7, buf, 8, 0, None) == kq.KQ_ESHAPE
    assert lib.kq_accumulate_hessian(buf, 16, 8, 12, buf, 8, 0, None) == kq.KQ_ESHAPE
    assert lib.kq_accumulate_hessian(buf, 16, 0, 8, buf, 8, 0, None) == kq.KQ_ESHAPE
    assert lib.kq_accumulate_hessian(buf, 16, 8, 8, buf, 4, 0, None) == kq.KQ_ESHAPE
    assert lib.kq_accumulate_hessian(buf, 16, 8, 8, buf, 8, 2, None) == kq.KQ_EINVAL
    assert lib.kq_accumulate_hessian(ctypes.c_void_p(0x1002), 16, 8, 8, buf, 8, 0, None) == kq.KQ_EINVAL
    assert b"lda" in lib.kq_last_error() or len(lib.kq_last_error()) > 0


def test_sensitivity_rejects_bad_arguments_on_host():
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    out = (ctypes.c_double * 3)()
    assert lib.kq_sensitivity(None, 4, 4, buf, 4, 4, ctypes.cast(out, ctypes.c_void_p), None) == kq.KQ_EINVAL
    assert lib.kq_sensitivity(buf, 4, 4, buf, 4, 4, None, None) == kq.KQ_EINVAL
    assert lib.kq_sensitivity(buf, 4, 3, buf, 4, 4, ctypes.cast(out, ctypes.c_void_p), None) == kq.KQ_ESHAPE
    assert lib.kq_sensitivity_async(None, 4, 4, buf, 4, 4, buf, None) == kq.KQ_EINVAL
    assert lib.kq_sensitivity_async(buf, 4, 4, buf, 4, 4, None, None) == kq.KQ_EINVAL
    assert lib.kq_sensitivity_async(buf, 4, 4, buf, 0, 4, buf, None) == kq.KQ_ESHAPE
    assert lib.kq_sensitivity_async(buf, 4, 4, buf, 4, 3, buf, None) == kq.KQ_ESHAPE


def test_allocator_rejects_bad_arguments():
    with pytest.raises(kq.KQError):
        kq.kq_allocate_bits([1.0, -1.0], [10, 10])
    with pytest.raises(kq.KQError):
        kq.kq_allocate_bits([1.0, 2.0], [10, 0])
    with pytest.raises(kq.KQError):
        kq.kq_allocate_bits([1.0], [10], allowed=(2, 2))
    with pytest.raises(kq.KQError):
        kq.kq_allocate_bits([1.0], [10], target_num=0)
    assert kq.kq_allocate_bits([], []) == []


def test_allocator_worked_examples_match():
    assert kq.kq_allocate_bits([64, 16, 4, 1], [1, 1, 1, 1]) == [4, 2, 2, 2]
    assert kq.kq_allocate_bits([100, 10, 1, 0.1], [1, 1, 1, 1]) == [4, 2, 2, 2]
    assert kq.kq_allocate_bits([1, 1, 1, 1], [1, 1, 1, 1]) == [3, 3, 2, 2]


@pytest.mark.parametrize("seed", range(25))
def test_allocator_bit_exact_against_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    if seed % 3 == 0:
        # decoder-stack shape: 32 layers x 7 sublayers of Llama-2-7B
        numel = [4096 * 4096] * 4 + [11008 * 4096] * 3
        numel = numel * 32
    else:
        numel = list(rng.integers(1, 50, size=int(rng.integers(1, 40))) * 128)
    L = len(numel)
    sens = np.exp(3.0 * rng.standard_normal(L)) * 1e12
    if seed % 5 == 1:
        sens[: L // 2] = sens[0]        # exact ties
    allowed = (2, 3, 4) if seed % 4 else (2, 4, 8)
    tn, td = ((5, 2), (3, 1), (11, 4), (2, 1))[seed % 4]
    got = kq.kq_allocate_bits(sens, numel, allowed, tn, td)
    want = o.allocate_bits(sens, numel, allowed, tn, td)
    assert got == want


def test_deploy_layer_struct_matches_the_header(tmp_path):
    """The binding's kq_deploy_layer has the size and field offsets the C compiler gives the
    header's struct."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in kq.DeployLayer._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kq.h"\nint main(void) {\n'
                    '  printf("%zu", sizeof(kq_deploy_layer));\n'
                    + "".join(f'  printf(" %zu", offsetof(kq_deploy_layer, {f}));\n' for f in fields)
                    + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(kq.DeployLayer)] + [getattr(kq.DeployLayer, f).offset for f in fields]
    assert got == want


def test_deploy_rejects_bad_arguments_on_host():
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    L = kq.DeployLayer(buf, buf, buf, 4, 128, 64, None, None, None, None, 0, 0, buf)
    arr = (kq.DeployLayer * 9)(*([L] * 9))
    assert lib.kq_deploy_linear_group(arr, 0, 256, buf, None) == kq.KQ_ESHAPE
    assert lib.kq_deploy_linear_group(arr, 9, 256, buf, None) == kq.KQ_ESHAPE
    assert lib.kq_deploy_linear_group(arr, 1, 100, buf, None) == kq.KQ_ESHAPE
    assert lib.kq_deploy_linear_group(arr, 1, 256, None, None) == kq.KQ_EINVAL
    bad = (kq.DeployLayer * 2)(L, kq.DeployLayer(buf, buf, buf, 3, 128, 64, None, None, None, None,
                                                  0, 0, buf))
    assert lib.kq_deploy_linear_group(bad, 2, 256, buf, None) == kq.KQ_ENOTIMPL
    assert b"layer 1" in lib.kq_last_error()
    assert lib.kq_deploy_linear(buf, buf, buf, 4, 100, 64, 256, None, None, None, None, 0, 0, buf,
                                buf, None) == kq.KQ_ESHAPE


def test_flipflop_rejects_bad_arguments_on_host():
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    b = ctypes.c_size_t(0)
    assert lib.kq_flipflop_workspace(1000, 256, 384, ctypes.byref(b)) == kq.KQ_OK and b.value > 0
    assert lib.kq_flipflop_workspace(1000, 200, 384, ctypes.byref(b)) == kq.KQ_ESHAPE
    assert lib.kq_flipflop_workspace(0, 256, 384, ctypes.byref(b)) == kq.KQ_ESHAPE
    need = kq.kq_flipflop_workspace(1000, 256, 384)
    args = (buf, 256, buf, 384, 1000, 256, 384)
    assert lib.kq_flipflop(*args, 0, buf, buf, buf, need, None, None) == kq.KQ_ESHAPE
    assert lib.kq_flipflop(*args, 1, buf, buf, buf, need - 1, None, None) == kq.KQ_EWORKSPACE
    assert lib.kq_flipflop(buf, 256, buf, 384, 1000, 256, 384, 1, None, buf, buf, need, None, None) == kq.KQ_EINVAL
    assert lib.kq_flipflop(buf, 260, buf, 384, 1000, 256, 384, 1, buf, buf, buf, need, None, None) == kq.KQ_ESHAPE


def test_automatic_hadamard_block_beyond_8192_is_refused_on_host():
    """Block 0 means the largest power of 2 dividing the size.  For 16384 that is 16384, which
    no kernel here runs: the library says so instead of rotating with a smaller block, and an
    explicit block of 8192 is accepted by the host checks."""
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    f = ctypes.c_float(0.25)
    # in = 16384, automatic input block
    assert lib.kq_biip_rotate(buf, buf, 64, 16384, buf, buf, buf, buf, buf, buf, 0, 0, f,
                              kq.KQ_BIIP_FULL, buf, buf, None) == kq.KQ_ENOTIMPL
    assert b"8192" in lib.kq_last_error()
    # out = 16384 on the output side only
    assert lib.kq_biip_rotate(buf, buf, 16384, 64, buf, buf, buf, buf, buf, buf, 0, 0, f,
                              kq.KQ_BIIP_OUT_ONLY, buf, buf, None) == kq.KQ_ENOTIMPL
    L = kq.DeployLayer(buf, buf, buf, 4, 128, 64, None, None, None, None, 0, 0, buf)
    arr = (kq.DeployLayer * 1)(L)
    assert lib.kq_deploy_linear_group(arr, 1, 16384, buf, None) == kq.KQ_ENOTIMPL
    L2 = kq.DeployLayer(buf, buf, buf, 4, 128, 16384, None, None, None, None, 0, 0, buf)
    arr2 = (kq.DeployLayer * 1)(L2)
    assert lib.kq_deploy_linear_group(arr2, 1, 256, buf, None) == kq.KQ_ENOTIMPL


def test_testing_selector_rejects_bad_arguments():
    lib = _raw()
    assert lib.kq_testing_select(99, 0) == kq.KQ_EINVAL
    assert lib.kq_testing_select(kq.KQ_TESTING_SYRK_KERNEL, -2) == kq.KQ_EINVAL
    with kq.testing_select(kq.KQ_TESTING_ROW_LDS_BYTES, 0):
        pass
    assert lib.kq_testing_select(kq.KQ_TESTING_ROW_LDS_BYTES, -1) == kq.KQ_OK


def test_async_and_noalloc_quantizers_reject_bad_arguments_on_host():
    """The asynchronous quantizer needs a device status word; the allocation-free one refuses a
    layer whose workspace exceeds its fixed array before any device call."""
    lib = _raw()
    buf = ctypes.c_void_p(0x1000)
    p = kq.make_params(2, 128, 128, 0.01)
    need = kq.kq_quantize_layer_workspace(p, 256, 256, False)
    args = (ctypes.byref(p), buf, buf, None, 256, 256, buf, buf, buf, None, None)
    assert lib.kq_quantize_layer_async(*args, None, buf, need, None) == kq.KQ_EINVAL
    assert b"status" in lib.kq_last_error()
    assert lib.kq_quantize_layer_async(*args, buf, buf, need - 1, None) == kq.KQ_EWORKSPACE
    bad = kq.make_params(5, 128, 128, 0.01)
    assert lib.kq_quantize_layer_async(ctypes.byref(bad), *args[1:], buf, buf, need, None) == kq.KQ_EINVAL
    # 4096 x 8192 needs far more than the fixed 64 MiB
    assert lib.kq_quantize_layer_noalloc(ctypes.byref(p), buf, buf, None, 4096, 8192, buf, buf, buf,
                                         None, None, None) == kq.KQ_EWORKSPACE
    assert lib.kq_quantize_layer_noalloc(ctypes.byref(bad), buf, buf, None, 256, 256, buf, buf, buf,
                                         None, None, None) == kq.KQ_EINVAL
