"""GPU parity: the deploy-side forward of a quantized layer (kq_deploy_linear) against the
oracle's y = D_out^-1 P_out^T Qhat P_in D_in^-1 x, with Qhat dequantized from codes that the
oracle packs itself.  fp32 accumulation over at most 11008 products: relative L2 error
<= 1e-5."""
import numpy as np
import pytest

import oracle as o
from tests.gpu_util import announce, rel_fro, torch_cuda

pytestmark = pytest.mark.gpu


def _layer(rng, out_n, in_n, bits, group, rescale=True, signs=True):
    codes = rng.integers(0, 2 ** bits, size=(out_n, in_n))
    ng = in_n // group
    scales = (np.exp(0.3 * rng.standard_normal((out_n, ng))) * 0.01).astype(np.float32)
    zeros = rng.integers(0, 2 ** bits, size=(out_n, ng)).astype(np.uint8)
    d_in = np.exp(0.5 * rng.standard_normal(in_n)).astype(np.float32) if rescale else None
    d_out = np.exp(0.5 * rng.standard_normal(out_n)).astype(np.float32) if rescale else None
    s_in = rng.choice([-1, 1], in_n).astype(np.int8) if signs else None
    s_out = rng.choice([-1, 1], out_n).astype(np.int8) if signs else None
    x = rng.standard_normal(in_n).astype(np.float32)
    return codes, scales, zeros, d_in, d_out, s_in, s_out, x


def _gpu(torch, codes, scales, zeros, bits, group, d_in, d_out, s_in, s_out, bin_, bout, x,
         ws=None, repeat=1):
    import post_quantization_syrk_amd as kq
    dev = "cuda"
    t = lambda a, dt=None: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    packed = t(o.pack_codes(codes, bits).view(np.int32))
    if ws is None:
        ws = torch.zeros(kq.kq_deploy_linear_workspace(codes.shape[0], bout), dtype=torch.uint8,
                         device=dev)
    y = torch.empty(codes.shape[0], device=dev)
    ys = []
    for _ in range(repeat):
        kq.kq_deploy_linear(packed, t(scales), t(zeros), bits, group, t(d_in), t(d_out), t(s_in),
                            t(s_out), bin_, bout, t(x), y, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy().copy())
    return ys, ws


def _ref(codes, scales, zeros, group, d_in, d_out, s_in, s_out, bin_, bout, x):
    out_n, in_n = codes.shape
    Q = o.dequant(codes, scales, zeros, group)
    one = lambda a, n: np.ones(n) if a is None else a.astype(np.float64)  # noqa: E731
    return o.deploy_linear(Q, one(d_in, in_n), one(d_out, out_n), one(s_in, in_n), one(s_out, out_n),
                           bin_, bout, x.astype(np.float64))


@pytest.mark.parametrize("out_n,in_n,bits,group,bin_,bout", [
    (64, 256, 4, 128, 256, 64),        # output blocks finished through the row counters
    (48, 512, 2, 512, 128, 16),        # blocks within one workgroup; per-channel grid
    (40, 96, 4, 96, 32, 8),            # ragged last workgroup
    (4096, 4096, 4, 128, 4096, 4096),  # Llama-2-7B q/k/v/o
    (11008, 4096, 2, 128, 4096, 256),  # gate/up: 43 output blocks of 256
    (4096, 11008, 4, 128, 256, 4096),  # down: 43 input blocks of 256, several chunk batches
    (4096, 11008, 2, 11008, 256, 4096),
])
def test_deploy_matches_oracle(out_n, in_n, bits, group, bin_, bout):
    torch = torch_cuda()
    announce(f"deploy out={out_n} in={in_n} W{bits} g{group} b=({bin_},{bout})")
    rng = np.random.default_rng(out_n + 3 * in_n + bits)
    codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, out_n, in_n, bits, group)
    ys, _ = _gpu(torch, codes, scales, zeros, bits, group, d_in, d_out, s_in, s_out, bin_, bout, x)
    ref = _ref(codes, scales, zeros, group, d_in, d_out, s_in, s_out, bin_, bout, x)
    assert rel_fro(ys[0], ref) <= 1e-5


def test_deploy_without_processing_and_repeated_calls():
    """No rescale, no signs, no Hadamard: the plain dequantized product; and the row counters
    are left zero, so a second call on the same workspace gives the same result."""
    torch = torch_cuda()
    announce("deploy plain product / repeated calls")
    rng = np.random.default_rng(7)
    codes, scales, zeros, _, _, _, _, x = _layer(rng, 96, 256, 4, 128, rescale=False, signs=False)
    ys, _ = _gpu(torch, codes, scales, zeros, 4, 128, None, None, None, None, 1, 1, x)
    Q = o.dequant(codes, scales, zeros, 128)
    assert rel_fro(ys[0], Q @ x.astype(np.float64)) <= 1e-5
    codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, 512, 1024, 2, 128)
    ys, ws = _gpu(torch, codes, scales, zeros, 2, 128, d_in, d_out, s_in, s_out, 1024, 512, x,
                  repeat=3)
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])
    assert int(ws.sum().item()) == int(ws[256:].sum().item())   # counters (first 256 bytes) zero


def test_deploy_rejects_unsupported():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    packed = torch.zeros((16, 12), dtype=torch.int32, device="cuda")
    sc = torch.ones((16, 1), device="cuda")
    zr = torch.zeros((16, 1), dtype=torch.uint8, device="cuda")
    x, y = torch.zeros(128, device="cuda"), torch.zeros(16, device="cuda")
    with pytest.raises(kq.KQError):   # 3-bit codes are not supported on the deploy side
        kq.kq_deploy_linear(packed, sc, zr, 3, 128, None, None, None, None, 1, 1, x, y)
    with pytest.raises(kq.KQError):   # an output block of 64 does not divide 16 rows
        kq.kq_deploy_linear(packed, sc, zr, 4, 128, None, None, None, None, 1, 64, x, y)
    p32 = torch.zeros((32, 16), dtype=torch.int32, device="cuda")
    s32, z32 = torch.ones((32, 1), device="cuda"), torch.zeros((32, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:   # an output block over 16 rows needs the workspace
        kq.kq_deploy_linear(p32, s32, z32, 4, 128, None, None, None, None, 1, 0, x,
                            torch.zeros(32, device="cuda"))
    assert e.value.status == kq.KQ_EWORKSPACE


def test_deploy_after_engine_quantization():
    """Engine output end to end: BiIP + GPTQ on a small layer, then the deploy forward of its
    packed codes equals the oracle's forward of the engine's dequantized weights, and is
    close to W x (the quantization error only)."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("deploy after engine quantization")
    rng = np.random.default_rng(11)
    out_n, in_n, bits, group = 128, 512, 4, 128
    W = (rng.standard_normal((out_n, in_n)) * 0.02).astype(np.float32)
    A = rng.standard_normal((4 * in_n, in_n)).astype(np.float32)
    B = rng.standard_normal((4 * out_n, out_n)).astype(np.float32)
    dev = "cuda"
    HX = torch.from_numpy(A.T @ A).to(dev)
    HG = torch.from_numpy(B.T @ B).to(dev)
    s_in = torch.from_numpy(rng.choice([-1, 1], in_n).astype(np.int8)).to(dev)
    s_out = torch.from_numpy(rng.choice([-1, 1], out_n).astype(np.int8)).to(dev)
    Wd = torch.from_numpy(W).to(dev)
    Wt = torch.empty_like(Wd)
    di, do = torch.empty(in_n, device=dev), torch.empty(out_n, device=dev)
    kq.kq_biip_rotate(Wd, Wt, HX, HX, HG, HG, s_in, s_out, di, do, 0.25, kq.KQ_BIIP_FULL, 0, 0)
    p = kq.make_params(bits, group, 128, 0.01)
    ws = torch.empty(kq.kq_quantize_layer_workspace(p, out_n, in_n, False), dtype=torch.uint8, device=dev)
    packed = torch.zeros((out_n, in_n * bits // 32), dtype=torch.int32, device=dev)
    scales = torch.zeros((out_n, in_n // group), device=dev)
    zeros = torch.zeros((out_n, in_n // group), dtype=torch.uint8, device=dev)
    codes = torch.zeros((out_n, in_n), dtype=torch.uint8, device=dev)
    kq.kq_quantize_layer(p, Wt, HX, HG, packed, scales, zeros, ws, codes=codes)
    x = torch.from_numpy(rng.standard_normal(in_n).astype(np.float32)).to(dev)
    y = torch.empty(out_n, device=dev)
    dws = torch.zeros(kq.kq_deploy_linear_workspace(out_n, 0), dtype=torch.uint8, device=dev)
    kq.kq_deploy_linear(packed, scales, zeros, bits, group, di, do, s_in, s_out, 0, 0, x, y, dws)
    torch.cuda.synchronize()
    Q = o.dequant(codes.cpu().numpy().astype(np.int64), scales.cpu().numpy(), zeros.cpu().numpy(), group)
    ref = o.deploy_linear(Q, di.cpu().numpy(), do.cpu().numpy(), s_in.cpu().numpy(),
                          s_out.cpu().numpy(), in_n, out_n, x.cpu().numpy().astype(np.float64))
    yv = y.cpu().numpy()
    assert rel_fro(yv, ref) <= 1e-5
    exact = W.astype(np.float64) @ x.cpu().numpy()
    assert rel_fro(yv, exact) < 0.2   # W4 quantization error of a random layer
