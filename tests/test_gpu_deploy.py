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
         repeat=1):
    import post_quantization_syrk_amd as kq
    dev = "cuda"
    t = lambda a, dt=None: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    packed = t(o.pack_codes(codes, bits).view(np.int32))
    y = torch.empty(codes.shape[0], device=dev)
    ys = []
    for _ in range(repeat):
        kq.kq_deploy_linear(packed, t(scales), t(zeros), bits, group, t(d_in), t(d_out), t(s_in),
                            t(s_out), bin_, bout, t(x), y)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy().copy())
    return ys


def _ref(codes, scales, zeros, group, d_in, d_out, s_in, s_out, bin_, bout, x):
    out_n, in_n = codes.shape
    Q = o.dequant(codes, scales, zeros, group)
    one = lambda a, n: np.ones(n) if a is None else a.astype(np.float64)  # noqa: E731
    return o.deploy_linear(Q, one(d_in, in_n), one(d_out, out_n), one(s_in, in_n), one(s_out, out_n),
                           bin_, bout, x.astype(np.float64))


@pytest.mark.parametrize("out_n,in_n,bits,group,bin_,bout", [
    (64, 256, 4, 128, 256, 64),        # output blocks rotated by the second kernel
    (96, 256, 2, 128, 2, 32),          # radix-2 input stages; a 32-row output block
    (48, 512, 2, 512, 128, 16),        # blocks within one workgroup; per-channel grid
    (40, 96, 4, 96, 32, 8),            # ragged last workgroup
    (4096, 4096, 4, 128, 4096, 4096),  # Llama-2-7B q/k/v/o
    (11008, 4096, 2, 128, 4096, 256),  # gate/up: 43 output blocks of 256
    (4096, 11008, 4, 128, 256, 4096),  # down: 43 input blocks of 256, several chunk batches
    (4096, 11008, 2, 11008, 256, 4096),
    (256, 8192, 4, 128, 8192, 256),    # 8192-entry input blocks (a last radix-2 round)
    (8192, 256, 2, 128, 256, 8192),    # 8192-entry output blocks: one workgroup per block
    (6144, 1024, 2, 128, 1024, 1),     # no output rotation; 384 workgroups
])
def test_deploy_matches_oracle(out_n, in_n, bits, group, bin_, bout):
    torch = torch_cuda()
    announce(f"deploy out={out_n} in={in_n} W{bits} g{group} b=({bin_},{bout})")
    rng = np.random.default_rng(out_n + 3 * in_n + bits)
    codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, out_n, in_n, bits, group)
    ys = _gpu(torch, codes, scales, zeros, bits, group, d_in, d_out, s_in, s_out, bin_, bout, x)
    ref = _ref(codes, scales, zeros, group, d_in, d_out, s_in, s_out, bin_, bout, x)
    assert rel_fro(ys[0], ref) <= 1e-5


def test_deploy_without_processing_and_repeated_calls():
    """No rescale, no signs, no Hadamard: the plain dequantized product; and repeated calls
    (the output rotated in place by the second kernel) give the same result."""
    torch = torch_cuda()
    announce("deploy plain product / repeated calls")
    rng = np.random.default_rng(7)
    codes, scales, zeros, _, _, _, _, x = _layer(rng, 96, 256, 4, 128, rescale=False, signs=False)
    ys = _gpu(torch, codes, scales, zeros, 4, 128, None, None, None, None, 1, 1, x)
    Q = o.dequant(codes, scales, zeros, 128)
    assert rel_fro(ys[0], Q @ x.astype(np.float64)) <= 1e-5
    codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, 512, 1024, 2, 128)
    ys = _gpu(torch, codes, scales, zeros, 2, 128, d_in, d_out, s_in, s_out, 1024, 512, x, repeat=3)
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])
    ref = _ref(codes, scales, zeros, 128, d_in, d_out, s_in, s_out, 1024, 512, x)
    assert rel_fro(ys[0], ref) <= 1e-5


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
    big = 36864 + 2048   # the LDS copy of x~ would exceed 160 KB
    pb = torch.zeros((16, big * 4 // 32), dtype=torch.int32, device="cuda")
    sb, zb = torch.ones((16, big // 128), device="cuda"), torch.zeros((16, big // 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.kq_deploy_linear(pb, sb, zb, 4, 128, None, None, None, None, 1, 1,
                            torch.zeros(big, device="cuda"), torch.zeros(16, device="cuda"))
    assert e.value.status == kq.KQ_ESHAPE


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
    kq.kq_deploy_linear(packed, scales, zeros, bits, group, di, do, s_in, s_out, 0, 0, x, y)
    torch.cuda.synchronize()
    Q = o.dequant(codes.cpu().numpy().astype(np.int64), scales.cpu().numpy(), zeros.cpu().numpy(), group)
    ref = o.deploy_linear(Q, di.cpu().numpy(), do.cpu().numpy(), s_in.cpu().numpy(),
                          s_out.cpu().numpy(), in_n, out_n, x.cpu().numpy().astype(np.float64))
    yv = y.cpu().numpy()
    assert rel_fro(yv, ref) <= 1e-5
    exact = W.astype(np.float64) @ x.cpu().numpy()
    assert rel_fro(yv, exact) < 0.2   # W4 quantization error of a random layer


def test_deploy_in_a_captured_graph():
    """Three layers (two of them with the second, output-rotation kernel) captured in one HIP
    graph: every replay, with eager launches and synchronizations between the replays, gives
    the eager outputs bit for bit."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("deploy in a captured graph")
    rng = np.random.default_rng(21)
    shapes = [(512, 1024, 4, 128), (1024, 512, 2, 128), (384, 256, 4, 256)]
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    calls = []
    for out_n, in_n, bits, group in shapes:
        codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, out_n, in_n, bits, group)
        calls.append((t(o.pack_codes(codes, bits).view(np.int32)), t(scales), t(zeros), bits, group,
                      t(d_in), t(d_out), t(s_in), t(s_out), t(x), torch.empty(out_n, device=dev)))

    def run(stream=None):
        for p, sc, zr, bits, group, di, do, si, so, x, y in calls:
            kq.kq_deploy_linear(p, sc, zr, bits, group, di, do, si, so, 0, 0, x, y, stream=stream)

    run()
    torch.cuda.synchronize()
    eager = [c[-1].clone() for c in calls]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(side)
    for rep in range(4):
        for c in calls:
            c[-1].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for c, ye in zip(calls, eager):
            assert torch.equal(c[-1], ye), f"replay {rep}"
        run()                      # eager work between the replays
        torch.cuda.synchronize()


def test_deploy_long_rows():
    """in = 28672 (Llama-2-70B down_proj): the LDS copy of x~ is over 64 KB.  Reference from
    the oracle's block rotations (the dense P_in would not fit in memory)."""
    torch = torch_cuda()
    announce("deploy long rows 128 x 28672")
    rng = np.random.default_rng(28672)
    out_n, in_n, bits, group, bin_, bout = 128, 28672, 4, 128, 4096, 128
    codes, scales, zeros, d_in, d_out, s_in, s_out, x = _layer(rng, out_n, in_n, bits, group)
    ys = _gpu(torch, codes, scales, zeros, bits, group, d_in, d_out, s_in, s_out, bin_, bout, x)
    Q = o.dequant(codes, scales, zeros, group)
    xt = o.rotate_cols((x.astype(np.float64) / d_in)[:, None], s_in.astype(np.float64), bin_)[:, 0]
    yt = Q @ xt
    # P_out^T yt = S_out Had(yt) / sqrt(b): the block transform of yt with unit signs, then S
    ref = o.rotate_cols(yt[:, None], np.ones(out_n), bout)[:, 0] * s_out / d_out
    assert rel_fro(ys[0], ref) <= 1e-5


def _group_case(torch, rng, in_n, specs):
    """specs: (out, bits, group, had_in, had_out) per layer; returns the binding's layer dicts,
    the oracle's outputs and x."""
    dev = "cuda"
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    x = rng.standard_normal(in_n).astype(np.float32)
    layers, refs = [], []
    for out_n, bits, group, bin_, bout in specs:
        codes, scales, zeros, d_in, d_out, s_in, s_out, _ = _layer(rng, out_n, in_n, bits, group)
        layers.append(dict(packed=t(o.pack_codes(codes, bits).view(np.int32)), scales=t(scales),
                           zeros=t(zeros), bits=bits, group=group, d_in=t(d_in), d_out=t(d_out),
                           sign_in=t(s_in), sign_out=t(s_out), had_in=bin_, had_out=bout,
                           y=torch.full((out_n,), float("nan"), device=dev)))
        refs.append(_ref(codes, scales, zeros, group, d_in, d_out, s_in, s_out, bin_, bout, x))
    return layers, refs, t(x)


@pytest.mark.parametrize("in_n,specs", [
    # mixed widths, groups, blocks: an output rotation kernel for two layers, a local one
    (1024, [(256, 4, 128, 1024, 256), (96, 2, 1024, 256, 16), (512, 2, 128, 0, 512)]),
    # Llama-2-7B q/k/v with mixed widths (inter-layer mixed precision)
    (4096, [(4096, 4, 128, 0, 0), (4096, 2, 128, 0, 0), (4096, 4, 128, 0, 0)]),
    # gate/up
    (4096, [(11008, 4, 128, 0, 0), (11008, 4, 128, 0, 0)]),
    # eight layers of different heights
    (512, [(16 * (k + 1), 4 if k % 2 else 2, 128, 0, 0) for k in range(8)]),
    # more 16-row tiles than the device holds at once: 32 rows per workgroup, a ragged last
    # workgroup of 8 rows, output blocks of 8 rotated in the matvec kernel
    (512, [(8200, 4, 128, 0, 0), (8200, 2, 128, 0, 0)]),
])
def test_deploy_group_matches_oracle_and_single_calls(in_n, specs):
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce(f"deploy group in={in_n} layers={len(specs)}")
    rng = np.random.default_rng(in_n + len(specs))
    layers, refs, x = _group_case(torch, rng, in_n, specs)
    kq.kq_deploy_linear_group(layers, x)
    torch.cuda.synchronize()
    for k, (L, ref) in enumerate(zip(layers, refs)):
        yg = L["y"].cpu().numpy()
        assert rel_fro(yg, ref) <= 1e-5, k
        ys = torch.empty_like(L["y"])
        kq.kq_deploy_linear(L["packed"], L["scales"], L["zeros"], L["bits"], L["group"], L["d_in"],
                            L["d_out"], L["sign_in"], L["sign_out"], L["had_in"], L["had_out"], x, ys)
        torch.cuda.synchronize()
        assert np.allclose(yg, ys.cpu().numpy(), rtol=1e-6, atol=1e-7), k
