"""GPU parity: two-sided rounding (kq_quantize_two_sided) against the oracle's coordinate-by-
coordinate GPTQ on vec(W) under H_X (x) H_G.

Codes are integers decided in floating point: the GPU divides by fp32 scales in fp32, the
oracle in fp64, so a value within 1e-4 of a rounding midpoint may land on either neighbour;
the oracle adopts the GPU's neighbour there (the tie protocol of its GPTQ) and keeps
following its own arithmetic otherwise.  Bar: no other code differs; scales within fp32
rounding of the oracle's fp64 ones; zero points equal; dequantized weights within 1e-5
relative Frobenius (fp32 feedback over at most a few thousand terms per coordinate)."""
import numpy as np
import pytest

import oracle as o
from tests.gpu_util import announce, rel_fro, torch_cuda

pytestmark = pytest.mark.gpu


def _case(seed, m, n):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    A = rng.standard_normal((3 * n, n)) * np.exp(0.7 * rng.standard_normal(n))
    A[:, 1::3] += 0.5 * A[:, 0::3][:, :A[:, 1::3].shape[1]]
    B = rng.standard_normal((3 * m, m)) * np.exp(0.7 * rng.standard_normal(m))
    B[:, 2::4] -= 0.6 * B[:, 1::4][:, :B[:, 2::4].shape[1]]
    return W, (A.T @ A).astype(np.float32), (B.T @ B).astype(np.float32)


def _gpu(torch, W, HX, HG, bits, group, damp):
    import post_quantization_syrk_amd as kq
    m, n = W.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")  # noqa: E731
    p = kq.make_params(bits, group, 128, damp)
    packed = torch.zeros((m, n * bits // 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((m, n // group), device="cuda")
    zeros = torch.zeros((m, n // group), dtype=torch.uint8, device="cuda")
    codes = torch.zeros((m, n), dtype=torch.uint8, device="cuda")
    kq.kq_quantize_two_sided(p, d(W), d(HX), d(HG), packed, scales, zeros, codes=codes)
    torch.cuda.synchronize()
    return (packed.cpu().numpy().view(np.uint32), scales.cpu().numpy(), zeros.cpu().numpy(),
            codes.cpu().numpy().astype(np.int64))


def _check(gpu, ref, bits):
    packed, scales, zeros, codes = gpu
    assert ref.hard_mismatches == 0, ref.hard_mismatches
    assert np.array_equal(codes, ref.codes)
    assert np.allclose(scales, ref.scales, rtol=2 ** -23, atol=0)
    assert np.array_equal(zeros, ref.zeros.astype(np.uint8))
    assert np.array_equal(packed, o.pack_codes(codes, bits))
    g = np.arange(codes.shape[1]) // (codes.shape[1] // scales.shape[1])
    qhat = scales[:, g].astype(np.float64) * (codes - zeros[:, g].astype(np.float64))
    assert rel_fro(qhat, ref.qhat) <= 1e-5


@pytest.mark.parametrize("m,n,bits,group,damp", [
    (128, 128, 3, 64, 0.01),    # 4 x 4 tiles, 3-bit codes across word boundaries
    (256, 128, 2, 128, 0.02),   # more rows than columns
    (128, 256, 4, 32, 0.01),    # more columns; a group per tile
    (384, 384, 3, 64, 0.01),    # pulls over two slices, far pushes over two chunks
])
def test_two_sided_matches_oracle(m, n, bits, group, damp):
    torch = torch_cuda()
    announce(f"two-sided m={m} n={n} W{bits} g{group}")
    W, HX, HG = _case(m + 7 * n + bits, m, n)
    gpu = _gpu(torch, W, HX, HG, bits, group, damp)
    ref = o.two_sided_gptq(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64), bits,
                           group, damp, replay_codes=gpu[3])
    print(f"  ties adopted {ref.accepted_ties}, hard mismatches {ref.hard_mismatches}")
    _check(gpu, ref, bits)


def test_two_sided_dead_channels():
    """A zero diagonal in either factor: its column (input) or row (output) of W is zeroed
    and takes no feedback."""
    torch = torch_cuda()
    announce("two-sided dead channels")
    W, HX, HG = _case(71, 128, 128)
    HX[5, :] = HX[:, 5] = 0.0
    HG[9, :] = HG[:, 9] = 0.0
    gpu = _gpu(torch, W, HX, HG, 4, 128, 0.01)
    ref = o.two_sided_gptq(W.astype(np.float64), HX.astype(np.float64), HG.astype(np.float64), 4, 128,
                           0.01, replay_codes=gpu[3])
    _check(gpu, ref, 4)


@pytest.mark.slow
def test_two_sided_full_size_leading_block():
    """Llama-2-7B q_proj size (4096 x 4096): the leading 128 x 128 block depends on nothing
    outside it, so the oracle checks it exactly with the leading blocks of the full factors."""
    torch = torch_cuda()
    announce("two-sided full size 4096 x 4096, leading block")
    m = n = 4096
    W, HX, HG = _case(72, m, n)
    gpu = _gpu(torch, W, HX, HG, 4, 128, 0.01)
    UX = o.damp_and_factor(HX.astype(np.float64), 0.01)[0]
    UG = o.damp_and_factor(HG.astype(np.float64), 0.01)[0]
    b = 128
    sc, zc = o.static_grid(W[:b, :b].astype(np.float64), 4, 128)
    ref = o.two_sided_rounding(W[:b, :b].astype(np.float64), UX[:b, :b], UG[:b, :b], sc, zc, 4, 128,
                               replay_codes=gpu[3][:b, :b])
    print(f"  ties adopted {ref.accepted_ties}, hard mismatches {ref.hard_mismatches}")
    assert ref.hard_mismatches == 0
    assert np.array_equal(gpu[3][:b, :b], ref.codes)
    assert np.allclose(gpu[1][:b, :1], ref.scales, rtol=2 ** -23, atol=0)
