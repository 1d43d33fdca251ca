"""GPU parity: the FlipFlop Hessian factors (kq_flipflop) against the oracle's fp64 iteration
on the same bf16 streams.

Tolerance: the Hessian factors' 1e-3 relative Frobenius error, on every A_k and B_k (k <= 3).
The GPU carries the inverse factor U (B^-1 = U^T U) into the per-token quadratic forms as
two bf16 terms (about 16 significant bits, relative error within 2^-17 per entry), and forms
each factor one-sided, sum_t a_t x_t^T with the weighted row a_t = w_t c x_t as two bf16
terms against the exact bf16 stream x_t; the products accumulate in fp32 and the
factorizations run in fp32.  With the weighted rows rounded to one bf16 term the error was
2.4e-3 at the first iteration (where U is the identity): a few heavy tokens dominate the
weighted sums, so their 2^-9 roundings do not average out."""
import numpy as np
import pytest

import oracle as o
import synthetic as syn
from tests.gpu_util import announce, rel_fro, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _gpu(torch, Xb, Gb, iters):
    import post_quantization_syrk_amd as kq
    T, n = Xb.shape
    m = Gb.shape[1]
    A = torch.empty((n, n), device="cuda")
    B = torch.empty((m, m), device="cuda")
    kq.kq_flipflop(to_dev_bf16(Xb), to_dev_bf16(Gb), iters, A, B)
    return A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,n,m", [(1000, 256, 384), (3000, 384, 128), (480, 256, 128)])
def test_flipflop_matches_oracle(T, n, m):
    torch = torch_cuda()
    announce(f"flipflop T={T} n={n} m={m}")
    cfg = syn.C1.scaled(name=f"ff-{T}-{n}-{m}", inp=n, out=m, tokens=T)
    Xb, Gb = syn.flipflop_streams(cfg)
    X, G = syn.bf16_bits_to_f32(Xb).astype(np.float64), syn.bf16_bits_to_f32(Gb).astype(np.float64)
    ref = o.flipflop(X, G, 3)
    for k in (1, 2, 3):
        A, B = _gpu(torch, Xb, Gb, k)
        Ar, Br = ref[k - 1]
        ea, eb = rel_fro(A, Ar), rel_fro(B, Br)
        print(f"  k={k}: rel err A {ea:.2e}  B {eb:.2e}")
        assert ea <= TOL and eb <= TOL, (k, ea, eb)
        assert np.array_equal(A, A.T) and np.array_equal(B, B.T)


def test_flipflop_full_factorial_closed_form():
    """Tokens = every pair of 160 activations and 144 gradients: the fixed point after one
    iteration is A = Abar tr(Gbar) / m, B = m Gbar / tr(Gbar) (the oracle's pinned closed
    form), and the GPU stays on it at iteration 3."""
    torch = torch_cuda()
    announce("flipflop full factorial 128 x 128")
    n = m = 128
    rng = np.random.default_rng(41)
    xs = rng.standard_normal((160, n)) * np.exp(0.7 * rng.standard_normal(n))
    gs = rng.standard_normal((144, m)) * np.exp(0.7 * rng.standard_normal(m))
    xb, gb = syn.f32_to_bf16_bits(xs.astype(np.float32)), syn.f32_to_bf16_bits(gs.astype(np.float32))
    Xb = np.repeat(xb, 144, axis=0)
    Gb = np.tile(gb, (160, 1))
    xd, gd = syn.bf16_bits_to_f32(xb).astype(np.float64), syn.bf16_bits_to_f32(gb).astype(np.float64)
    Abar, Gbar = xd.T @ xd / 160, gd.T @ gd / 144
    for k in (1, 3):
        A, B = _gpu(torch, Xb, Gb, k)
        ea = rel_fro(A, Abar * np.trace(Gbar) / m)
        eb = rel_fro(B, m * Gbar / np.trace(Gbar))
        print(f"  k={k}: rel err A {ea:.2e}  B {eb:.2e}")
        assert ea <= TOL and eb <= TOL


@pytest.mark.slow
def test_flipflop_full_width():
    """Llama-2-7B q_proj width (4096 x 4096) on 16384 tokens of the c2 streams, two
    iterations, against the oracle."""
    torch = torch_cuda()
    announce("flipflop full width 4096 x 4096, T=16384")
    cfg = syn.C2.scaled(name="ff-c2-16k", tokens=16384)
    Xb, Gb = syn.flipflop_streams(cfg)
    X, G = syn.bf16_bits_to_f32(Xb).astype(np.float64), syn.bf16_bits_to_f32(Gb).astype(np.float64)
    ref = o.flipflop(X, G, 2)
    A, B = _gpu(torch, Xb, Gb, 2)
    ea, eb = rel_fro(A, ref[1][0]), rel_fro(B, ref[1][1])
    print(f"  k=2: rel err A {ea:.2e}  B {eb:.2e}")
    assert ea <= TOL and eb <= TOL
