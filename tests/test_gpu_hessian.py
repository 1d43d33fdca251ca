"""GPU parity: Hessian factors and sensitivity against the fp64 oracle.

Tolerance: relative Frobenius error of H <= 1e-3 (bf16 products are exact in
fp32; accumulation is fp32, so ~1e-6 is expected); traces within 1e-5."""
import numpy as np
import pytest

import oracle as o
import synthetic as syn
from tests.gpu_util import announce, rel_fro, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu


def gpu_hessian(bits, lda=None, accumulate_from=None):
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    T, n = bits.shape
    A = to_dev_bf16(bits, lda)
    H = torch.full((n, n), float("nan"), device="cuda", dtype=torch.float32)
    if accumulate_from is not None:
        H.copy_(torch.from_numpy(accumulate_from.astype(np.float32)))
    kq.kq_accumulate_hessian(A, H, accumulate=accumulate_from is not None)
    torch.cuda.synchronize()
    return H.cpu().numpy()


def test_c1_hessians_match_oracle():
    cfg = syn.C1
    for which in ("x", "g"):
        announce(f"c1 hessian {which}")
        bits = syn.stream(cfg, which)
        H = gpu_hessian(bits)
        ref = o.hessian_factor(o.bf16_bits_to_f64(bits))
        assert rel_fro(H, ref) <= 1e-3
        assert rel_fro(H, ref) <= 1e-5   # fp32 accumulation of exact products
        assert np.array_equal(H, H.T)


@pytest.mark.parametrize("T,n,lda", [(1000, 300, 304), (64, 1, 8), (777, 520, 520), (1, 17, 24),
                                     (4096, 512, 512), (130, 257, 264)])
def test_ragged_shapes(T, n, lda):
    announce(f"hessian ragged T={T} n={n} lda={lda}")
    rng = np.random.default_rng(T * 1000 + n)
    x = (rng.standard_normal((T, n)) * np.exp(rng.standard_normal(n))).astype(np.float32)
    bits = syn.f32_to_bf16_bits(x)
    H = gpu_hessian(bits, lda)
    ref = o.hessian_factor(o.bf16_bits_to_f64(bits))
    assert rel_fro(H, ref) <= 1e-5
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("T,n,lda", [(20000, 600, 608), (31, 256, 256), (1000, 300, 304)])
def test_kernel_variants_agree(variant, T, n, lda):
    """Every SYRK kernel (the register-staged fallback with 4/8 waves, tile/split-major; the
    direct-to-LDS default) against the oracle, on shapes with many token splits, a ragged
    last stage and a ragged last tile."""
    import post_quantization_syrk_amd as kq
    announce(f"hessian variant {variant} T={T} n={n} lda={lda}")
    rng = np.random.default_rng(T + n)
    x = (rng.standard_normal((T, n)) * np.exp(rng.standard_normal(n))).astype(np.float32)
    bits = syn.f32_to_bf16_bits(x)
    with kq.testing_select(kq.KQ_TESTING_SYRK_KERNEL, variant):
        H = gpu_hessian(bits, lda)
    ref = o.hessian_factor(o.bf16_bits_to_f64(bits))
    assert rel_fro(H, ref) <= 1e-5
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("T,n,lda", [(200, 600, 600), (100, 257, 264), (480, 1024, 1032)])
def test_single_token_split_several_tiles(T, n, lda):
    """Fewer than 512 tokens make one token split over several (ragged) tiles; H starts as
    NaN, so an entry left unwritten fails.  A second chunk is then accumulated on top."""
    announce(f"hessian single split T={T} n={n} lda={lda}")
    rng = np.random.default_rng(T * n)
    x = (rng.standard_normal((2 * T, n)) * np.exp(rng.standard_normal(n))).astype(np.float32)
    bits = syn.f32_to_bf16_bits(x)
    H = gpu_hessian(bits[:T], lda)
    ref = o.hessian_factor(o.bf16_bits_to_f64(bits[:T]))
    assert rel_fro(H, ref) <= 1e-5
    assert np.array_equal(H, H.T)
    H2 = gpu_hessian(bits[T:], lda, accumulate_from=H)
    ref2 = o.hessian_factor(o.bf16_bits_to_f64(bits))
    assert rel_fro(H2, ref2) <= 1e-5
    assert np.array_equal(H2, H2.T)


def test_empty_stream_gives_zero_and_accumulate_keeps():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("hessian T=0")
    A = torch.zeros((0, 40), dtype=torch.bfloat16, device="cuda")
    H = torch.full((40, 40), 7.0, device="cuda")
    kq.kq_accumulate_hessian(A, H, accumulate=False)
    assert float(H.abs().max()) == 0.0
    H.fill_(3.0)
    kq.kq_accumulate_hessian(A, H, accumulate=True)
    assert float((H - 3.0).abs().max()) == 0.0


def test_accumulate_over_chunks_equals_whole_stream():
    announce("hessian accumulate chunks")
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((3000, 384)) * np.exp(rng.standard_normal(384))).astype(np.float32)
    bits = syn.f32_to_bf16_bits(x)
    H1 = gpu_hessian(bits[:1234])
    H2 = gpu_hessian(bits[1234:], accumulate_from=H1)
    ref = o.hessian_factor(o.bf16_bits_to_f64(bits))
    assert rel_fro(H2, ref) <= 1e-5


def test_c1_sensitivity_matches_oracle():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("c1 sensitivity")
    cfg = syn.C1
    bx, bg = syn.stream(cfg, "x"), syn.stream(cfg, "g")
    HX = torch.from_numpy(gpu_hessian(bx)).cuda()
    HG = torch.from_numpy(gpu_hessian(bg)).cuda()
    tx, tg, s = kq.kq_sensitivity(HX, HG)
    X, G = o.bf16_bits_to_f64(bx), o.bf16_bits_to_f64(bg)
    ox, og, os_ = o.sensitivity(o.hessian_factor(X), o.hessian_factor(G))
    assert tx == pytest.approx(ox, rel=1e-5)
    assert tg == pytest.approx(og, rel=1e-5)
    assert s == pytest.approx(os_, rel=1e-5)
    # independent route: stream norms
    assert s == pytest.approx(o.stream_sq_norm(X) * o.stream_sq_norm(G), rel=1e-5)
    # the device-memory variant: the same three values, bit for bit
    dev = torch.full((3,), float("nan"), dtype=torch.float64, device="cuda")
    kq.kq_sensitivity_async(HX, HG, dev)
    torch.cuda.synchronize()
    assert dev.cpu().tolist() == [tx, tg, s]


@pytest.mark.slow
def test_c2_full_size_sampled_entries():
    """Llama-2-7B q_proj stream (131072 x 4096): sampled entries computed one by one in fp64."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    cfg = syn.C2
    announce("c2 full-size hessian x")
    bits = syn.stream(cfg, "x")
    A = to_dev_bf16(bits)
    H = torch.empty((cfg.inp, cfg.inp), device="cuda")
    kq.kq_accumulate_hessian(A, H)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    i = rng.integers(0, cfg.inp, 48)
    j = rng.integers(0, cfg.inp, 48)
    i[:8] = j[:8]                             # diagonal samples
    Hs = H[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].cpu().numpy()
    Xi = o.bf16_bits_to_f64(bits[:, i])
    Xj = o.bf16_bits_to_f64(bits[:, j])
    ref = o.hessian_factor_entry(Xi, Xj)
    scale = np.sqrt(o.hessian_factor_entry(Xi, Xi) * o.hessian_factor_entry(Xj, Xj))
    assert np.max(np.abs(Hs - ref) / scale) <= 1e-5
    Hc = H.cpu().numpy()
    assert np.array_equal(Hc, Hc.T)
    # trace through the library against the stream's squared norm (chunked, fp64)
    tx, _, _ = kq.kq_sensitivity(H, H)
    norm = sum(o.stream_sq_norm(o.bf16_bits_to_f64(bits[t:t + 8192])) for t in range(0, cfg.tokens, 8192))
    assert tx == pytest.approx(norm, rel=1e-5)
