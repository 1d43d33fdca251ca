"""GPU parity: bidirectional incoherence processing against the fp64 oracle.

Tolerance (rotated weights and factors): relative Frobenius error <= 1e-5.
The oracle takes its own fp64 factors from the same seeded streams; the GPU
path takes the factors its own SYRK built."""
import numpy as np
import pytest

import oracle as o
import synthetic as syn
from tests.gpu_util import announce, rel_fro, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu

MODES = {"full": 0, "no_rescale": 1, "in_only": 2, "out_only": 3}


def spd(rng, n, T=None):
    T = T or 2 * n
    A = rng.standard_normal((T, n)) * np.exp(rng.standard_normal(n))
    return A.T @ A


def run_gpu_biip(W, HX, HG, s_in, s_out, alpha, mode, bin_, bout, inplace=False):
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    dev = "cuda"
    Wd = torch.from_numpy(W.astype(np.float32)).to(dev)
    HXd = torch.from_numpy(HX.astype(np.float32)).to(dev)
    HGd = None if HG is None else torch.from_numpy(HG.astype(np.float32)).to(dev)
    if inplace:
        Wo, HXo, HGo = Wd, HXd, HGd
    else:
        Wo, HXo = torch.empty_like(Wd), torch.empty_like(HXd)
        HGo = None if HGd is None else torch.empty_like(HGd)
    si = torch.from_numpy(s_in.astype(np.int8)).to(dev)
    so = torch.from_numpy(s_out.astype(np.int8)).to(dev)
    di = torch.empty(W.shape[1], device=dev)
    do = torch.empty(W.shape[0], device=dev)
    kq.kq_biip_rotate(Wd, Wo, HXd, HXo, HGd, HGo, si, so, di, do, alpha, mode, bin_, bout)
    torch.cuda.synchronize()
    return (Wo.cpu().numpy(), HXo.cpu().numpy(), None if HGo is None else HGo.cpu().numpy(),
            di.cpu().numpy(), do.cpu().numpy())


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("out_n,in_n,bin_,bout", [(256, 256, 256, 256), (96, 768, 256, 32),
                                                  (512, 1024, 1024, 512), (64, 2048, 2048, 16),
                                                  (40, 4096, 0, 8), (24, 8192, 8192, 4),
                                                  (48, 1536, 0, 0), (16, 8192, 4096, 16),
                                                  (2048, 4096, 0, 16)])
def test_biip_matches_oracle(mode, out_n, in_n, bin_, bout):
    announce(f"biip {mode} out={out_n} in={in_n} b=({bin_},{bout})")
    rng = np.random.default_rng(out_n * 7 + in_n)
    W = (rng.standard_normal((out_n, in_n)) * 0.02).astype(np.float32)
    W[:, rng.choice(in_n, 3, replace=False)] *= 20
    HX = spd(rng, in_n, 256).astype(np.float32).astype(np.float64)
    HG = spd(rng, out_n, 256).astype(np.float32).astype(np.float64)
    s_in = rng.choice([-1, 1], in_n)
    s_out = rng.choice([-1, 1], out_n)
    m = MODES[mode]
    Wt, HXt, HGt, di, do = run_gpu_biip(W, HX, HG, s_in, s_out, 0.25, m, bin_, bout)
    rWt, rHXt, rHGt, rdi, rdo = o.biip(W.astype(np.float64), HX, HG, s_in, s_out, 0.25, m,
                                       bin_, bout)
    assert rel_fro(di, rdi) <= 1e-6
    assert rel_fro(do, rdo) <= 1e-6
    assert rel_fro(Wt, rWt) <= 1e-5
    assert rel_fro(HXt, rHXt) <= 1e-5
    assert rel_fro(HGt, rHGt) <= 1e-5


def test_biip_in_place_and_without_hg():
    announce("biip in place / in-only without H_G")
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((128, 512)) * 0.02).astype(np.float32)
    HX = spd(rng, 512).astype(np.float32).astype(np.float64)
    HG = spd(rng, 128).astype(np.float32).astype(np.float64)
    s_in, s_out = rng.choice([-1, 1], 512), rng.choice([-1, 1], 128)
    Wt, HXt, HGt, _, _ = run_gpu_biip(W, HX, HG, s_in, s_out, 0.25, 0, 0, 0, inplace=True)
    rWt, rHXt, rHGt, _, _ = o.biip(W.astype(np.float64), HX, HG, s_in, s_out, 0.25, 0)
    assert rel_fro(Wt, rWt) <= 1e-5 and rel_fro(HXt, rHXt) <= 1e-5 and rel_fro(HGt, rHGt) <= 1e-5
    Wt, HXt, HGt, _, _ = run_gpu_biip(W, HX, None, s_in, s_out, 0.25, 2, 0, 0)
    rWt, rHXt, _, _, _ = o.biip(W.astype(np.float64), HX, None, s_in, s_out, 0.25, 2)
    assert HGt is None
    assert rel_fro(Wt, rWt) <= 1e-5 and rel_fro(HXt, rHXt) <= 1e-5


def test_biip_rejects_bad_blocks():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    W = torch.zeros((64, 96), device="cuda")
    HX = torch.zeros((96, 96), device="cuda")
    HG = torch.zeros((64, 64), device="cuda")
    s = torch.ones(96, dtype=torch.int8, device="cuda")
    so = torch.ones(64, dtype=torch.int8, device="cuda")
    d1, d2 = torch.empty(96, device="cuda"), torch.empty(64, device="cuda")
    with pytest.raises(kq.KQError):
        kq.kq_biip_rotate(W, W, HX, HX, HG, HG, s, so, d1, d2, 0.25, 0, 64, 0)   # 64 does not divide 96
    with pytest.raises(kq.KQError):
        kq.kq_biip_rotate(W, W, HX, HX, None, None, s, so, d1, d2, 0.25, 0, 0, 0)  # H_G needed


def test_c1_end_to_end_rotation():
    """From the seeded c1 streams: GPU SYRKs + BiIP vs the oracle's own fp64 pipeline."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("c1 end-to-end biip")
    cfg = syn.C1
    bx, bg = syn.stream(cfg, "x"), syn.stream(cfg, "g")
    W = syn.weights(cfg)
    s_in, s_out = syn.signs(cfg, "in"), syn.signs(cfg, "out")
    HXd = torch.empty((cfg.inp, cfg.inp), device="cuda")
    HGd = torch.empty((cfg.out, cfg.out), device="cuda")
    kq.kq_accumulate_hessian(to_dev_bf16(bx), HXd)
    kq.kq_accumulate_hessian(to_dev_bf16(bg), HGd)
    Wd = torch.from_numpy(W).cuda()
    Wt = torch.empty_like(Wd)
    di, do = torch.empty(cfg.inp, device="cuda"), torch.empty(cfg.out, device="cuda")
    kq.kq_biip_rotate(Wd, Wt, HXd, HXd, HGd, HGd, torch.from_numpy(s_in).cuda(),
                      torch.from_numpy(s_out).cuda(), di, do, cfg.alpha, 0, cfg.had_in, cfg.had_out)
    torch.cuda.synchronize()
    HX = o.hessian_factor(o.bf16_bits_to_f64(bx))
    HG = o.hessian_factor(o.bf16_bits_to_f64(bg))
    rWt, rHXt, rHGt, rdi, rdo = o.biip(W.astype(np.float64), HX, HG, s_in, s_out, cfg.alpha, 0,
                                       cfg.had_in, cfg.had_out)
    assert rel_fro(Wt.cpu().numpy(), rWt) <= 1e-5
    assert rel_fro(HXd.cpu().numpy(), rHXt) <= 1e-5
    assert rel_fro(HGd.cpu().numpy(), rHGt) <= 1e-5
