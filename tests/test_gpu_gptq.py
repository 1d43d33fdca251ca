"""GPU parity: damped factorization + blocked GPTQ + packing + proxy losses.

Codes are compared with the replay rule: walking the columns in order, the
oracle adopts the GPU's code only where its own pre-rounding value w/s lies
within 1e-4 of a rounding midpoint and the GPU chose the other neighbour (both
are correct results); any other difference is a hard mismatch.  Gate: 0 hard
mismatches and at most 0.1 % accepted flips.  Scales within 1e-5 relative,
zero points equal, losses within 1e-3 relative, packed words bit-exact with
the oracle's packing of the GPU's codes."""
import numpy as np
import pytest

import oracle as o
import synthetic as syn
from tests.gpu_util import announce, rel_fro, to_dev_bf16, torch_cuda

pytestmark = pytest.mark.gpu


def spd(rng, n, T=None, outliers=0):
    T = T or 2 * n
    sc = np.exp(rng.standard_normal(n))
    if outliers:
        sc[rng.choice(n, outliers, replace=False)] *= 20
    A = rng.standard_normal((T, n)) * sc
    return A.T @ A


def gpu_quantize(Wt, HXt, HGt, bits, group, block, damp=0.01, want_loss=True, act_order=0,
                 w_clip=0):
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    out_n, in_n = Wt.shape
    p = kq.make_params(bits, group, block, damp, act_order=act_order, w_clip=w_clip)
    ws = torch.empty(kq.kq_quantize_layer_workspace(p, out_n, in_n, want_loss), dtype=torch.uint8,
                     device="cuda")
    W = torch.from_numpy(np.ascontiguousarray(Wt, dtype=np.float32)).cuda()
    HX = torch.from_numpy(np.ascontiguousarray(HXt, dtype=np.float32)).cuda()
    HG = None if HGt is None else torch.from_numpy(np.ascontiguousarray(HGt, dtype=np.float32)).cuda()
    packed = torch.zeros((out_n, in_n * bits // 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((out_n, in_n // group), device="cuda")
    zeros = torch.zeros((out_n, in_n // group), dtype=torch.uint8, device="cuda")
    codes = torch.zeros((out_n, in_n), dtype=torch.uint8, device="cuda")
    loss = kq.kq_quantize_layer(p, W, HX, HG, packed, scales, zeros, ws, codes=codes,
                                want_loss=want_loss)
    torch.cuda.synchronize()
    return dict(E=W.cpu().numpy(), packed=packed.cpu().numpy().view(np.uint32),
                scales=scales.cpu().numpy(), zeros=zeros.cpu().numpy(),
                codes=codes.cpu().numpy().astype(np.int64), loss=loss)


def check_against_oracle(g, Wt, HXt, HGt, bits, group, damp=0.01, rows=None, act_order=False,
                         w_clip=False):
    sel = slice(None) if rows is None else rows
    ref = o.quantize_layer(Wt, HXt, HGt, bits, group, damp, replay_codes=g["codes"][sel],
                           rows=rows, act_order=act_order, w_clip=w_clip,
                           replay_scales=g["scales"][sel][:, 0] if w_clip else None)
    if w_clip:
        # the clip search: same candidate as the oracle, or one within 1e-5 of its best error
        assert ref["clip_hard_mismatches"] == 0
    res = ref["gptq"]
    n_codes = res.codes.size
    assert res.hard_mismatches == 0, f"{res.hard_mismatches} hard mismatches at {res.mismatch_positions[:5]}"
    assert res.accepted_ties <= 0.001 * n_codes
    gc = g["codes"] if rows is None else g["codes"][rows]
    assert np.array_equal(res.codes, gc)
    gs = g["scales"] if rows is None else g["scales"][rows]
    gz = g["zeros"] if rows is None else g["zeros"][rows]
    assert np.max(np.abs(gs - res.scales) / np.abs(res.scales)) <= 1e-5
    assert np.array_equal(gz.astype(np.int64), res.zeros.astype(np.int64))
    # packed words: the oracle's bit-by-bit packing of these codes
    gp = g["packed"] if rows is None else g["packed"][rows]
    assert np.array_equal(gp, o.pack_codes(gc, bits))
    # GPTQ's errors e_j are left in W_rot
    gE = g["E"] if rows is None else g["E"][rows]
    assert rel_fro(gE, res.E) <= 1e-4
    if rows is None and g["loss"] is not None:
        ld, lp = g["loss"]
        assert ld == pytest.approx(ref["loss_direct"], rel=1e-3)
        assert lp == pytest.approx(ref["loss_pred"], rel=1e-3)
    return ref


@pytest.mark.parametrize("bits,group,block", [(2, 64, 64), (2, 128, 128), (3, 32, 128), (4, 128, 128),
                                              (4, 16, 64), (3, 64, 128), (2, 256, 64), (3, 32, 64)])
def test_quantize_synthetic_layers(bits, group, block):
    announce(f"gptq synthetic bits={bits} group={group} block={block}")
    rng = np.random.default_rng(bits * 100 + group + block)
    out_n, in_n = 72, 256
    Wt = rng.standard_normal((out_n, in_n)) * 0.05
    HXt = spd(rng, in_n, outliers=2).astype(np.float32).astype(np.float64)
    HGt = spd(rng, out_n).astype(np.float32).astype(np.float64)
    Wt = Wt.astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, HGt, bits, group, block)
    check_against_oracle(g, Wt, HXt, HGt, bits, group)


@pytest.mark.parametrize("bits,block,act_order,w_clip,with_hg", [
    (2, 128, 1, 0, True), (3, 64, 1, 0, False), (4, 128, 0, 1, True), (2, 64, 0, 1, False),
    (2, 128, 1, 1, True), (3, 128, 1, 1, False), (4, 64, 1, 1, True)])
def test_quantize_act_order_and_clip(bits, block, act_order, w_clip, with_hg):
    """The base recipe's options: one grid per row (group = in), act_order and/or w_clip."""
    announce(f"gptq act_order={act_order} w_clip={w_clip} bits={bits} block={block}")
    rng = np.random.default_rng(bits * 10 + block + 3 * act_order + 5 * w_clip)
    out_n, in_n = 72, 256
    Wt = rng.standard_normal((out_n, in_n)) * 0.05
    Wt[:, rng.choice(in_n, 3, replace=False)] *= 8
    HXt = spd(rng, in_n, outliers=3).astype(np.float32).astype(np.float64)
    HGt = spd(rng, out_n).astype(np.float32).astype(np.float64) if with_hg else None
    Wt = Wt.astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, HGt, bits, in_n, block, act_order=act_order, w_clip=w_clip)
    ref = check_against_oracle(g, Wt, HXt, HGt, bits, in_n, act_order=bool(act_order),
                               w_clip=bool(w_clip))
    if act_order:
        assert not np.array_equal(ref["perm"], np.arange(in_n))
    if w_clip:
        assert np.any(ref["clip_choice"] > 0)


def test_quantize_act_order_dead_channel_and_direct_paths():
    """act_order with a dead channel (its zero diagonal ranks as 1), and the row kernels'
    direct (no LDS staging) paths that rows longer than 16384 floats take."""
    import post_quantization_syrk_amd as kq
    with kq.testing_select(kq.KQ_TESTING_ROW_LDS_BYTES, 0):
        _act_order_dead_channel()


def _act_order_dead_channel():
    announce("gptq act_order + w_clip, dead channel, direct row paths")
    rng = np.random.default_rng(41)
    HXt = spd(rng, 192, outliers=2)
    HXt[7, :] = 0
    HXt[:, 7] = 0
    HXt = HXt.astype(np.float32).astype(np.float64)
    Wt = (rng.standard_normal((40, 192)) * 0.05).astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, None, 3, 192, 64, act_order=1, w_clip=1)
    ref = check_against_oracle(g, Wt, HXt, None, 3, 192, act_order=True, w_clip=True)
    assert ref["dead"][7]
    assert np.all(g["codes"][:, 7] == g["zeros"][:, 0])   # a zeroed column codes as the zero point


def test_act_order_needs_one_grid_per_row():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    for kw in ({"act_order": 1}, {"w_clip": 1}):
        p = kq.make_params(2, 64, 64, **kw)
        with pytest.raises(kq.KQError) as e:
            kq.kq_quantize_layer_workspace(p, 16, 128, False)
        assert e.value.status == kq.KQ_ENOTIMPL


@pytest.mark.parametrize("bits,group,block", [(4, 128, 128), (2, 64, 64), (3, 640, 128)])
def test_quantize_block_pairs(bits, group, block):
    """640 columns: two-block launches whose feedback product has columns before them, and a
    last odd block alone (block 128); group 640 takes the one-grid-per-row kernel."""
    announce(f"gptq block pairs bits={bits} group={group} block={block}")
    rng = np.random.default_rng(bits * 1000 + group + block)
    out_n, in_n = 72, 640
    Wt = rng.standard_normal((out_n, in_n)) * 0.05
    HXt = spd(rng, in_n, outliers=2).astype(np.float32).astype(np.float64)
    HGt = spd(rng, out_n).astype(np.float32).astype(np.float64)
    Wt = Wt.astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, HGt, bits, group, block)
    check_against_oracle(g, Wt, HXt, HGt, bits, group)


@pytest.mark.parametrize("sb", [128, 256, 512, 1024])
def test_factorization_superblock_widths(sb):
    """The factorization defers each block's update of the columns left of its super-block to
    one rank-(super-block) product; every width (one block per super-block boundary at 128,
    none at 1024 for this 1024-wide layer) gives GPTQ results that match the oracle."""
    import post_quantization_syrk_amd as kq
    announce(f"gptq factorization with super-blocks of {sb} columns")
    rng = np.random.default_rng(21)
    out_n, in_n = 72, 1024
    Wt = (rng.standard_normal((out_n, in_n)) * 0.05).astype(np.float32).astype(np.float64)
    HXt = spd(rng, in_n, outliers=2).astype(np.float32).astype(np.float64)
    HGt = spd(rng, out_n).astype(np.float32).astype(np.float64)
    with kq.testing_select(kq.KQ_TESTING_FACTOR_SUPERBLOCK, sb):
        g = gpu_quantize(Wt, HXt, HGt, 3, 128, 128)
    check_against_oracle(g, Wt, HXt, HGt, 3, 128)


def test_quantize_without_hg_and_ragged_rows():
    announce("gptq no H_G, out=50")
    rng = np.random.default_rng(11)
    Wt = (rng.standard_normal((50, 384)) * 0.05).astype(np.float32).astype(np.float64)
    HXt = spd(rng, 384).astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, None, 2, 128, 128)
    check_against_oracle(g, Wt, HXt, None, 2, 128)


def test_quantize_dead_channel():
    announce("gptq dead channel")
    rng = np.random.default_rng(12)
    HXt = spd(rng, 128)
    HXt[5, :] = 0
    HXt[:, 5] = 0
    HXt = HXt.astype(np.float32).astype(np.float64)
    Wt = (rng.standard_normal((32, 128)) * 0.05).astype(np.float32).astype(np.float64)
    g = gpu_quantize(Wt, HXt, None, 4, 64, 64)
    ref = check_against_oracle(g, Wt, HXt, None, 4, 64)
    assert ref["dead"][5]


def test_quantize_not_spd_raises():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("gptq not spd")
    rng = np.random.default_rng(13)
    H = spd(rng, 64)
    H[10, 10] = -50.0 * H[10, 10]
    with pytest.raises(kq.NotSPDError):
        gpu_quantize(rng.standard_normal((16, 64)), H, None, 2, 64, 64, want_loss=False)


def test_workspace_too_small():
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    p = kq.make_params(2, 64, 64)
    W = torch.zeros((16, 64), device="cuda")
    H = torch.eye(64, device="cuda")
    packed = torch.zeros((16, 4), dtype=torch.int32, device="cuda")
    sc = torch.zeros((16, 1), device="cuda")
    zr = torch.zeros((16, 1), dtype=torch.uint8, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.kq_quantize_layer(p, W, H, None, packed, sc, zr, ws)
    assert e.value.status == kq.KQ_EWORKSPACE


def test_c1_end_to_end():
    """Seeded c1 layer through all GPU stages vs the oracle's own fp64 pipeline."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("c1 end-to-end quantize")
    cfg = syn.C1
    bx, bg = syn.stream(cfg, "x"), syn.stream(cfg, "g")
    W = syn.weights(cfg)
    s_in, s_out = syn.signs(cfg, "in"), syn.signs(cfg, "out")
    HXd = torch.empty((cfg.inp, cfg.inp), device="cuda")
    HGd = torch.empty((cfg.out, cfg.out), device="cuda")
    kq.kq_accumulate_hessian(to_dev_bf16(bx), HXd)
    kq.kq_accumulate_hessian(to_dev_bf16(bg), HGd)
    Wd = torch.from_numpy(W).cuda()
    di, do = torch.empty(cfg.inp, device="cuda"), torch.empty(cfg.out, device="cuda")
    kq.kq_biip_rotate(Wd, Wd, HXd, HXd, HGd, HGd, torch.from_numpy(s_in).cuda(),
                      torch.from_numpy(s_out).cuda(), di, do, cfg.alpha, 0, cfg.had_in, cfg.had_out)
    p = kq.make_params(cfg.bits, cfg.group, cfg.block, cfg.damp)
    ws = torch.empty(kq.kq_quantize_layer_workspace(p, cfg.out, cfg.inp, True), dtype=torch.uint8,
                     device="cuda")
    packed = torch.zeros((cfg.out, cfg.inp * cfg.bits // 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((cfg.out, cfg.inp // cfg.group), device="cuda")
    zeros = torch.zeros((cfg.out, cfg.inp // cfg.group), dtype=torch.uint8, device="cuda")
    codes = torch.zeros((cfg.out, cfg.inp), dtype=torch.uint8, device="cuda")
    loss = kq.kq_quantize_layer(p, Wd, HXd, HGd, packed, scales, zeros, ws, codes=codes,
                                want_loss=True)
    g = dict(E=Wd.cpu().numpy(), packed=packed.cpu().numpy().view(np.uint32),
             scales=scales.cpu().numpy(), zeros=zeros.cpu().numpy(),
             codes=codes.cpu().numpy().astype(np.int64), loss=loss)
    # oracle: own fp64 factors and rotation from the same streams
    HX = o.hessian_factor(o.bf16_bits_to_f64(bx))
    HG = o.hessian_factor(o.bf16_bits_to_f64(bg))
    Wt, HXt, HGt, _, _ = o.biip(W.astype(np.float64), HX, HG, s_in, s_out, cfg.alpha, 0,
                                cfg.had_in, cfg.had_out)
    ref = check_against_oracle(g, Wt, HXt, HGt, cfg.bits, cfg.group, cfg.damp)
    # the raw-domain loss equals the rotated-domain loss (BiIP invariance)
    print(f"c1: loss_direct {loss[0]:.6e} (oracle {ref['loss_direct']:.6e}), "
          f"accepted ties {ref['gptq'].accepted_ties}")


@pytest.mark.parametrize("dead_ch", [None, 7])
def test_engine_damping_read_from_its_losses(dead_ch):
    """The engine's lambda, pinned without the oracle: with H_G = I the predicted loss exceeds
    the direct one by exactly lambda ||W~ - Qhat||_F^2 (W~ - Qhat = E U and U H_d U^T = I).
    lambda must be 1 % of the mean diagonal of the H~_X it is given, a dead channel (zero
    diagonal) counting as 1.  The diagonal is scaled to a mean of 1e-3, so a mean taken before
    the dead channel is set (or a trace, or another damp) misses by far more than the
    tolerance."""
    torch_cuda()
    rng = np.random.default_rng(41)
    out_n, n = 64, 256
    H = spd(rng, n, outliers=6)
    H *= 1e-3 / np.mean(np.diag(H))       # diagonal ~1e-3: a dead channel's 1 moves the mean 4x
    if dead_ch is not None:
        H[dead_ch, :] = 0.0
        H[:, dead_ch] = 0.0
    H = H.astype(np.float32).astype(np.float64)
    diag = [1.0 if H[i, i] == 0.0 else float(H[i, i]) for i in range(n)]
    lam_hand = 0.01 * sum(diag) / n
    W = (rng.standard_normal((out_n, n)) * 0.02).astype(np.float32)
    g = gpu_quantize(W, H, None, 2, 64, 64, damp=0.01, want_loss=True)
    W0 = W.astype(np.float64)
    if dead_ch is not None:
        W0[:, dead_ch] = 0.0
    s = np.repeat(g["scales"].astype(np.float64), 64, axis=1)
    z = np.repeat(g["zeros"].astype(np.float64), 64, axis=1)
    dW = W0 - s * (g["codes"] - z)
    lam_engine = (g["loss"][1] - g["loss"][0]) / float(np.sum(dW * dW))
    announce(f"damping: engine lambda {lam_engine:.6e}, by hand {lam_hand:.6e}")
    assert lam_engine == pytest.approx(lam_hand, rel=1e-3)


def test_quantize_async_matches_sync_and_reports_status():
    """kq_quantize_layer_async leaves the status and losses in device memory: on several
    streams at once its outputs equal the synchronous call's bit for bit, its losses match
    the synchronous ones, and a non-positive pivot is reported as KQ_ENOTSPD in the status."""
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    announce("gptq async calls on three streams")
    rng = np.random.default_rng(31)
    cases = []
    for out_n, in_n, bits, group in ((96, 512, 3, 128), (64, 384, 4, 128), (130, 256, 2, 64)):
        Wt = (rng.standard_normal((out_n, in_n)) * 0.05).astype(np.float32)
        HXt = spd(rng, in_n, outliers=2).astype(np.float32)
        HGt = spd(rng, out_n).astype(np.float32)
        cases.append((Wt, HXt, HGt, bits, group))
    streams = [torch.cuda.Stream() for _ in cases]
    outs = []
    for (Wt, HXt, HGt, bits, group), st in zip(cases, streams):
        out_n, in_n = Wt.shape
        p = kq.make_params(bits, group, 128 if in_n % 128 == 0 else 64, 0.01)
        with torch.cuda.stream(st):
            W = torch.from_numpy(Wt).cuda()
            HX, HG = torch.from_numpy(HXt).cuda(), torch.from_numpy(HGt).cuda()
            ws = torch.empty(kq.kq_quantize_layer_workspace(p, out_n, in_n, True), dtype=torch.uint8,
                             device="cuda")
            o = dict(W=W, packed=torch.zeros((out_n, in_n * bits // 32), dtype=torch.int32, device="cuda"),
                     scales=torch.zeros((out_n, in_n // group), device="cuda"),
                     zeros=torch.zeros((out_n, in_n // group), dtype=torch.uint8, device="cuda"),
                     codes=torch.zeros((out_n, in_n), dtype=torch.uint8, device="cuda"),
                     loss=torch.zeros(2, dtype=torch.float64, device="cuda"),
                     status=torch.full((1,), -1, dtype=torch.int32, device="cuda"), ws=ws, HX=HX, HG=HG)
            kq.kq_quantize_layer_async(p, W, HX, HG, o["packed"], o["scales"], o["zeros"], ws, o["status"],
                                       codes=o["codes"], loss=o["loss"], stream=st)
        outs.append((o, p))
    torch.cuda.synchronize()
    for (Wt, HXt, HGt, bits, group), (o, p) in zip(cases, outs):
        assert int(o["status"].item()) == kq.KQ_OK
        ref = gpu_quantize(Wt.astype(np.float64), HXt.astype(np.float64), HGt.astype(np.float64), bits,
                           group, p.block)
        assert np.array_equal(o["codes"].cpu().numpy().astype(np.int64), ref["codes"])
        assert np.array_equal(o["packed"].cpu().numpy().view(np.uint32), ref["packed"])
        assert np.array_equal(o["scales"].cpu().numpy(), ref["scales"])
        assert np.array_equal(o["W"].cpu().numpy(), ref["E"])
        lo = o["loss"].cpu().numpy()
        assert lo[0] == pytest.approx(ref["loss"][0], rel=1e-9)
        assert lo[1] == pytest.approx(ref["loss"][1], rel=1e-9)
    # a non-positive pivot: no exception, the status says so
    H = spd(rng, 64)
    H[10, 10] = -50.0 * H[10, 10]
    p = kq.make_params(2, 64, 64, 0.01)
    W = torch.from_numpy(rng.standard_normal((16, 64)).astype(np.float32)).cuda()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(kq.kq_quantize_layer_workspace(p, 16, 64, False), dtype=torch.uint8, device="cuda")
    kq.kq_quantize_layer_async(p, W, torch.from_numpy(H.astype(np.float32)).cuda(), None,
                               torch.zeros((16, 4), dtype=torch.int32, device="cuda"),
                               torch.zeros((16, 1), device="cuda"),
                               torch.zeros((16, 1), dtype=torch.uint8, device="cuda"), ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == kq.KQ_ENOTSPD
