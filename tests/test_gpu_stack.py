"""GPU parity on the decoder-stack workload: 32 Llama-2-7B layers x 7 linears,
32768 calibration tokens per layer, per-sublayer bits in {2, 3, 4} allocated from
tr(H_G) tr(H_X) to an average of 2.5 bits per weight.

The engine builds all 224 pairs of factors and their traces (kq_accumulate_hessian,
kq_sensitivity); the oracle takes each trace as the stream's squared norm
(tr(A^T A) = ||A||_F^2, exact in fp64).  Bits: identical between the library
allocator on the engine's traces and the oracle allocator on the oracle's traces
(and on shared inputs); the smallest relative gap between winning and runner-up
gains is reported as the tie margin.  One sublayer of each shape is then quantized
at full size with its allocated width (sampled-row parity and both losses)."""
import time

import numpy as np
import pytest

import oracle as o
import synthetic as syn
from tests.fullsize_util import check_rows, dequant, oracle_hessian, run_engine
from tests.gpu_util import announce, rel_fro, torch_cuda

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sq_norm(bits: np.ndarray, chunk: int = 8192) -> float:
    """||A||_F^2 of a bf16 stream: squares exact in fp32, summed in fp64, threaded."""
    from concurrent.futures import ThreadPoolExecutor

    def part(t):
        a = (bits[t:t + chunk].astype(np.uint32) << np.uint32(16)).view(np.float32)
        return float(np.sum(a * a, dtype=np.float64))

    with ThreadPoolExecutor(16) as ex:
        return float(np.sum(list(ex.map(part, range(0, bits.shape[0], chunk)))))


def _gen(c, which):
    """One stream of a sublayer and its squared norm (host, fp64)."""
    bits = syn.stream(c, which)
    return bits, _sq_norm(bits)


def _submit_layer(pool, layer):
    """Queue a layer's distinct streams: its activation streams (q/k/v share one, gate/up
    share one) and its seven gradient streams."""
    cfgs = syn.stack_sublayer_configs(layer)
    xs = {}
    for c in cfgs:
        xs.setdefault(c.x_stream, c)
    fx = {k: pool.submit(_gen, c, "x") for k, c in xs.items()}
    fg = [pool.submit(_gen, c, "g") for c in cfgs]
    return cfgs, fx, fg


def test_decoder_stack_allocation_and_sublayers():
    from concurrent.futures import ThreadPoolExecutor
    torch = torch_cuda()
    import post_quantization_syrk_amd as kq
    t_all = time.time()
    sens_gpu, sens_ref, numel, names = [], [], [], []
    # streams are drawn on the host a layer ahead of the GPU work, four at a time (each
    # stream's generator is itself threaded over its token chunks)
    with ThreadPoolExecutor(4) as pool:
        nxt = _submit_layer(pool, 0)
        for layer in range(syn.STACK_LAYERS):
            cfgs, fx, fg = nxt
            if layer + 1 < syn.STACK_LAYERS:
                nxt = _submit_layer(pool, layer + 1)
            hx, nx = {}, {}
            for k, f in fx.items():
                bits, nx[k] = f.result()
                c = next(c for c in cfgs if c.x_stream == k)
                X = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
                H = torch.empty((c.inp, c.inp), device="cuda")
                kq.kq_accumulate_hessian(X, H)
                hx[k] = H
                del X, bits
            for c, f in zip(cfgs, fg):
                bits, ng = f.result()
                G = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
                HG = torch.empty((c.out, c.out), device="cuda")
                kq.kq_accumulate_hessian(G, HG)
                tx, tg, s = kq.kq_sensitivity(hx[c.x_stream], HG)
                assert tx == pytest.approx(nx[c.x_stream], rel=1e-5)
                assert tg == pytest.approx(ng, rel=1e-5)
                sens_gpu.append(s)
                sens_ref.append(nx[c.x_stream] * ng)
                numel.append(c.params)
                names.append(c.name)
                del G, HG, bits
            del hx, fx, fg
            announce(f"stack layer {layer}: traces done ({time.time() - t_all:.0f} s)")
    assert len(sens_gpu) == 224
    bits_ref, margin = o.allocate_bits(sens_ref, numel, (2, 3, 4), 5, 2, report_margin=True)
    bits_lib_shared = kq.kq_allocate_bits(sens_ref, numel, (2, 3, 4), 5, 2)
    bits_lib_own = kq.kq_allocate_bits(sens_gpu, numel, (2, 3, 4), 5, 2)
    rel_s = max(abs(a - b) / b for a, b in zip(sens_gpu, sens_ref))
    avg = sum(b * n for b, n in zip(bits_ref, numel)) / sum(numel)
    announce(f"stack: max sensitivity rel diff {rel_s:.2e}, tie margin {margin:.3e}, "
             f"avg bits {avg:.4f}, counts {{2: {bits_ref.count(2)}, 3: {bits_ref.count(3)}, 4: {bits_ref.count(4)}}}")
    assert bits_lib_shared == bits_ref
    assert bits_lib_own == bits_ref
    assert sum(b * n for b, n in zip(bits_ref, numel)) <= (sum(numel) * 5) // 2
    assert set(bits_ref) <= {2, 3, 4}
    torch.cuda.empty_cache()
    # full-size quantization of one sublayer of each shape (q 4096 x 4096, gate 11008 x 4096,
    # down 4096 x 11008) at its allocated width, the widths spread over {2, 3, 4} where the
    # allocation allows: sampled-row codes, and both losses against the oracle's own factors
    picks, used = [], set()
    for k in (0, 4, 6):
        cands = [layer for layer in range(syn.STACK_LAYERS) if bits_ref[layer * 7 + k] not in used]
        layer = cands[0] if cands else (0, 15, 31)[(0, 4, 6).index(k)]
        used.add(bits_ref[layer * 7 + k])
        picks.append((layer, k))
    for layer, k in picks:
        cfg = syn.stack_sublayer_configs(layer)[k]
        cfg = cfg.scaled(bits=bits_ref[layer * 7 + k])
        bx, bg, W = syn.stream(cfg, "x"), syn.stream(cfg, "g"), syn.weights(cfg)
        s_in, s_out = syn.signs(cfg, "in"), syn.signs(cfg, "out")
        g = run_engine(cfg, bx, bg, W, s_in, s_out, want_loss=True)
        HX, HG = oracle_hessian(bx), oracle_hessian(bg)
        assert rel_fro(g["HX"], HX) <= 1e-5 and rel_fro(g["HG"], HG) <= 1e-5
        Wt, HXt, HGt, _, _ = o.biip(W.astype(np.float64), HX, HG, s_in, s_out, cfg.alpha, o.BIIP_FULL,
                                    cfg.had_in, cfg.had_out)
        assert rel_fro(g["Wt"], Wt) <= 1e-5 and rel_fro(g["HXt"], HXt) <= 1e-5
        assert rel_fro(g["HGt"], HGt) <= 1e-5
        rows = np.sort(np.random.default_rng(layer).choice(cfg.out, 32, replace=False))
        res = check_rows(g, Wt, HXt, cfg, rows, o.damp_and_factor(HXt, cfg.damp))
        dW = Wt - dequant(g["codes"], g["scales"], g["zeros"], cfg.group)
        L_direct = o.proxy_loss(dW, HXt, HGt)
        L_pred = o.predicted_loss(g["E"], HGt)
        announce(f"stack: {cfg.name} W{cfg.bits} sampled rows match ({res.accepted_ties} ties adopted); "
                 f"losses engine {g['loss'][0]:.6e} / {g['loss'][1]:.6e}, oracle {L_direct:.6e} / {L_pred:.6e}")
        assert g["loss"][0] == pytest.approx(L_direct, rel=1e-3)
        assert g["loss"][1] == pytest.approx(L_pred, rel=1e-3)
        assert g["loss"][1] > g["loss"][0]
        del bx, bg, g
        torch.cuda.empty_cache()
