"""Throughput of the KronQ per-layer quantization engine on one MI355X.

One step = the whole per-layer path on one synthetic layer whose inputs are
already resident in HBM: H_X = X^T X and H_G = G^T G (bf16 MFMA SYRK),
sensitivity tr(H_G) tr(H_X), BiIP (rescale + randomized Hadamard on both
sides), damping + reverse Cholesky + triangular inverse, blocked GPTQ to
packed codes with scales and zero points.  The proxy loss is a verification
output and is not part of the step.

Default workload: Llama-3-70B-shaped up_proj, 28672 x 8192 weights (bf16 values
~N(0, 0.01^2), 0.1 % outlier input channels x30), 262144 calibration tokens of X
(8192 wide) and G (28672 wide: a 28672 x 28672 fp32 H_G on one GPU), bf16 with
log-normal channel scales (sigma 1 / 1.5), W2 asymmetric min-max, group 128,
block 128, 8192-point input Hadamard, 7 x 4096 output Hadamard.  Other layer
workloads: --workload c1|c2|c2r|c3; --workload c4 runs the 32-layer Llama-2-7B
decoder stack (224 linears, bits allocated to 2.5 per weight).

Prints one JSON line: quantized params/s, the dominant kernel's roofline
(the SYRK, timed with HIP events on its stream) and the CPU oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as syn  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0

WORKLOADS = {"c1": syn.C1, "c2": syn.C2, "c2r": syn.C2R, "c3": syn.C3, "c5": syn.C5}
STACK = "c4"   # the decoder stack (not a single layer)
STACK_STREAMS = 6   # streams the stack's sublayer quantizations are dealt to (pass 2: 905, 835, 850 ms on 4, 6, 8)
DEFAULT_WORKLOAD = "c5"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS) + [STACK],
                    help=f"default {DEFAULT_WORKLOAD} (c2 with --flipflop / --two-sided)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stack-streams", type=int, default=STACK_STREAMS,
                    help="with --workload c4: streams the sublayer quantizations are dealt to")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU budget of the oracle sample")
    ap.add_argument("--deploy-bits", type=int, choices=(2, 4), default=None,
                    help="time the deploy side instead: one decode token (batch 1) through the "
                         "224 packed linears of Llama-2-7B at this width")
    ap.add_argument("--deploy-single", action="store_true",
                    help="with --deploy-bits: one call per layer instead of grouped calls")
    ap.add_argument("--flipflop", type=int, default=None, metavar="ITERS",
                    help="time the FlipFlop Hessian factors instead: ITERS alternating "
                         "iterations from the identity on the workload's streams")
    ap.add_argument("--two-sided", action="store_true",
                    help="round with two-sided GPTQ under H_X (x) H_G instead of GPTQ")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB fp32 tensor three times (scale for the HBM byte "
                         "counters FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="only time the vendor library's dense GEMMs (torch.mm: bf16 and fp32) "
                         "as a measured achievable MFMA peak, print one JSON line and exit")
    return ap.parse_args()


def copy_calibration() -> None:
    """A plain device copy of known size: 1 GiB read + 1 GiB written per dispatch."""
    import torch
    x = torch.ones(2 ** 28, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        y = x.clone()
    torch.cuda.synchronize()
    del y
    print(json.dumps({"copy_calibration_bytes_per_dispatch": 2 ** 30, "dispatches": 3}), flush=True)


def gemm_calibration(steps: int) -> None:
    """The vendor BLAS (torch.mm, hipBLASLt / rocBLAS) on dense products of known size, timed
    with HIP events: an achievable MFMA rate on this GPU under its clock and power limits, to
    set beside the datasheet peaks.  Shapes: bf16 8192^3; bf16 A^T A for a 131072 x 4096
    stream (the full square product over the tokens, the left operand transposed into a
    contiguous copy first); fp32 8192^3."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    res = {}

    def timed(name, fn, flops):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms": round(ms, 4), "TFLOP/s": round(flops / (ms / 1e3) / 1e12, 1)}

    a = torch.randn((8192, 8192), device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev, generator=g).to(torch.bfloat16)
    timed("bf16_8192^3", lambda: torch.mm(a, b), 2.0 * 8192 ** 3)
    X = torch.randn((131072, 4096), device=dev, generator=g).to(torch.bfloat16)
    Xt = X.t().contiguous()
    timed("bf16_XtX_131072x4096", lambda: torch.mm(Xt, X), 2.0 * 4096 * 4096 * 131072)
    del X, Xt, a, b
    a = torch.randn((8192, 8192), device=dev, generator=g)
    b = torch.randn((8192, 8192), device=dev, generator=g)
    timed("fp32_8192^3", lambda: torch.mm(a, b), 2.0 * 8192 ** 3)
    print(json.dumps({"gemm_calibration": res, "steps": steps,
                      "peaks_TFLOP/s": {"bf16": PEAK_BF16_TFLOPS, "fp32": PEAK_FP32_TFLOPS}}), flush=True)


def syrk_flops(n: int, T: int) -> float:
    """Algorithmic flops of one factor: n(n+1)/2 distinct entries x 2T."""
    return float(n) * (n + 1) * T


def pipeline_lower_bound_ms(out_n: int, in_n: int, T: int, block: int, bits: int) -> dict:
    """Whole-path time at the datasheet peaks, by term (ms): both SYRKs on bf16 MFMA; the
    feedback products out in (in - B) and the factorization 2 in^3 / 3 on fp32 MFMA; one read
    and one write of W, H_X and H_G in fp32 for the rotation, plus the codes (one byte each)
    read and packed at `bits` bits, through HBM."""
    syrk = syrk_flops(in_n, T) + syrk_flops(out_n, T)
    fp32 = float(out_n) * in_n * (in_n - block) + 2.0 * float(in_n) ** 3 / 3
    hbm = 8.0 * (out_n * in_n + in_n * in_n + out_n * out_n) + out_n * in_n * (1 + bits / 8)
    return {"syrk": syrk / (PEAK_BF16_TFLOPS * 1e9),
            "factor_and_feedback": fp32 / (PEAK_FP32_TFLOPS * 1e9),
            "hbm": hbm / (PEAK_HBM_GBS * 1e6)}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_profile_name(kernel: str, workload: str) -> str:
    return f"{kernel}_{workload}_hbm_traffic.json"


def traffic_from_profile(kernel_src: str, kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, from the committed rocprofv3 counter
    summary of that kernel and workload, if it was taken on the current kernel source;
    else None."""
    p = os.path.join(ROOT, "profiles", traffic_profile_name(kernel, workload))
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != source_hash(kernel_src):
        return None
    return d.get("hbm_bytes_per_launch")


def deploy_traffic_from_profile(bits: int, call: str):
    """HBM bytes of one deploy call of the given class (matvec + output rotation kernels), from
    the committed rocprofv3 counter summary if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"deploy_w{bits}_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    src = os.path.join(ROOT, "post_quantization_syrk_amd", "csrc", "deploy.hip")
    if d.get("kernel_source_sha256_16") != source_hash(src):
        return None
    return d.get("classes", {}).get(call, {}).get("hbm_bytes_per_call")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def oracle_layer_times(cfg, budget_s: float) -> dict:
    """The fp64 CPU oracle, as it stands, on a bounded sample of one layer workload; returns
    the full-size time of each part (seconds) and what was sampled.

    Hessians on the first T_s tokens (cost linear in tokens: scaled by T / T_s); BiIP of W
    and H_X and the damped factorization at full size; H~_G's rescale and rotation at full
    size when out <= 8192, else on one stripe of 4096 rows, whose row pass stands for every
    stripe's row pass and column pass alike (x 2 out / 4096); GPTQ on R_s rows (rows are
    independent given U: scaled by out / R_s).
    """
    import oracle as o

    out_n, in_n, T = cfg.out, cfg.inp, cfg.tokens
    scale = budget_s / 20.0
    T_s = int(min(T, max(1024, 8192 * scale * (4096.0 / max(in_n, out_n)) ** 2)))
    T_s -= T_s % 64
    R_s = int(min(out_n, max(16, 256 * scale * 4096.0 / in_n)))
    t = {}
    X = o.bf16_bits_to_f64(syn.stream(cfg, "x", tokens=T_s))
    G = o.bf16_bits_to_f64(syn.stream(cfg, "g", tokens=T_s))
    t0 = time.perf_counter()
    HX = o.hessian_factor(X)
    t["hessian_x"] = (time.perf_counter() - t0) * T / T_s
    t0 = time.perf_counter()
    HG = o.hessian_factor(G)
    t["hessian_g"] = (time.perf_counter() - t0) * T / T_s
    del X, G
    W = syn.weights(cfg).astype(np.float64)
    s_in, s_out = syn.signs(cfg, "in"), syn.signs(cfg, "out")
    stripe = 4096
    full_hg = out_n <= 8192
    t0 = time.perf_counter()
    o.sensitivity(HX, HG)
    Wt, HXt, _, _, d_out = o.biip(W, HX, HG if full_hg else None, s_in, s_out, cfg.alpha,
                                  o.BIIP_FULL, cfg.had_in, cfg.had_out,
                                  hg_diag=None if full_hg else np.diag(HG))
    t["sensitivity_biip"] = time.perf_counter() - t0
    if not full_hg:
        t0 = time.perf_counter()
        part = HG[:stripe] / np.outer(d_out[:stripe], d_out)
        o.rotate_rows(part, s_out, cfg.had_out)
        t["sensitivity_biip"] += (time.perf_counter() - t0) * 2 * out_n / stripe
        del part
    del HG, W
    t0 = time.perf_counter()
    perm = o.act_order_perm(HXt) if cfg.act_order else np.arange(in_n)
    fac = o.damp_and_factor(HXt[np.ix_(perm, perm)] if cfg.act_order else HXt, cfg.damp)
    t["factor"] = time.perf_counter() - t0
    rows = np.random.default_rng(0).choice(out_n, R_s, replace=False)
    t0 = time.perf_counter()
    r = o.quantize_layer(Wt, HXt, None, cfg.bits, cfg.group, cfg.damp, rows=rows, factor=fac,
                         act_order=bool(cfg.act_order), w_clip=bool(cfg.w_clip))
    o.pack_codes(r["gptq"].codes, cfg.bits)
    t["gptq_pack"] = (time.perf_counter() - t0) * out_n / R_s
    sample = (f"Hessians on {T_s} of {T} tokens (x{T / T_s:.1f}), BiIP of W and H_X and the "
              f"factorization at full size, "
              + ("H~_G at full size" if full_hg else
                 f"H~_G's rescale and row pass on {stripe} of {out_n} rows (x{2 * out_n / stripe:.0f} "
                 f"for every stripe's row and column passes)")
              + f", GPTQ+pack on {R_s} of {out_n} rows (x{out_n / R_s:.1f})")
    return {"times_s": t, "sample": sample}


def cpu_baseline(cfg, budget_s: float) -> dict:
    """The oracle's extrapolated full-layer time on the host cores, as params/s.  Reported,
    not a target."""
    r = oracle_layer_times(cfg, budget_s)
    full = sum(r["times_s"].values())
    return {"value": round(cfg.out * cfg.inp / full, 1), "unit": "params/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": r["sample"] + f"; extrapolated full-layer time {full:.1f} s",
            "extrapolated_s": {k: round(v, 2) for k, v in r["times_s"].items()}}


# The seven linears of one Llama-2-7B decoder block (out, in) and the block count: the
# model the pages time decoding on.  32 x 7 = 224 packed layers per token.
LLAMA2_7B_LINEARS = (("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096),
                     ("o_proj", 4096, 4096), ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                     ("down_proj", 4096, 11008))
LLAMA2_7B_BLOCKS = 32
DEPLOY_GROUP = 128


def deploy_bytes(out_n: int, in_n: int, bits: int, group: int) -> int:
    """Algorithmic HBM bytes of one batch-1 deploy launch: packed codes, fp32 scales, u8 zero
    points, the fp32 rescale vectors and int8 signs of both sides, x read and y written."""
    ng = in_n // group
    return (out_n * in_n * bits // 8 + out_n * ng * 5 + (in_n + out_n) * (4 + 1)
            + in_n * 4 + out_n * 4)


def deploy_cpu_baseline(bits: int, budget_s: float) -> dict:
    """The oracle's deploy forward (dequantize from codes, rotate, multiply, rotate back) on
    the seven linears of one block; the token time is that x 32."""
    import oracle as o
    rng = np.random.default_rng(2024)
    t_total, done = 0.0, []
    for name, out_n, in_n in LLAMA2_7B_LINEARS:
        codes = rng.integers(0, 2 ** bits, size=(out_n, in_n))
        ng = in_n // DEPLOY_GROUP
        sc = rng.random((out_n, ng)) * 0.01 + 1e-3
        zr = rng.integers(0, 2 ** bits, size=(out_n, ng))
        d_in, d_out = np.exp(0.5 * rng.standard_normal(in_n)), np.exp(0.5 * rng.standard_normal(out_n))
        s_in, s_out = rng.choice([-1.0, 1.0], in_n), rng.choice([-1.0, 1.0], out_n)
        x = rng.standard_normal(in_n)
        t0 = time.perf_counter()
        Q = o.dequant(codes, sc, zr, DEPLOY_GROUP)
        o.deploy_linear(Q, d_in, d_out, s_in, s_out, o.hadamard_block_size(in_n, 0),
                        o.hadamard_block_size(out_n, 0), x)
        t_total += time.perf_counter() - t0
        done.append(name)
        if t_total > budget_s:
            break
    per_block = t_total * len(LLAMA2_7B_LINEARS) / len(done)
    token_s = per_block * LLAMA2_7B_BLOCKS
    return {"value": round(1.0 / token_s, 4), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"{', '.join(done)} of one block (dequantize from codes + rotated fp64 "
                       f"matvec), x{LLAMA2_7B_BLOCKS * len(LLAMA2_7B_LINEARS) / len(done):.0f} "
                       f"to a token; {token_s:.1f} s per token"),
            "measured_s": round(t_total, 2)}


def deploy_main(a) -> None:
    """One decode token at batch 1 through all 224 quantized linears of Llama-2-7B: each layer
    its own packed codes, scales, zero points, rescale vectors and signs (nothing stays in
    cache from one layer to the next), the Hadamard blocks BiIP picks by default (4096 on
    the 4096 sides, 256 on the 11008 sides).  Calls follow a decoder's dependencies: the
    layers that read the same activation go in one grouped call (q/k/v, then o, then
    gate/up, then down: 128 calls), or one call per layer with --deploy-single.  The token is
    captured in one HIP graph and replayed; the roofline is the HBM bound of the call class
    with the most time."""
    import torch
    import post_quantization_syrk_amd as kq
    bits, group = a.deploy_bits, DEPLOY_GROUP
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kq.load_library()
    g = torch.Generator(device=dev)
    g.manual_seed(20240 + bits)
    t0 = time.time()
    blocks = []
    for blk in range(LLAMA2_7B_BLOCKS):
        lay = {}
        for name, out_n, in_n in LLAMA2_7B_LINEARS:
            ng = in_n // group
            lay[name] = dict(
                packed=torch.randint(0, 256, (out_n, in_n * bits // 8), dtype=torch.uint8, device=dev,
                                     generator=g).view(torch.int32),
                scales=torch.rand((out_n, ng), device=dev, generator=g) * 0.01 + 1e-3,
                zeros=torch.randint(0, 2 ** bits, (out_n, ng), dtype=torch.uint8, device=dev, generator=g),
                bits=bits, group=group,
                d_in=torch.exp(0.5 * torch.randn(in_n, device=dev, generator=g)),
                d_out=torch.exp(0.5 * torch.randn(out_n, device=dev, generator=g)),
                sign_in=torch.randint(0, 2, (in_n,), dtype=torch.int8, device=dev, generator=g) * 2 - 1,
                sign_out=torch.randint(0, 2, (out_n,), dtype=torch.int8, device=dev, generator=g) * 2 - 1,
                had_in=0, had_out=0, y=torch.empty(out_n, device=dev))
        blocks.append(lay)
    xs = {n: torch.randn(n, device=dev, generator=g) for n in (4096, 11008)}
    shape = {name: (o_, i_) for name, o_, i_ in LLAMA2_7B_LINEARS}
    groups = ([["q_proj"], ["k_proj"], ["v_proj"], ["o_proj"], ["gate_proj"], ["up_proj"], ["down_proj"]]
              if a.deploy_single else
              [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]])
    calls = [("+".join(gr), [blk[nm] for nm in gr], shape[gr[0]][1]) for blk in blocks for gr in groups]
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    def token(stream, events=None):
        for i, (_, lays, in_n) in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            if len(lays) == 1:
                L = lays[0]
                kq.kq_deploy_linear(L["packed"], L["scales"], L["zeros"], bits, group, L["d_in"],
                                    L["d_out"], L["sign_in"], L["sign_out"], 0, 0, xs[in_n], L["y"],
                                    stream=stream)
            else:
                kq.kq_deploy_linear_group(lays, xs[in_n], stream=stream)
            if events is not None:
                events[i][1].record(stream)

    # eager token with an event pair around every call: per-call kernel durations
    stream = torch.cuda.current_stream()
    token(stream)
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in calls]
    token(stream, events)
    torch.cuda.synchronize()
    outs = [L["y"] for _, lays, _ in calls for L in lays]
    eager_y = [y.clone() for y in outs]
    per = {}
    for (name, lays, in_n), (e0, e1) in zip(calls, events):
        per.setdefault(name, []).append(e0.elapsed_time(e1))

    # the token as one HIP graph; replays must give the eager outputs bit for bit
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        token(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        token(side)
    for _ in range(a.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(a.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_token = wall * 1e3 / a.steps
    for y, ye in zip(outs, eager_y):
        if not torch.equal(y, ye):
            raise RuntimeError("graph replay differs from the eager calls")

    tot_bytes = sum(deploy_bytes(o_, i_, bits, group) for _, o_, i_ in LLAMA2_7B_LINEARS) * LLAMA2_7B_BLOCKS
    classes = {}
    for name, ts in per.items():
        avg = float(np.mean(ts))
        b = sum(deploy_bytes(*shape[nm], bits, group) for nm in name.split("+"))
        classes[name] = {"calls": len(ts), "avg_us": round(avg * 1e3, 2),
                         "GB/s": round(b / (avg / 1e3) / 1e9, 1), "bytes": b}
    dom = max(classes.items(), key=lambda kv: kv[1]["calls"] * kv[1]["avg_us"])
    kernel_sum_ms = sum(c["calls"] * c["avg_us"] for c in classes.values()) / 1e3
    roofline = {"bound": "hbm", "achieved": dom[1]["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(dom[1]["GB/s"] / PEAK_HBM_GBS, 4),
                "traffic": deploy_traffic_from_profile(bits, dom[0]),
                "kernel": f"deploy_matvec_kernel + deploy_outrot_kernel: one {dom[0]} call",
                "algorithmic_bytes_per_launch": dom[1]["bytes"]}
    cpu = None if a.no_cpu_baseline else deploy_cpu_baseline(bits, a.cpu_seconds)
    line = {
        "metric": "decode tokens/s through the quantized linears (batch 1)",
        "value": round(1e3 / ms_per_token, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_token, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"u{bits} codes / f32 activations and accumulate",
        "data": "synthetic (seeded random codes, scales, zero points, rescale vectors, signs)",
        "config": {"workload": f"llama2-7b-decode-linears-W{bits}-g{group}",
                   "layers": len(LLAMA2_7B_LINEARS) * LLAMA2_7B_BLOCKS, "calls": len(calls),
                   "grouped": not a.deploy_single, "bits": bits, "group": group,
                   "hadamard": "4096 / 256 (default blocks)", "graph": True},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_bytes_per_token": tot_bytes,
        "token_GB/s": round(tot_bytes / (ms_per_token / 1e3) / 1e9, 1),
        "kernel_sum_ms_eager": round(kernel_sum_ms, 4),
        "classes": classes,
        "input_generation_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def flipflop_cpu_baseline(cfg, iters: int, budget_s: float) -> dict:
    """The oracle's FlipFlop iteration on token samples of the same streams; its cost is
    a + b T (inverses, then products linear in the tokens), fitted on two samples and
    evaluated at the workload's T."""
    import oracle as o
    Xb, Gb = syn.flipflop_streams(cfg, tokens=4096)
    times = []
    for Ts in (2048, 4096):
        X = syn.bf16_bits_to_f32(Xb[:Ts]).astype(np.float64)
        G = syn.bf16_bits_to_f32(Gb[:Ts]).astype(np.float64)
        t0 = time.perf_counter()
        o.flipflop(X, G, 1)
        times.append(time.perf_counter() - t0)
    b = (times[1] - times[0]) / 2048.0
    a0 = max(times[0] - b * 2048, 0.0)
    per_iter = a0 + b * cfg.tokens
    return {"value": round(1.0 / per_iter, 5), "unit": "iterations/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"one iteration on 2048 and 4096 tokens ({times[0]:.1f} s, {times[1]:.1f} s), "
                       f"fitted a + b T and evaluated at T = {cfg.tokens}: {per_iter:.0f} s per iteration")}


def flipflop_main(a) -> None:
    """FlipFlop Hessian factors (kq_flipflop) on the workload's streams with correlated
    per-token magnitudes: one step = a.flipflop iterations from the identity.  The
    roofline is the per-token quadratic-form kernel (bf16 MFMA), its HIP-event time per
    launch from the call's phase timer."""
    import torch
    import post_quantization_syrk_amd as kq
    cfg = WORKLOADS[a.workload]
    iters = a.flipflop
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kq.load_library()
    t0 = time.time()
    Xb, Gb = syn.flipflop_streams(cfg)
    X = torch.from_numpy(Xb.view(np.int16)).to(dev)
    G = torch.from_numpy(Gb.view(np.int16)).to(dev)
    del Xb, Gb
    gen_s = time.time() - t0
    T, n, m = cfg.tokens, cfg.inp, cfg.out
    A = torch.empty((n, n), device=dev)
    B = torch.empty((m, m), device=dev)
    ws = torch.empty(kq.kq_flipflop_workspace(T, n, m), dtype=torch.uint8, device=dev)
    for _ in range(a.warmup):
        kq.kq_flipflop(X, G, iters, A, B, ws)
    torch.cuda.synchronize()
    phases = {"factor": 0.0, "quadratic_forms": 0.0, "scale": 0.0, "syrk": 0.0}
    t_start = time.perf_counter()
    for _ in range(a.steps):
        ph = kq.kq_flipflop(X, G, iters, A, B, ws, phases=True)
        for k_, v in ph.items():
            phases[k_] += v
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / a.steps
    launches = 2 * iters * a.steps           # quadratic-form launches (one per half step)
    qf_ms = phases["quadratic_forms"] / launches
    # algorithmic flops of one launch: T k (k + 1) (only U's upper triangle), averaged over
    # the two half steps (k = m, then n)
    flops = 0.5 * (T * m * (m + 1) + T * n * (n + 1))
    achieved = flops / (qf_ms / 1e3) / 1e12
    cpu = None if a.no_cpu_baseline else flipflop_cpu_baseline(cfg, iters, a.cpu_seconds)
    line = {
        "metric": "FlipFlop Hessian iterations per second (both factors, from the identity)",
        "value": round(iters / (ms_per_step / 1e3), 3), "unit": "iterations/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 products / f32 accumulate",
        "data": "synthetic (seeded log-normal-channel streams with correlated per-token magnitudes)",
        "config": {"workload": cfg.name + "-flipflop", "in": n, "out": m, "tokens": T,
                   "iterations_per_step": iters},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(
                         os.path.join(ROOT, "post_quantization_syrk_amd", "csrc", "flipflop.hip"),
                         "qform_kernel", a.workload),
                     "kernel": "qform_kernel", "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu,
        "phases_ms_per_iteration": {k_: round(v / (iters * a.steps), 3) for k_, v in phases.items()},
        "input_generation_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def two_sided_cpu_baseline(cfg) -> dict:
    """The oracle's two-sided rounding on the layer's leading 128 x 128 block (a problem of
    its own), scaled by the work count sum_{r, i} (m - r)(n - i) of the full layer; the
    Hessian and BiIP legs of the step are not added (they are the GPTQ baseline's)."""
    import oracle as o
    b = 128
    rng = np.random.default_rng(0)
    W = rng.standard_normal((b, b)) * 0.02
    A = rng.standard_normal((3 * b, b))
    B = rng.standard_normal((3 * b, b))
    t0 = time.perf_counter()
    o.two_sided_gptq(W, A.T @ A, B.T @ B, cfg.bits, min(cfg.group, b))
    t = time.perf_counter() - t0
    work = lambda m, n: (m * (m + 1) / 2) * (n * (n + 1) / 2)  # noqa: E731
    full = t * work(cfg.out, cfg.inp) / work(b, b)
    return {"value": round(cfg.out * cfg.inp / full, 3), "unit": "params/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"two-sided rounding of a {b} x {b} block in {t:.1f} s, scaled by the "
                       f"O(m^2 n^2) work count to {cfg.out} x {cfg.inp}: {full:.3g} s")}


def stack_work(bits_of) -> dict:
    """Algorithmic work of one pass over the decoder stack: SYRK flops (each distinct stream's
    factor once: per layer 4 activation and 7 gradient factors), fp32 flops (feedback
    products and factorizations per sublayer) and HBM bytes (rotation and packing per
    sublayer).  bits_of(layer, k) gives sublayer k's width."""
    T = syn.STACK_TOKENS
    syrk = fp32 = hbm = 0.0
    for layer in range(syn.STACK_LAYERS):
        seen = set()
        for k, (_, out_n, in_n, xs, _, _) in enumerate(syn.LLAMA2_7B_SUBLAYERS):
            if xs not in seen:
                seen.add(xs)
                syrk += syrk_flops(in_n, T)
            syrk += syrk_flops(out_n, T)
            fp32 += float(out_n) * in_n * (in_n - 128) + 2.0 * float(in_n) ** 3 / 3
            hbm += (8.0 * (out_n * in_n + in_n * in_n + out_n * out_n)
                    + out_n * in_n * (1 + bits_of(layer, k) / 8))
    return {"syrk_flops": syrk, "fp32_flops": fp32, "hbm_bytes": hbm}


def stack_cpu_baseline(budget_s: float) -> dict:
    """The oracle on samples of the stack's three sublayer shapes (4096 x 4096, 11008 x 4096,
    4096 x 11008 at 32768 tokens), each as oracle_layer_times, combined with the stack's
    counts: per layer 3 + 1 activation factors (4096 / 11008 wide), 5 + 2 gradient factors
    (4096 / 11008 wide), and BiIP, factorization and GPTQ for 4 + 2 + 1 sublayers; x 32."""
    cfgs = syn.stack_sublayer_configs(0)
    shape = {"sq": cfgs[0], "wide_out": cfgs[4], "wide_in": cfgs[6]}
    r = {k: oracle_layer_times(c, budget_s / 3.0) for k, c in shape.items()}
    rest = lambda k: sum(v for n, v in r[k]["times_s"].items() if not n.startswith("hessian"))  # noqa: E731
    per_layer = (3 * r["sq"]["times_s"]["hessian_x"] + r["wide_in"]["times_s"]["hessian_x"]
                 + 5 * r["sq"]["times_s"]["hessian_g"] + 2 * r["wide_out"]["times_s"]["hessian_g"]
                 + 4 * rest("sq") + 2 * rest("wide_out") + rest("wide_in"))
    full = per_layer * syn.STACK_LAYERS
    params = syn.STACK_LAYERS * sum(o_ * i_ for _, o_, i_, _, _, _ in syn.LLAMA2_7B_SUBLAYERS)
    return {"value": round(params / full, 1), "unit": "params/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": ("the three sublayer shapes of layer 0, each: " + r["sq"]["sample"]
                       + f"; combined per layer and x{syn.STACK_LAYERS}: extrapolated stack time "
                       f"{full:.0f} s (allocation not counted)"),
            "extrapolated_s_per_layer": round(per_layer, 2)}


def stack_main(a) -> None:
    """The decoder stack: 32 Llama-2-7B layers x 7 linears (q, k, v, o 4096 x 4096; gate, up
    11008 x 4096; down 4096 x 11008), 32768 calibration tokens per layer, bits in {2, 3, 4}
    allocated from tr(H_G) tr(H_X) to 2.5 bits per weight on average.

    One step, inputs resident in HBM (every layer's 4 activation streams, q/k/v and gate/up
    sharing theirs, 7 gradient streams and 7 weight matrices):
      pass 1: per layer, H_X of each distinct activation stream and H_G of each sublayer
              (kq_accumulate_hessian), the 224 sensitivities (kq_sensitivity_async);
      bits:   one synchronization, the sensitivities to the host, kq_allocate_bits;
      pass 2: per sublayer, BiIP out of place from the raw factors (q/k/v and gate/up share
              H_X) and GPTQ to packed codes at the allocated width (kq_quantize_layer_async),
              the sublayers dealt round-robin to --stack-streams streams with a workspace each,
              so that one sublayer's latency-bound factorization chain overlaps others' work;
              every status is checked after the timed steps.
    The streams are drawn on the device (torch's generator, seeded per layer and stream) with
    the stack's recipe: per-channel std exp(sigma N(0, 1)), sigma per layer in U[0.5, 2] as
    the parity tests' generator gives it, N(0, 1) entries, rounded to bf16; weights
    N(0, 0.02^2) rounded to bf16.  Drawing 138 GB on the host would dominate the run."""
    import torch
    import post_quantization_syrk_amd as kq
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kq.load_library()
    stream = torch.cuda.current_stream()
    T, L = syn.STACK_TOKENS, syn.STACK_LAYERS
    subl = syn.LLAMA2_7B_SUBLAYERS
    gen = torch.Generator(device=dev)

    def draw(seed, rows, n, sigma):
        gen.manual_seed(seed)
        sc = torch.exp(sigma * torch.randn(n, device=dev, generator=gen))
        out = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
        for r0 in range(0, rows, 8192):
            r1 = min(rows, r0 + 8192)
            out[r0:r1] = (torch.randn((r1 - r0, n), device=dev, generator=gen) * sc).to(torch.bfloat16)
        return out

    t0 = time.time()
    layers = []
    for layer in range(L):
        sx, sg = syn.stack_layer_sigmas(layer)
        base = 1_000_003 * (layer + 1)
        xs, hx = {}, {}
        for _, _, in_n, xid, _, _ in subl:
            if xid not in xs:
                xs[xid] = draw(base + xid, T, in_n, sx)
                hx[xid] = torch.empty((in_n, in_n), device=dev)
        subs = []
        for k, (_, out_n, in_n, xid, hin, hout) in enumerate(subl):
            gen.manual_seed(base + 100 + k)
            W = (torch.randn((out_n, in_n), device=dev, generator=gen) * 0.02).to(torch.bfloat16).float()
            subs.append(dict(
                G=draw(base + 10 + k, T, out_n, sg), HG=torch.empty((out_n, out_n), device=dev), W=W,
                s_in=(torch.randint(0, 2, (in_n,), device=dev, generator=gen, dtype=torch.int8) * 2 - 1),
                s_out=(torch.randint(0, 2, (out_n,), device=dev, generator=gen, dtype=torch.int8) * 2 - 1),
                packed=torch.empty(out_n * in_n * 4 // 32, dtype=torch.int32, device=dev),
                scales=torch.empty((out_n, in_n // 128), device=dev),
                zeros=torch.empty((out_n, in_n // 128), dtype=torch.uint8, device=dev),
                out=out_n, inp=in_n, xid=xid, hin=hin, hout=hout))
        layers.append((xs, hx, subs))
    nmax = max(max(o_, i_) for _, o_, i_, _, _, _ in subl)
    params = {b: kq.make_params(b, 128, 128, 0.01) for b in (2, 3, 4)}
    ws_bytes = max(kq.kq_quantize_layer_workspace(params[b], o_, i_, False)
                   for b in (2, 3, 4) for _, o_, i_, _, _, _ in subl)
    # per pass-2 stream: processed factors, weights, rescale vectors and a workspace
    lanes = [dict(stream=torch.cuda.Stream(), HXt=torch.empty(nmax * nmax, device=dev),
                  HGt=torch.empty(nmax * nmax, device=dev),
                  Wt=torch.empty(max(o_ * i_ for _, o_, i_, _, _, _ in subl), device=dev),
                  d_in=torch.empty(nmax, device=dev), d_out=torch.empty(nmax, device=dev),
                  ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev))
             for _ in range(a.stack_streams)]
    status = torch.full((L * len(subl),), -1, dtype=torch.int32, device=dev)
    sens = torch.empty((L * len(subl), 3), dtype=torch.float64, device=dev)
    numel = [o_ * i_ for _ in range(L) for _, o_, i_, _, _, _ in subl]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(record):
        syrk_ev = []
        e = [ev() for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        i = 0
        for xs, hx, subs in layers:
            for xid, X in xs.items():
                if record:
                    syrk_ev.append((ev(), ev()))
                    syrk_ev[-1][0].record(stream)
                kq.kq_accumulate_hessian(X, hx[xid], stream=stream)
                if record:
                    syrk_ev[-1][1].record(stream)
            for sb in subs:
                if record:
                    syrk_ev.append((ev(), ev()))
                    syrk_ev[-1][0].record(stream)
                kq.kq_accumulate_hessian(sb["G"], sb["HG"], stream=stream)
                if record:
                    syrk_ev[-1][1].record(stream)
                kq.kq_sensitivity_async(hx[sb["xid"]], sb["HG"], sens[i], stream=stream)
                i += 1
        if record:
            e[1].record(stream)
        s_host = sens[:, 2].cpu().numpy()          # synchronizes the stream
        bits = kq.kq_allocate_bits(list(s_host), numel, (2, 3, 4), 5, 2)
        if record:
            e[2].record(stream)
        # pass 2 on the lanes' streams, after everything above on the main stream
        for ln in lanes:
            ln["stream"].wait_stream(stream)
        i = 0
        for xs, hx, subs in layers:
            for sb in subs:
                ln = lanes[i % len(lanes)]
                st = ln["stream"]
                o_, i_ = sb["out"], sb["inp"]
                hxt, hgt = ln["HXt"][:i_ * i_].view(i_, i_), ln["HGt"][:o_ * o_].view(o_, o_)
                wt = ln["Wt"][:o_ * i_].view(o_, i_)
                kq.kq_biip_rotate(sb["W"], wt, hx[sb["xid"]], hxt, sb["HG"], hgt, sb["s_in"],
                                  sb["s_out"], ln["d_in"][:i_], ln["d_out"][:o_], 0.25,
                                  kq.KQ_BIIP_FULL, sb["hin"], sb["hout"], stream=st)
                b = bits[i]
                packed = sb["packed"][:o_ * i_ * b // 32].view(o_, i_ * b // 32)
                kq.kq_quantize_layer_async(params[b], wt, hxt, hgt, packed, sb["scales"], sb["zeros"],
                                           ln["ws"], status[i:i + 1], stream=st)
                i += 1
        # the next step's pass 1 overwrites the raw factors pass 2 reads
        for ln in lanes:
            stream.wait_stream(ln["stream"])
        if record:
            e[3].record(stream)
        return e, syrk_ev, bits

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    recs = []
    t_start = time.perf_counter()
    for _ in range(a.steps):
        recs.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / a.steps
    bad = int((status != kq.KQ_OK).sum().item())
    if bad:
        raise RuntimeError(f"{bad} sublayers did not quantize (status != KQ_OK)")
    total_params = float(sum(numel))
    stages = {nm: float(np.mean([r[0][i].elapsed_time(r[0][i + 1]) for r in recs]))
              for i, nm in enumerate(["pass1_hessians_sensitivities", "allocation", "pass2_biip_quantize"])}
    syrk_ms = [s0.elapsed_time(s1) for r in recs for s0, s1 in r[1]]
    bits = recs[-1][2]
    work = stack_work(lambda layer, k: bits[layer * len(subl) + k])
    n_syrk = len(syrk_ms) / a.steps
    flops_per_launch = work["syrk_flops"] / n_syrk
    achieved = flops_per_launch / (float(np.mean(syrk_ms)) / 1e3) / 1e12
    lb = {"syrk": work["syrk_flops"] / (PEAK_BF16_TFLOPS * 1e9),
          "factor_and_feedback": work["fp32_flops"] / (PEAK_FP32_TFLOPS * 1e9),
          "hbm": work["hbm_bytes"] / (PEAK_HBM_GBS * 1e6)}
    lb_ms = sum(lb.values())
    cpu = None if a.no_cpu_baseline else stack_cpu_baseline(a.cpu_seconds)
    line = {
        "metric": "quantized params/s per layer incl. Hessian build",
        "value": round(total_params / (ms_per_step / 1e3), 1), "unit": "params/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 products / f32 accumulate and quantizer",
        "data": "synthetic (log-normal-channel streams drawn on the device per layer, Llama-shaped)",
        "config": {"workload": "llama2-7b-decoder-stack-32x7-T32768-mixed-2.5bit", "layers": L,
                   "sublayers": L * len(subl), "tokens": T, "params": int(total_params),
                   "bits_allowed": [2, 3, 4], "avg_bits_target": 2.5,
                   "avg_bits": round(sum(b * n for b, n in zip(bits, numel)) / total_params, 4),
                   "bits_count": {str(b): bits.count(b) for b in (2, 3, 4)},
                   "group": 128, "block": 128, "alpha": 0.25, "damp": 0.01,
                   "pass2_streams": a.stack_streams},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(
                         os.path.join(ROOT, "post_quantization_syrk_amd", "csrc", "syrk.hip"),
                         "syrk_dma_kernel", STACK),
                     "kernel": "syrk_dma_kernel",
                     "algorithmic_flops_per_launch": flops_per_launch,
                     "launches_per_step": int(n_syrk)},
        "cpu_baseline": cpu,
        "pipeline_roofline": {"lower_bound_ms": round(lb_ms, 3), "frac": round(lb_ms / ms_per_step, 4),
                              "terms_ms": {k: round(v, 3) for k, v in lb.items()}},
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "syrk_ms_per_step": round(sum(syrk_ms) / a.steps, 3),
        "input_generation_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {a.gpus} is not supported "
              "(the multi-GPU sharding plan is described in the design notes)", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gemm_calibration:
        gemm_calibration(a.steps)
        return
    if a.workload is None:
        a.workload = "c2" if (a.flipflop is not None or a.two_sided) else DEFAULT_WORKLOAD
    if a.workload == STACK:
        if a.flipflop is not None or a.two_sided or a.deploy_bits is not None:
            print("bench.py: --workload c4 times the GPTQ path of the decoder stack only",
                  file=sys.stderr)
            sys.exit(2)
        stack_main(a)
        return
    if a.deploy_bits is not None:
        deploy_main(a)
        return
    if a.flipflop is not None:
        flipflop_main(a)
        return
    import torch
    import post_quantization_syrk_amd as kq

    cfg = WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kq.load_library()
    stream = torch.cuda.current_stream()

    # ---- inputs (untimed): seeded synthetic streams and weights, uploaded once ----
    t0 = time.time()
    bx = syn.stream(cfg, "x")
    X = torch.from_numpy(bx.view(np.int16)).to(dev).view(torch.bfloat16)
    del bx
    bg = syn.stream(cfg, "g")
    G = torch.from_numpy(bg.view(np.int16)).to(dev).view(torch.bfloat16)
    del bg
    W0 = torch.from_numpy(syn.weights(cfg)).to(dev)
    s_in = torch.from_numpy(syn.signs(cfg, "in")).to(dev)
    s_out = torch.from_numpy(syn.signs(cfg, "out")).to(dev)
    gen_s = time.time() - t0

    out_n, in_n, T = cfg.out, cfg.inp, cfg.tokens
    HX = torch.empty((in_n, in_n), device=dev)
    HG = torch.empty((out_n, out_n), device=dev)
    Wt = torch.empty_like(W0)
    d_in = torch.empty(in_n, device=dev)
    d_out = torch.empty(out_n, device=dev)
    p = kq.make_params(cfg.bits, cfg.group, cfg.block, cfg.damp, act_order=cfg.act_order,
                       w_clip=cfg.w_clip)
    if a.two_sided:
        ws = torch.empty(kq.kq_quantize_two_sided_workspace(p, out_n, in_n), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(kq.kq_quantize_layer_workspace(p, out_n, in_n, False), dtype=torch.uint8, device=dev)
    packed = torch.empty((out_n, in_n * cfg.bits // 32), dtype=torch.int32, device=dev)
    scales = torch.empty((out_n, in_n // cfg.group), device=dev)
    zeros = torch.empty((out_n, in_n // cfg.group), dtype=torch.uint8, device=dev)

    sens_dev = torch.empty(3, dtype=torch.float64, device=dev)   # tr H_X, tr H_G, product
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stage_names = ["syrk_x", "syrk_g", "sensitivity", "biip", "quantize"]

    def step(record):
        e = [ev() for _ in range(6)] if record else None
        if record:
            e[0].record(stream)
        kq.kq_accumulate_hessian(X, HX, stream=stream)
        if record:
            e[1].record(stream)
        kq.kq_accumulate_hessian(G, HG, stream=stream)
        if record:
            e[2].record(stream)
        kq.kq_sensitivity_async(HX, HG, sens_dev, stream=stream)
        if record:
            e[3].record(stream)
        kq.kq_biip_rotate(W0, Wt, HX, HX, HG, HG, s_in, s_out, d_in, d_out, cfg.alpha,
                          kq.KQ_BIIP_FULL, cfg.had_in, cfg.had_out, stream=stream)
        if record:
            e[4].record(stream)
        if a.two_sided:
            kq.kq_quantize_two_sided(p, Wt, HX, HG, packed, scales, zeros, ws, stream=stream)
        else:
            kq.kq_quantize_layer(p, Wt, HX, HG, packed, scales, zeros, ws, stream=stream)
        if record:
            e[5].record(stream)
        return e

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    events = []
    t_start = time.perf_counter()
    for _ in range(a.steps):
        events.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / a.steps
    stage_ms = {nm: float(np.mean([es[i].elapsed_time(es[i + 1]) for es in events]))
                for i, nm in enumerate(stage_names)}
    params = out_n * in_n
    value = params / (ms_per_step / 1e3)

    # dominant kernel: the SYRK (one launch per factor); HIP events on its stream
    syrk_launch_ms = float(np.mean([es[0].elapsed_time(es[1]) for es in events] +
                                   [es[1].elapsed_time(es[2]) for es in events]))
    flops_per_launch = 0.5 * (syrk_flops(in_n, T) + syrk_flops(out_n, T))
    achieved = flops_per_launch / (syrk_launch_ms / 1e3) / 1e12
    traffic = traffic_from_profile(os.path.join(ROOT, "post_quantization_syrk_amd", "csrc", "syrk.hip"),
                                   "syrk_dma_kernel", a.workload)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "syrk_dma_kernel",
                "algorithmic_flops_per_launch": flops_per_launch}
    if a.two_sided:
        # the rounding wavefront dominates: its pulls and pushes are m n (m + n) / 2 fp32 MACs
        ts_ms = stage_ms["quantize"]
        ts_flops = float(out_n) * in_n * (out_n + in_n)
        ts_ach = ts_flops / (ts_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ts_ach, 2), "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ts_ach / PEAK_FP32_TFLOPS, 4), "traffic": None,
                    "kernel": "two-sided rounding (pull / round / push wavefront, with its factors)",
                    "algorithmic_flops_per_launch": ts_flops}

    pipeline = None
    if not a.two_sided:
        lb = pipeline_lower_bound_ms(out_n, in_n, T, cfg.block, cfg.bits)
        lb_ms = sum(lb.values())
        pipeline = {"lower_bound_ms": round(lb_ms, 4), "frac": round(lb_ms / ms_per_step, 4),
                    "terms_ms": {k: round(v, 4) for k, v in lb.items()}}

    cpu = None
    if not a.no_cpu_baseline:
        del X, G
        torch.cuda.empty_cache()
        cpu = two_sided_cpu_baseline(cfg) if a.two_sided else cpu_baseline(cfg, a.cpu_seconds)

    line = {
        "metric": "quantized params/s per layer incl. Hessian build",
        "value": round(value, 1), "unit": "params/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 products / f32 accumulate and quantizer",
        "data": "synthetic (seeded log-normal-channel streams, Llama-shaped)",
        "config": {"workload": cfg.name, "out": out_n, "in": in_n, "tokens": T, "bits": cfg.bits,
                   "group": cfg.group, "block": cfg.block, "hadamard_in": cfg.had_in,
                   "hadamard_out": cfg.had_out, "alpha": cfg.alpha, "damp": cfg.damp,
                   "act_order": cfg.act_order, "w_clip": cfg.w_clip,
                   "rounding": "two-sided" if a.two_sided else "gptq"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pipeline_roofline": pipeline,
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "input_generation_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
