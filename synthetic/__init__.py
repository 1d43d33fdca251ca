"""Seeded synthetic inputs for the KronQ per-layer quantization engine.

This module only draws numbers: calibration activation streams X (tokens x in),
output-gradient streams G (tokens x out), weights W (out x in) and the random
+-1 sign vectors of the randomized Hadamard rotation.  It holds none of the
method's arithmetic; the GPU path and the CPU oracle both consume what it
returns, and neither is imported here.

Workloads stand in for the pages' calibration data (the KronQ README's
"Reproduce from scratch" section calibrates Llama-2/Llama-3 linears on real
activations and backpropagated gradients with 128 samples).  Real weights and
datasets are not used: every tensor is synthetic, with Llama-shaped sizes and
log-normal per-channel scales.

Generator recipe (one per tensor and token chunk, so chunks can be drawn in
parallel and reproducibly):
  numpy.random.default_rng(SeedSequence([seed, cfg_index, tensor_id, layer, chunk]))
  per-channel std  s_i = exp(sigma * N(0,1))         (drawn once per tensor)
  stream chunk     N(0,1) * s  (fp32), rounded to bf16 (round-to-nearest-even)
  weights          N(0, w_std^2) or w_std * Student-t(4), outlier input
                   columns multiplied by a constant, rounded to bf16 unless
                   the config keeps fp32 weights
  signs            int8 +-1, uniform
  token magnitudes (streams for the FlipFlop factors) a_t = exp(0.5 z_t) on X's
                   rows and b_t = exp(0.5 (0.8 z_t + 0.6 u_t)) on G's rows, z, u
                   N(0,1): correlated per-token sizes, so E[(g^T B^-1 g) x x^T]
                   differs from the marginal factor
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# tensor ids inside the seed sequence
_TID_W, _TID_X, _TID_G, _TID_SIN, _TID_SOUT, _TID_SCALE_X, _TID_SCALE_G, _TID_OUTL = range(8)
_TID_LAYER_SIGMA = 8
_TID_TOKMAG = 9

CHUNK_TOKENS = 8192


@dataclass(frozen=True)
class LayerConfig:
    """One linear layer's workload: shapes, input recipe and quantizer knobs."""
    name: str
    cfg_index: int
    out: int
    inp: int
    tokens: int
    w_dtype: str = "bf16"          # "bf16" or "fp32" (storage of the original weights)
    w_dist: str = "normal"         # "normal" or "student_t4"
    w_std: float = 0.02
    n_outliers: int = 0            # input columns scaled by outlier_scale
    outlier_scale: float = 1.0
    sigma_x: float = 1.0
    sigma_g: float = 1.5
    bits: int = 2
    group: int = 128
    block: int = 128
    had_in: int = 0                # Hadamard block size; 0 = largest power-of-2 divisor
    had_out: int = 0
    damp: float = 0.01
    alpha: float = 0.25
    act_order: int = 0             # quantizer options (group must then equal inp)
    w_clip: int = 0
    seed: int = 0
    layer: int = 0
    # streams shared between sublayers (c4): ids of the X and G streams
    x_stream: int = 0
    g_stream: int = 0

    @property
    def params(self) -> int:
        return self.out * self.inp

    def scaled(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


def largest_pow2_divisor(n: int) -> int:
    return n & (-n)


# ---------------------------------------------------------------------------
# Workload registry.  Sizes are those of Llama-2-7B / Llama-3-70B linears.
# ---------------------------------------------------------------------------
C1 = LayerConfig(name="single-256x256-T2048-W2", cfg_index=1, out=256, inp=256, tokens=2048,
                 w_dtype="fp32", w_std=0.02, n_outliers=4, outlier_scale=20.0,
                 sigma_x=1.0, sigma_g=1.5, bits=2, group=64, block=64,
                 had_in=256, had_out=256)
C2 = LayerConfig(name="llama2-7b-q_proj-4096x4096-T131072-W4", cfg_index=2, out=4096, inp=4096,
                 tokens=131072, w_std=0.02, n_outliers=4, outlier_scale=30.0,
                 sigma_x=1.0, sigma_g=1.5, bits=4, group=128, block=128,
                 had_in=4096, had_out=4096)
C3 = LayerConfig(name="llama2-7b-down_proj-4096x11008-T131072-W2", cfg_index=3, out=4096, inp=11008,
                 tokens=131072, w_dist="student_t4", w_std=0.015, sigma_x=1.0, sigma_g=1.5,
                 bits=2, group=128, block=128, had_in=256, had_out=4096)
C5 = LayerConfig(name="llama3-70b-up_proj-28672x8192-T262144-W2", cfg_index=5, out=28672, inp=8192,
                 tokens=262144, w_std=0.01, n_outliers=8, outlier_scale=30.0,
                 sigma_x=1.0, sigma_g=1.5, bits=2, group=128, block=128,
                 had_in=8192, had_out=4096)

# c2 with the base recipe's quantizer options (--w_groupsize -1 --w_clip --act_order)
C2R = C2.scaled(name="llama2-7b-q_proj-4096x4096-T131072-W4-rowgrid-clip-actorder", group=4096,
                act_order=1, w_clip=1)

CONFIGS = {"c1": C1, "c2": C2, "c2r": C2R, "c3": C3, "c5": C5}

# Decoder-stack workload (32 Llama-2-7B layers, 7 linears each, 32768 tokens).
LLAMA2_7B_SUBLAYERS = (
    # name, out, in, x stream id (within the layer), hadamard in, hadamard out
    ("q", 4096, 4096, 0, 4096, 4096),
    ("k", 4096, 4096, 0, 4096, 4096),
    ("v", 4096, 4096, 0, 4096, 4096),
    ("o", 4096, 4096, 1, 4096, 4096),
    ("gate", 11008, 4096, 2, 4096, 256),
    ("up", 11008, 4096, 2, 4096, 256),
    ("down", 4096, 11008, 3, 256, 4096),
)
STACK_LAYERS = 32
STACK_TOKENS = 32768


def stack_layer_sigmas(layer: int, seed: int = 0) -> tuple[float, float]:
    """Per-layer log-normal sigma for the X and G streams, uniform in [0.5, 2]."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4, _TID_LAYER_SIGMA, layer, 0]))
    sx, sg = rng.uniform(0.5, 2.0, size=2)
    return float(sx), float(sg)


def stack_sublayer_configs(layer: int, seed: int = 0, tokens: int = STACK_TOKENS) -> list[LayerConfig]:
    sx, sg = stack_layer_sigmas(layer, seed)
    cfgs = []
    for k, (nm, out, inp, xs, hin, hout) in enumerate(LLAMA2_7B_SUBLAYERS):
        cfgs.append(LayerConfig(
            name=f"llama2-7b-L{layer}-{nm}", cfg_index=4, out=out, inp=inp, tokens=tokens,
            w_std=0.02, sigma_x=sx, sigma_g=sg, bits=2, group=128, block=128,
            had_in=hin, had_out=hout, seed=seed, layer=layer, x_stream=xs, g_stream=k))
    return cfgs


# ---------------------------------------------------------------------------
# bf16 helpers (storage only: bf16 values travel as uint16 bit patterns)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: LayerConfig, tid: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence([cfg.seed, cfg.cfg_index, tid, cfg.layer * 64 + stream, chunk]))


def channel_scales(cfg: LayerConfig, which: str) -> np.ndarray:
    """Per-channel standard deviations exp(sigma * N(0,1)) of the X or G stream."""
    if which == "x":
        n, sigma, tid, stream = cfg.inp, cfg.sigma_x, _TID_SCALE_X, cfg.x_stream
    else:
        n, sigma, tid, stream = cfg.out, cfg.sigma_g, _TID_SCALE_G, cfg.g_stream
    z = _rng(cfg, tid, stream, 0).standard_normal(n)
    return np.exp(sigma * z).astype(np.float32)


def _stream_chunk(cfg: LayerConfig, which: str, scales: np.ndarray, c: int, t0: int, t1: int,
                  out: np.ndarray) -> None:
    if which == "x":
        tid, stream = _TID_X, cfg.x_stream
    else:
        tid, stream = _TID_G, cfg.g_stream
    rng = _rng(cfg, tid, stream, c)
    a = rng.standard_normal((t1 - t0, scales.shape[0]), dtype=np.float32)
    a *= scales[None, :]
    out[t0:t1] = f32_to_bf16_bits(a)


def stream(cfg: LayerConfig, which: str, tokens: int | None = None, threads: int | None = None,
           out: np.ndarray | None = None) -> np.ndarray:
    """Calibration stream as bf16 bit patterns, uint16 [tokens x width].

    which = "x" (activations, width = in) or "g" (output gradients, width = out).
    Token chunk c always draws the same numbers, so a prefix of the stream is
    reproducible on its own (tokens < cfg.tokens gives the first rows).
    """
    T = cfg.tokens if tokens is None else tokens
    width = cfg.inp if which == "x" else cfg.out
    scales = channel_scales(cfg, which)
    if out is None:
        out = np.empty((T, width), dtype=np.uint16)
    nchunks = (T + CHUNK_TOKENS - 1) // CHUNK_TOKENS
    jobs = [(c, c * CHUNK_TOKENS, min(T, (c + 1) * CHUNK_TOKENS)) for c in range(nchunks)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr <= 1 or nchunks == 1:
        for c, t0, t1 in jobs:
            _stream_chunk(cfg, which, scales, c, t0, t1, out)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda j: _stream_chunk(cfg, which, scales, j[0], j[1], j[2], out), jobs))
    return out


def token_magnitudes(cfg: LayerConfig, tokens: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-token row factors (a, b) of the X and G streams for the FlipFlop workload."""
    rng = _rng(cfg, _TID_TOKMAG, cfg.x_stream, 0)
    z = rng.standard_normal(tokens)
    u = rng.standard_normal(tokens)
    return np.exp(0.5 * z).astype(np.float32), np.exp(0.5 * (0.8 * z + 0.6 * u)).astype(np.float32)


def flipflop_streams(cfg: LayerConfig, tokens: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """The X and G streams with their rows scaled by token_magnitudes, re-rounded to bf16."""
    T = cfg.tokens if tokens is None else tokens
    X = stream(cfg, "x", T)
    G = stream(cfg, "g", T)
    a, b = token_magnitudes(cfg, T)
    for t0 in range(0, T, CHUNK_TOKENS):
        t1 = min(T, t0 + CHUNK_TOKENS)
        X[t0:t1] = f32_to_bf16_bits(bf16_bits_to_f32(X[t0:t1]) * a[t0:t1, None])
        G[t0:t1] = f32_to_bf16_bits(bf16_bits_to_f32(G[t0:t1]) * b[t0:t1, None])
    return X, G


def weights(cfg: LayerConfig) -> np.ndarray:
    """Original weights W [out x in] as fp32 values (bf16-representable unless w_dtype is fp32)."""
    rng = _rng(cfg, _TID_W, cfg.g_stream, 0)
    if cfg.w_dist == "normal":
        w = rng.standard_normal((cfg.out, cfg.inp), dtype=np.float32) * np.float32(cfg.w_std)
    elif cfg.w_dist == "student_t4":
        w = (rng.standard_t(4.0, size=(cfg.out, cfg.inp)) * cfg.w_std).astype(np.float32)
    else:
        raise ValueError(cfg.w_dist)
    if cfg.n_outliers:
        cols = _rng(cfg, _TID_OUTL, cfg.g_stream, 0).choice(cfg.inp, size=cfg.n_outliers, replace=False)
        w[:, np.sort(cols)] *= np.float32(cfg.outlier_scale)
    if cfg.w_dtype == "bf16":
        w = bf16_bits_to_f32(f32_to_bf16_bits(w))
    return np.ascontiguousarray(w, dtype=np.float32)


def outlier_columns(cfg: LayerConfig) -> np.ndarray:
    if not cfg.n_outliers:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg, _TID_OUTL, cfg.g_stream, 0).choice(cfg.inp, size=cfg.n_outliers, replace=False))


def signs(cfg: LayerConfig, side: str) -> np.ndarray:
    """Random +-1 signs (int8) of the input ("in") or output ("out") rotation."""
    n, tid = (cfg.inp, _TID_SIN) if side == "in" else (cfg.out, _TID_SOUT)
    rng = _rng(cfg, tid, cfg.g_stream, 0)
    return (rng.integers(0, 2, size=n, dtype=np.int8) * 2 - 1).astype(np.int8)


def small_dense(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Plain seeded N(0, scale^2) fp64 array for unit tests."""
    return np.random.default_rng(seed).standard_normal(shape) * scale
