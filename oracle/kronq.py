"""fp64 reference of KronQ's per-layer quantization engine (test infrastructure).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may use this module; the product path never does.  Nothing here is shared
with, or imported from, the HIP library.

Notation (as in the KronQ README's opening section and the arXiv abstract):
W is out x in (rows = output channels), X is tokens x in (activations),
G is tokens x out (output gradients).  Under the Kronecker-factored (K-FAC)
Hessian H ~ H_X (x) H_G the layer loss of a weight perturbation dW is
tr(H_G dW H_X dW^T).  Quantities after incoherence processing carry the
suffix "t" (W~, H~).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "hessian_factor", "hessian_factor_entry", "stream_sq_norm", "trace",
    "sensitivity", "sylvester_hadamard", "hadamard_block_size", "rotate_rows", "rotate_cols",
    "rotation_matrix", "rescale_vectors", "biip", "BIIP_FULL", "BIIP_NO_RESCALE", "BIIP_IN_ONLY",
    "BIIP_OUT_ONLY", "damp_and_factor", "AsymMinMaxGrid", "FixedUniformGrid", "gptq",
    "GptqResult", "quantize_layer", "pack_codes", "unpack_codes", "proxy_loss", "predicted_loss",
    "allocate_bits", "brute_force_min_loss", "NotSPDError", "ClippedMinMaxGrid",
    "act_order_perm", "CLIP_NORM", "CLIP_GRID", "CLIP_MAXSHRINK", "dequant", "deploy_linear",
    "quadratic_forms", "flipflop_input_factor", "flipflop_output_factor", "flipflop",
    "flipflop_objective", "static_grid", "TwoSidedResult", "two_sided_gptq", "two_sided_rounding",
]

BIIP_FULL, BIIP_NO_RESCALE, BIIP_IN_ONLY, BIIP_OUT_ONLY = 0, 1, 2, 3


class NotSPDError(ValueError):
    """The damped input Hessian has no Cholesky factor (not positive definite)."""


# ---------------------------------------------------------------------------
# Hessian factors
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to fp64 values: the 16 bits are the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def hessian_factor(A: np.ndarray) -> np.ndarray:
    """One Kronecker factor of the layer Hessian: A^T A = sum over tokens of a a^T.

    [KronQ-README], opening section: H ~ H_X (x) H_G; H_X is built from the
    calibration activations X (A = X, tokens x in) and H_G from the output
    gradients G (A = G, tokens x out).  [WaterKron] Table 1, row "Marginal":
    the input factor is E[x x^T] and the output factor E[g g^T], taken
    independently.  READING: unnormalized sums (no 1/T), since codes do not
    depend on a common scale of H_X and T is equal across the sublayers that
    a sensitivity ranking compares.
    """
    A = np.asarray(A, dtype=np.float64)
    return A.T @ A


def hessian_factor_entry(A_cols_i: np.ndarray, A_cols_j: np.ndarray) -> np.ndarray:
    """Sampled entries H[i, j] = sum_t A[t, i] A[t, j] for paired column vectors (fp64)."""
    return np.einsum("ti,ti->i", np.asarray(A_cols_i, np.float64), np.asarray(A_cols_j, np.float64))


def stream_sq_norm(A: np.ndarray) -> float:
    """||A||_F^2 straight from the stream: equals tr(A^T A) (closed form)."""
    A = np.asarray(A, dtype=np.float64)
    return float(np.sum(A * A))


def trace(H: np.ndarray) -> float:
    """tr(H), summed in fp64 with exact rounding of the sum (math.fsum)."""
    return math.fsum(np.diag(np.asarray(H, dtype=np.float64)).tolist())


def sensitivity(HX: np.ndarray, HG: np.ndarray) -> tuple[float, float, float]:
    """Per-sublayer sensitivity s = tr(H_G) * tr(H_X).

    [KronQ-README] opening section (bit widths across sublayers are chosen from
    the product of the two factors' traces); [KronQ-abstract] point (2).  READING: taken
    on the raw factors, before incoherence processing (rotation keeps the
    trace, rescaling does not; the raw value is the layer's own property).
    Returns (tr H_X, tr H_G, product).
    """
    tx, tg = trace(HX), trace(HG)
    return tx, tg, tx * tg


# ---------------------------------------------------------------------------
# Randomized Hadamard rotation
# ---------------------------------------------------------------------------
def sylvester_hadamard(b: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order b (power of 2), natural order.

    Entry (i, j) is (-1)^popcount(i AND j).  [KronQ-README] flags section:
    the incoherence kernel is "had" (Hadamard).
    """
    if b <= 0 or b & (b - 1):
        raise ValueError("Hadamard order must be a power of 2")
    i = np.arange(b, dtype=np.int64)
    x = i[:, None] & i[None, :]
    par = np.zeros_like(x)
    while np.any(x):
        par ^= x & 1
        x >>= 1
    return (1 - 2 * par).astype(np.float64)


def hadamard_block_size(n: int, block: int = 0) -> int:
    """Block of the block-diagonal Hadamard.  READING: 0 selects the largest
    power of two that divides n (11008 = 43 x 256, 28672 = 7 x 4096, 4096 and
    8192 whole)."""
    if block == 0:
        block = n & (-n)
    if block <= 0 or block & (block - 1) or n % block:
        raise ValueError(f"Hadamard block {block} does not tile n={n}")
    return block


def rotation_matrix(signs: np.ndarray, block: int = 0) -> np.ndarray:
    """Dense P = blockdiag(Had_b, ..., Had_b) diag(S) / sqrt(b) (orthogonal)."""
    n = signs.shape[0]
    b = hadamard_block_size(n, block)
    Hb = sylvester_hadamard(b) / math.sqrt(b)
    P = np.zeros((n, n))
    for k in range(n // b):
        P[k * b:(k + 1) * b, k * b:(k + 1) * b] = Hb
    return P * np.asarray(signs, np.float64)[None, :]


def rotate_rows(M: np.ndarray, signs: np.ndarray, block: int = 0) -> np.ndarray:
    """M P^T: every row of M mapped by P (signs first, then the block Hadamard)."""
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[1]
    b = hadamard_block_size(n, block)
    Hb = sylvester_hadamard(b) / math.sqrt(b)
    Ms = M * np.asarray(signs, np.float64)[None, :]
    out = np.empty_like(Ms)
    for k in range(n // b):
        sl = slice(k * b, (k + 1) * b)
        out[:, sl] = Ms[:, sl] @ Hb.T
    return out


def rotate_cols(M: np.ndarray, signs: np.ndarray, block: int = 0) -> np.ndarray:
    """P M: every column of M mapped by P."""
    return rotate_rows(np.asarray(M, np.float64).T, signs, block).T


# ---------------------------------------------------------------------------
# Bidirectional incoherence processing (BiIP)
# ---------------------------------------------------------------------------
def rescale_vectors(W: np.ndarray, HX: np.ndarray, HG: np.ndarray | None, alpha: float,
                    mode: int = BIIP_FULL, hg_diag: np.ndarray | None = None
                    ) -> tuple[np.ndarray, np.ndarray]:
    """Diagonal rescale factors of BiIP, input side d_in and output side d_out.

    [KronQ-README] opening section: BiIP rotates and rescales on the input side
    and on the output side; the flags table gives alpha = 0.25 for
    weight-only runs.  The formula is not on the pages.  READING:
        d_in[i]  = (H_X[i,i] / sum_r W[r,i]^2) ** alpha
        d_out[k] = (H_G[k,k] / sum_i W[k,i]^2) ** alpha
    (alpha = 1/4 is the diagonal rescale that minimizes tr(D^-1 H D^-1) *
    ||W D||_F^2 on each side; a zero norm or diagonal gives d = 1).
    Parity unpinned for the rule itself: only the loss invariance and the
    proxy-bound optimality constrain it.  Only diag(H_G) enters d_out, so it can
    be given directly as hg_diag (for output sizes whose full H_G is too large).
    """
    W = np.asarray(W, np.float64)
    out_n, in_n = W.shape
    d_in, d_out = np.ones(in_n), np.ones(out_n)
    if mode in (BIIP_FULL, BIIP_IN_ONLY):
        c = np.sum(W * W, axis=0)
        h = np.diag(np.asarray(HX, np.float64))
        ok = (c > 0) & (h > 0)
        d_in[ok] = (h[ok] / c[ok]) ** alpha
    if mode in (BIIP_FULL, BIIP_OUT_ONLY):
        r = np.sum(W * W, axis=1)
        h = np.asarray(hg_diag, np.float64) if hg_diag is not None else np.diag(np.asarray(HG, np.float64))
        ok = (r > 0) & (h > 0)
        d_out[ok] = (h[ok] / r[ok]) ** alpha
    return d_in, d_out


def biip(W: np.ndarray, HX: np.ndarray, HG: np.ndarray | None, sign_in: np.ndarray,
         sign_out: np.ndarray | None, alpha: float = 0.25, mode: int = BIIP_FULL,
         had_in: int = 0, had_out: int = 0, hg_diag: np.ndarray | None = None):
    """Bidirectional incoherence processing of one linear layer.

    [KronQ-abstract] point (1) and [KronQ-README] opening section: the
    input-side random rotation is extended to the output dimension using the
    gradient covariance; both sides get a randomized Hadamard rotation plus a
    rescale.  [KronQ-news] also describes the rotation as carried over to the
    output side.
    READING (order and form):
      1. rescale   W <- D_out W D_in,  H_X <- D_in^-1 H_X D_in^-1,
                   H_G <- D_out^-1 H_G D_out^-1          (rescale_vectors)
      2. rotate    W~ = P_out W P_in^T,  H~_X = P_in H_X P_in^T,
                   H~_G = P_out H_G P_out^T,  P = blockdiag(Had_b) diag(S)/sqrt(b)
    so tr(H_G dW H_X dW^T) is unchanged for any dW mapped like W.
    mode: FULL (both sides, rescale + rotate), NO_RESCALE (both sides, rotate
    only), IN_ONLY / OUT_ONLY (one side, rescale + rotate).
    Returns (W~, H~_X, H~_G, d_in, d_out); H~_G is None when HG is None (then
    hg_diag, if given, supplies diag(H_G) for the output rescale).
    """
    W = np.asarray(W, np.float64)
    HX = np.asarray(HX, np.float64)
    HG = None if HG is None else np.asarray(HG, np.float64)
    if mode == BIIP_NO_RESCALE:
        d_in, d_out = np.ones(W.shape[1]), np.ones(W.shape[0])
    else:
        d_in, d_out = rescale_vectors(W, HX, HG, alpha, mode, hg_diag)
    Wt = W * d_out[:, None] * d_in[None, :]
    HXt = HX / np.outer(d_in, d_in)
    HGt = None if HG is None else HG / np.outer(d_out, d_out)
    if mode in (BIIP_FULL, BIIP_NO_RESCALE, BIIP_IN_ONLY):
        Wt = rotate_rows(Wt, sign_in, had_in)
        HXt = rotate_cols(rotate_rows(HXt, sign_in, had_in), sign_in, had_in)
    if mode in (BIIP_FULL, BIIP_NO_RESCALE, BIIP_OUT_ONLY):
        Wt = rotate_cols(Wt, sign_out, had_out)
        if HGt is not None:
            HGt = rotate_cols(rotate_rows(HGt, sign_out, had_out), sign_out, had_out)
    return Wt, HXt, HGt, d_in, d_out


# ---------------------------------------------------------------------------
# GPTQ with the damped Cholesky factor of H_X^-1
# ---------------------------------------------------------------------------
def damp_and_factor(HX: np.ndarray, damp: float = 0.01):
    """Damped inverse-Hessian Cholesky factor U = chol_upper((H_X + lam I)^-1).

    GPTQ convention, as KronQ runs it on the processed H~_X ([KronQ-README]
    flags table: GPTQ is the base quantizer): a zero diagonal entry marks a
    dead input channel (its diagonal becomes 1 and its weight column is
    zeroed), then lam = damp * mean(diag H), then U from the inverse.
    Deliberately computed as inv() followed by cholesky(), a different route
    from a reverse-order factorization.
    Returns (U, lam, dead_mask, H_damped).  Raises NotSPDError.
    """
    H = np.array(HX, dtype=np.float64, copy=True)
    n = H.shape[0]
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    lam = damp * float(np.mean(np.diag(H)))
    H[np.arange(n), np.arange(n)] += lam
    try:
        np.linalg.cholesky(H)
        Hinv = np.linalg.inv(H)
        Hinv = 0.5 * (Hinv + Hinv.T)
        U = np.linalg.cholesky(Hinv).T
    except np.linalg.LinAlgError as exc:
        raise NotSPDError(str(exc)) from exc
    return U, lam, dead, H


class AsymMinMaxGrid:
    """Asymmetric uniform min-max grid per (row, group) (`--w_asym`, `--w_groupsize`).

    [KronQ-README] flags table: weights are quantized with an asymmetric grid
    and group size 128 (or per-channel).  READINGS: the range is forced to
    include 0 (xmin = min(0, min), xmax = max(0, max)); scale s = (xmax - xmin)
    / (2^b - 1), or 1 when xmax = xmin; zero point z = rint(-xmin / s); code
    q = clip(rint(w / s) + z, 0, 2^b - 1); rint is round-half-to-even.  Group
    parameters are taken when the group's first column is reached, from the
    current (error-updated) weights.
    """

    def __init__(self, bits: int, group: int):
        if bits not in (2, 3, 4, 8) and not (1 <= bits <= 8):
            raise ValueError("bits")
        self.bits, self.group, self.maxq = bits, group, (1 << bits) - 1
        self.scale = self.zero = None

    def starts_group(self, j: int) -> bool:
        return j % self.group == 0

    def set_params(self, block: np.ndarray) -> None:
        xmin = np.minimum(block.min(axis=1), 0.0)
        xmax = np.maximum(block.max(axis=1), 0.0)
        s = (xmax - xmin) / self.maxq
        s[xmax == xmin] = 1.0
        self.scale = s
        self.zero = np.rint(-xmin / s)

    def unrounded(self, w: np.ndarray) -> np.ndarray:
        """w / s: the value rint() acts on (code = rint(w/s) + z, clamped)."""
        return w / self.scale

    def code(self, u: np.ndarray) -> np.ndarray:
        return np.clip(np.rint(u) + self.zero, 0, self.maxq)

    def dequant(self, q: np.ndarray) -> np.ndarray:
        return self.scale * (q - self.zero)


# The base recipe's `--w_clip` (KronQ README, "Reproduce from scratch"), which
# the pages name but do not define: READING, the shrink search of the GPTQ line
# of work, with these constants.
CLIP_NORM, CLIP_GRID, CLIP_MAXSHRINK = 2.4, 100, 0.8


class ClippedMinMaxGrid(AsymMinMaxGrid):
    """Min-max grid with a clip-ratio search (`--w_clip`).

    [KronQ-README] "Reproduce from scratch": the base recipe quantizes with
    `--w_clip --w_asym --w_groupsize -1`; the pages do not define the search.
    READING: for p = 1 - i / grid, i = 0 .. maxshrink * grid - 1, take the
    min-max grid (as AsymMinMaxGrid) of the shrunk range [p xmin, p xmax],
    quantize the group with it, and keep, per row, the p whose error
    sum |qhat - w|^norm is smallest (the first such p on equal errors).

    replay_scales (parity protocol, optional): another implementation's scale
    per row for the next group.  Where it picks a different candidate, its
    choice is adopted when that candidate's error here is within `tol`
    (relative) of the smallest (accepted_ties); otherwise this grid keeps its
    own choice (hard_mismatches).
    """

    def __init__(self, bits: int, group: int, norm: float = CLIP_NORM, grid: int = CLIP_GRID,
                 maxshrink: float = CLIP_MAXSHRINK, replay_scales=None, tol: float = 1e-5):
        super().__init__(bits, group)
        self.norm, self.grid, self.maxshrink = norm, grid, maxshrink
        self.replay_scales = replay_scales
        self.tol = tol
        self.accepted_ties = self.hard_mismatches = 0
        self.choice = None
        self.errors = None

    def candidates(self, block: np.ndarray):
        """Scales, zeros and errors of every candidate p, each [K x rows]."""
        block = np.asarray(block, np.float64)
        xmin0 = np.minimum(block.min(axis=1), 0.0)
        xmax0 = np.maximum(block.max(axis=1), 0.0)
        S, Z, E = [], [], []
        for i in range(int(self.maxshrink * self.grid)):
            p = 1.0 - i / self.grid
            xmin, xmax = p * xmin0, p * xmax0
            s = (xmax - xmin) / self.maxq
            s[xmax == xmin] = 1.0
            z = np.rint(-xmin / s)
            q = np.clip(np.rint(block / s[:, None]) + z[:, None], 0, self.maxq)
            err = np.sum(np.abs(s[:, None] * (q - z[:, None]) - block) ** self.norm, axis=1)
            S.append(s)
            Z.append(z)
            E.append(err)
        return np.array(S), np.array(Z), np.array(E)

    def set_params(self, block: np.ndarray) -> None:
        S, Z, E = self.candidates(block)
        rows = np.arange(S.shape[1])
        k = np.argmin(E, axis=0)   # first minimum
        if self.replay_scales is not None:
            other = np.asarray(self.replay_scales, np.float64)
            match = np.argmin(np.abs(S - other[None, :]), axis=0)
            found = np.abs(S[match, rows] - other) <= 1e-5 * np.abs(other)
            diff = match != k
            near = E[match, rows] <= E[k, rows] * (1.0 + self.tol)
            ok = diff & found & near
            k = np.where(ok, match, k)
            self.accepted_ties += int(ok.sum())
            self.hard_mismatches += int((diff & ~(found & near)).sum())
        self.choice = k
        self.errors = E
        self.scale = S[k, rows]
        self.zero = Z[k, rows]


def act_order_perm(HX: np.ndarray) -> np.ndarray:
    """Column order of `--act_order`: descending diag(H~_X).

    [KronQ-README] "Reproduce from scratch": the base recipe runs GPTQ with
    `--act_order`; the pages do not define it.  READING (GPTQ convention): a
    dead channel's zero diagonal counts as 1, as in damp_and_factor, and equal
    diagonals keep their index order (stable sort).  perm[p] is the original
    column quantized at position p.
    """
    d = np.array(np.diag(HX), dtype=np.float64, copy=True)
    d[d == 0] = 1.0
    return np.argsort(-d, kind="stable")


class FixedUniformGrid:
    """Unbounded uniform grid with one fixed step per column (no clamping).

    Used for the lattice picture of [WaterKron] Figure 1: lattice points
    diag(alpha) Z^n, each column j rounded to a multiple of alpha_j.
    """

    def __init__(self, steps: np.ndarray):
        self.steps = np.asarray(steps, np.float64)
        self.group = 1
        self.j = 0
        self.zero = 0.0

    def starts_group(self, j: int) -> bool:
        self.j = j
        return True

    def set_params(self, block: np.ndarray) -> None:
        self.scale = np.full(block.shape[0], self.steps[self.j])
        self.zero = np.zeros(block.shape[0])

    def unrounded(self, w):
        return w / self.scale

    def code(self, u):
        return np.rint(u)

    def dequant(self, q):
        return self.scale * q


@dataclass
class GptqResult:
    codes: np.ndarray          # int64 [out x in]
    scales: np.ndarray         # [out x groups]
    zeros: np.ndarray          # [out x groups]
    qhat: np.ndarray           # dequantized weights [out x in]
    E: np.ndarray              # whitened errors e_j as columns [out x in]
    unrounded: np.ndarray      # w/s at the moment each code was chosen [out x in]
    accepted_ties: int = 0
    hard_mismatches: int = 0
    mismatch_positions: list = field(default_factory=list)


def gptq(W: np.ndarray, U: np.ndarray, grid, dead: np.ndarray | None = None,
         replay_codes: np.ndarray | None = None, tie_window: float = 1e-4) -> GptqResult:
    """GPTQ error-feedback quantization, one column at a time (unblocked).

    Minimizes tr(dW H_d dW^T) column by column through U = chol_upper(H_d^-1):
    for j = 0..in-1: (at a group start) set the grid from the current weights;
    q_j = code(w_j); e_j = (w_j - qhat_j) / U[j,j]; w_k -= e_j U[j,k] for k > j.
    The lazy 128-column batching of blocked GPTQ is a reordering of these
    updates and does not change the result in exact arithmetic.  Rows are
    independent given U, so any subset of rows can be run on its own.

    replay_codes (parity protocol, optional): codes produced by another
    implementation from the same inputs.  Where they differ from this
    function's choice, the other code is adopted when it is the other
    neighbour of a value within tie_window of a rounding midpoint (both are
    correct results); the difference is then counted in accepted_ties.  Any
    other difference counts as a hard mismatch and this function keeps its
    own code.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    out_n, n = W.shape
    if dead is not None and np.any(dead):
        W[:, dead] = 0.0
    codes = np.zeros((out_n, n), dtype=np.int64)
    qhat = np.zeros((out_n, n))
    E = np.zeros((out_n, n))
    unr = np.zeros((out_n, n))
    ngroups = (n + grid.group - 1) // grid.group
    scales = np.zeros((out_n, ngroups))
    zeros = np.zeros((out_n, ngroups))
    acc = hard = 0
    positions = []
    for j in range(n):
        if grid.starts_group(j):
            g = j // grid.group
            grid.set_params(W[:, j:j + grid.group])
            scales[:, g], zeros[:, g] = grid.scale, grid.zero
        u = grid.unrounded(W[:, j])
        q = grid.code(u)
        if replay_codes is not None:
            other = replay_codes[:, j]
            diff = np.nonzero(q != other)[0]
            if diff.size:
                ud = u[diff]
                frac = ud - np.floor(ud)
                near = np.abs(frac - 0.5) < tie_window
                zero = np.broadcast_to(np.asarray(grid.zero, np.float64), u.shape)[diff]
                maxq = getattr(grid, "maxq", np.inf)
                lo = np.clip(np.floor(ud) + zero, 0, maxq)
                hi = np.clip(np.floor(ud) + 1.0 + zero, 0, maxq)
                ok = near & ((other[diff] == lo) | (other[diff] == hi))
                q[diff[ok]] = other[diff[ok]]
                acc += int(ok.sum())
                hard += int((~ok).sum())
                positions.extend((int(r), j) for r in diff[~ok])
        qh = grid.dequant(q)
        e = (W[:, j] - qh) / U[j, j]
        W[:, j + 1:] -= np.outer(e, U[j, j + 1:])
        codes[:, j], qhat[:, j], E[:, j], unr[:, j] = q, qh, e, u
    return GptqResult(codes, scales, zeros, qhat, E, unr, acc, hard, positions)


def proxy_loss(dW: np.ndarray, HX: np.ndarray, HG: np.ndarray | None = None) -> float:
    """K-FAC layer loss tr(H_G dW H_X dW^T) ([KronQ-README] opening section;
    [WaterKron] Table 1: H ~ A (x) B for H = E[x x^T (x) g g^T]).  H_G = None
    means the identity (GPTQ's objective)."""
    dW = np.asarray(dW, np.float64)
    A = dW @ np.asarray(HX, np.float64)
    if HG is None:
        return float(np.sum(A * dW))
    return float(np.sum((np.asarray(HG, np.float64) @ dW) * A))


def predicted_loss(E: np.ndarray, HG: np.ndarray | None = None) -> float:
    """GPTQ's accumulated per-column loss: sum_j e_j^T H_G e_j (e_j whitened errors)."""
    E = np.asarray(E, np.float64)
    if HG is None:
        return float(np.sum(E * E))
    return float(np.sum((np.asarray(HG, np.float64) @ E) * E))


def quantize_layer(Wt: np.ndarray, HXt: np.ndarray, HGt: np.ndarray | None, bits: int,
                   group: int, damp: float = 0.01, replay_codes: np.ndarray | None = None,
                   rows: np.ndarray | None = None, factor=None, act_order: bool = False,
                   w_clip: bool = False, replay_scales: np.ndarray | None = None):
    """Damp, factor and GPTQ-quantize a processed layer; also the two losses.

    [KronQ-README] opening section: KronQ extends GPTQ with H_G under the
    K-FAC objective; GPTQ itself rounds with H_X only.  Returns a dict with
    the GptqResult, U, lam, the direct loss tr(H~_G dW~ H~_X dW~^T) (undamped
    H~_X, dW~ = W~ - Qhat) and the predicted loss sum_j e_j^T H~_G e_j (which
    equals the direct loss taken with the damped H~_X).  With `rows`, only
    those rows are quantized (losses are then not computed).

    act_order / w_clip: the base recipe's `--act_order` and `--w_clip`
    ([KronQ-README] "Reproduce from scratch", with `--w_groupsize -1`), both
    for one grid per row (group = in).  With act_order, GPTQ runs on the
    columns in act_order_perm order (W~ and H~_X permuted, U refactored) and
    every per-column result is returned in the original order.  `factor`,
    when given, is that of the (permuted) H~_X; replay_codes are in the
    original order; replay_scales (w_clip) are per row.
    """
    W = np.asarray(Wt, np.float64)
    n = W.shape[1]
    if (act_order or w_clip) and group != n:
        raise ValueError("act_order and w_clip take one grid per row (group = in)")
    perm = act_order_perm(HXt) if act_order else np.arange(n)
    HXp = np.asarray(HXt, np.float64)[np.ix_(perm, perm)] if act_order else HXt
    if factor is None:
        U, lam, dead_p, Hd = damp_and_factor(HXp, damp)
    else:
        U, lam, dead_p, Hd = factor
    if rows is not None:
        W = W[rows]
    grid = (ClippedMinMaxGrid(bits, group, replay_scales=replay_scales) if w_clip
            else AsymMinMaxGrid(bits, group))
    rp = None if replay_codes is None else np.asarray(replay_codes)[:, perm]
    res = gptq(W[:, perm], U, grid, dead_p, rp)
    if act_order:
        for name in ("codes", "qhat", "E", "unrounded"):
            x = getattr(res, name)
            y = np.empty_like(x)
            y[:, perm] = x
            setattr(res, name, y)
        res.mismatch_positions = [(r, int(perm[j])) for r, j in res.mismatch_positions]
    dead = np.empty_like(dead_p)
    dead[perm] = dead_p
    out = {"gptq": res, "U": U, "lam": lam, "dead": dead, "perm": perm}
    if w_clip:
        out["clip_accepted_ties"] = grid.accepted_ties
        out["clip_hard_mismatches"] = grid.hard_mismatches
        out["clip_choice"] = grid.choice
        E = np.sort(grid.errors, axis=0)
        # smallest relative gap between the best and the runner-up candidate, over rows
        out["clip_margin"] = float(np.min((E[1] - E[0]) / np.maximum(E[0], 1e-300)))
    if rows is None:
        W0 = np.array(W, copy=True)
        W0[:, dead] = 0.0
        dW = W0 - res.qhat
        out["loss_direct"] = proxy_loss(dW, HXt, HGt)
        out["loss_pred"] = predicted_loss(res.E, HGt)
    return out


# ---------------------------------------------------------------------------
# Deploy side: the quantized layer's forward
# ---------------------------------------------------------------------------
def dequant(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """Qhat[r, c] = s[r, g] (q[r, c] - z[r, g]), g = c // group (the asymmetric grid's values)."""
    g = np.arange(codes.shape[1]) // group
    return np.asarray(scales, np.float64)[:, g] * (np.asarray(codes, np.float64)
                                                   - np.asarray(zeros, np.float64)[:, g])


def deploy_linear(Qhat: np.ndarray, d_in: np.ndarray, d_out: np.ndarray, sign_in: np.ndarray,
                  sign_out: np.ndarray, had_in: int, had_out: int, x: np.ndarray) -> np.ndarray:
    """y = D_out^-1 P_out^T Qhat P_in D_in^-1 x: a BiIP-quantized layer applied to x.

    [KronQ-README] opening section: the packed weights are dequantized on the
    fly in a fused dequant + BiIP matvec (the online BiIP forward of the
    deploy path).  Since W~ = P_out D_out W D_in P_in^T with P orthogonal and
    Qhat approximates W~, the layer is W ~ D_out^-1 P_out^T Qhat P_in D_in^-1:
    rescale and rotate the activation, multiply by Qhat, rotate back and
    rescale.  x may be one vector or a [batch x in] matrix (rows).
    """
    P_in = rotation_matrix(sign_in, had_in)
    P_out = rotation_matrix(sign_out, had_out)
    X = np.atleast_2d(np.asarray(x, np.float64))
    Xt = (X / np.asarray(d_in, np.float64)[None, :]) @ P_in.T
    Yt = Xt @ np.asarray(Qhat, np.float64).T
    Y = (Yt @ P_out) / np.asarray(d_out, np.float64)[None, :]
    return Y[0] if np.ndim(x) == 1 else Y


# ---------------------------------------------------------------------------
# FlipFlop Hessian factors
# ---------------------------------------------------------------------------
def _dead_to_unit(M: np.ndarray) -> np.ndarray:
    """Copy of M whose zero diagonal entries are 1.

    READING: a channel whose calibration data are all zero has a zero row and
    column in its factor; it counts as 1 on the diagonal, which leaves every
    quadratic form of the data unchanged (its entries are zero)."""
    M = np.array(M, dtype=np.float64, copy=True)
    d = np.diag(M).copy()
    z = d == 0.0
    M[np.flatnonzero(z), np.flatnonzero(z)] = 1.0
    return M


def quadratic_forms(S: np.ndarray, M: np.ndarray) -> np.ndarray:
    """q_t = s_t^T M^-1 s_t for every row s_t of S (zero-diagonal channels as in
    _dead_to_unit).  Written out: the explicit inverse, the product S M^-1, then a
    row-wise dot with S."""
    S = np.asarray(S, dtype=np.float64)
    Minv = np.linalg.inv(_dead_to_unit(M))
    return np.einsum("ti,ti->t", S @ Minv, S)


def flipflop_input_factor(X: np.ndarray, G: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A = E_t[(g_t^T B^-1 g_t) x_t x_t^T] / m.

    [WaterKron] Table 1, row "FlipFlop", input factor; E is the mean over the T
    calibration tokens (x_t, g_t are one token's activation and output
    gradient).  READING: the table gives the factors without constants; the
    1/m here (1/n for the output factor) is the classical flip-flop's, the
    maximum-likelihood fit of a Kronecker covariance to the samples
    vec(x_t g_t^T), and gives the iteration a fixed point when m != n.  A (x) B
    itself does not depend on it."""
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    T, m = G.shape
    w = quadratic_forms(G, B)
    return (X.T * w) @ X / (T * m)


def flipflop_output_factor(X: np.ndarray, G: np.ndarray, A: np.ndarray) -> np.ndarray:
    """B = E_t[(x_t^T A^-1 x_t) g_t g_t^T] / n ([WaterKron] Table 1, "FlipFlop",
    output factor; constants as in flipflop_input_factor)."""
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    T, n = X.shape
    v = quadratic_forms(X, A)
    return (G.T * v) @ G / (T * n)


def flipflop(X: np.ndarray, G: np.ndarray, iters: int, B0: np.ndarray | None = None):
    """The alternating fixed-point iteration of [WaterKron] Table 1 ("Frobenius
    and FlipFlop approximations are computed using the alternating fixed-point
    iteration, starting from the identity matrix").  READING: it starts from
    B = I and each iteration updates A from the current B, then B from the new
    A.  Returns [(A_1, B_1), ..., (A_iters, B_iters)]."""
    m = np.asarray(G).shape[1]
    B = np.eye(m) if B0 is None else np.asarray(B0, dtype=np.float64)
    out = []
    for _ in range(iters):
        A = flipflop_input_factor(X, G, B)
        B = flipflop_output_factor(X, G, A)
        out.append((A, B))
    return out


def flipflop_objective(X: np.ndarray, G: np.ndarray, A: np.ndarray, B: np.ndarray) -> float:
    """E_t[(x_t^T A^-1 x_t)(g_t^T B^-1 g_t)] + m log det A + n log det B: the Gaussian
    covariance fit of A (x) B to H = E[x x^T (x) g g^T], i.e. tr((A (x) B)^-1 H) +
    log det(A (x) B) ([WaterKron] abstract: minimizing the mismatch factor is a
    Gaussian covariance-fitting problem).  Each half step of flipflop minimizes
    it over one factor."""
    n, m = np.asarray(A).shape[0], np.asarray(B).shape[0]
    v = quadratic_forms(X, A)
    w = quadratic_forms(G, B)
    return float(np.mean(v * w) + m * np.linalg.slogdet(A)[1] + n * np.linalg.slogdet(B)[1])


# ---------------------------------------------------------------------------
# Two-sided rounding (GPTQ in the vectorized weight domain)
# ---------------------------------------------------------------------------
def static_grid(W: np.ndarray, bits: int, group: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-(row, group) asymmetric min-max grid taken once from W (the rules of
    AsymMinMaxGrid: range forced to include 0, s = (xmax - xmin) / (2^b - 1) or 1,
    z = rint(-xmin / s)).  READING for two-sided rounding: the grid does not follow
    the error-updated weights, so that every order of the rounding that respects
    the feedback's dependencies gives the same result."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    g = AsymMinMaxGrid(bits, group)
    ng = (n + group - 1) // group
    scales, zeros = np.zeros((m, ng)), np.zeros((m, ng))
    for k in range(ng):
        g.set_params(W[:, k * group:(k + 1) * group])
        scales[:, k], zeros[:, k] = g.scale, g.zero
    return scales, zeros


@dataclass
class TwoSidedResult:
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    qhat: np.ndarray
    accepted_ties: int = 0
    hard_mismatches: int = 0


def two_sided_gptq(W: np.ndarray, HX: np.ndarray, HG: np.ndarray, bits: int, group: int,
                   damp: float = 0.01, replay_codes: np.ndarray | None = None,
                   tie_window: float = 1e-4) -> TwoSidedResult:
    """GPTQ on vec(W) under the Kronecker Hessian H = H_X (x) H_G.

    [BaKron] abstract: GPTQ-style rounding applied directly in the vectorized
    weight domain with a two-sided Kronecker-factored Hessian (the formulation
    of BoA and YAQA), which BaKron then computes in O(m+n) sequential steps.
    Written out: with c = i m + r the position of W[r, i] in vec(W) (columns
    stacked), H_d = (H_X + lam_X I) (x) (H_G + lam_G I) and
    U = chol_upper(H_d^-1) = U_X (x) U_G, the coordinates are rounded in the
    order c = 0, 1, ...: q = code(w_c), e = (w_c - qhat_c) / U[c, c],
    w_c' -= e U[c, c'] for c' > c.  Since U[(i, r), (i', r')] = U_X[i, i']
    U_G[r, r'] vanishes unless i' >= i and r' >= r, each rounding feeds only the
    quadrant below and to the right of its coordinate; the update is written as
    that quadrant's outer product.  READINGS: damping and dead channels as in
    damp_and_factor on each factor (a dead output channel's row is zeroed like a
    dead input channel's column); grids from static_grid.  replay_codes: the
    tie protocol of gptq (another implementation's code is adopted at a value
    within tie_window of a rounding midpoint).
    """
    W = np.array(W, dtype=np.float64, copy=True)
    UX, _, deadX, _ = damp_and_factor(HX, damp)
    UG, _, deadG, _ = damp_and_factor(HG, damp)
    W[:, deadX] = 0.0
    W[deadG, :] = 0.0
    scales, zeros = static_grid(W, bits, group)
    return two_sided_rounding(W, UX, UG, scales, zeros, bits, group, replay_codes, tie_window)


def two_sided_rounding(W: np.ndarray, UX: np.ndarray, UG: np.ndarray, scales: np.ndarray,
                       zeros: np.ndarray, bits: int, group: int,
                       replay_codes: np.ndarray | None = None,
                       tie_window: float = 1e-4) -> TwoSidedResult:
    """The rounding loop of two_sided_gptq for given factors and grids.  Any leading block
    W[:a, :b] with the leading blocks of U_X and U_G is a problem of its own: its
    coordinates depend on none outside it."""
    W = np.array(W, dtype=np.float64, copy=True)
    m, n = W.shape
    maxq = (1 << bits) - 1
    codes = np.zeros((m, n), dtype=np.int64)
    qhat = np.zeros((m, n))
    acc = hard = 0
    for i in range(n):
        g = i // group
        for r in range(m):
            s, z = scales[r, g], zeros[r, g]
            u = W[r, i] / s
            q = int(np.clip(np.rint(u) + z, 0, maxq))
            if replay_codes is not None and int(replay_codes[r, i]) != q:
                other = int(replay_codes[r, i])
                lo = np.clip(np.floor(u) + z, 0, maxq)
                hi = np.clip(np.floor(u) + 1 + z, 0, maxq)
                if abs(u - np.floor(u) - 0.5) < tie_window and other in (lo, hi):
                    q = other
                    acc += 1
                else:
                    hard += 1
            qh = s * (q - z)
            e = (W[r, i] - qh) / (UX[i, i] * UG[r, r])
            W[r + 1:, i] -= e * UG[r, r + 1:] * UX[i, i]
            W[r:, i + 1:] -= e * np.outer(UG[r, r:], UX[i, i + 1:])
            codes[r, i], qhat[r, i] = q, qh
    return TwoSidedResult(codes, scales, zeros, qhat, acc, hard)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packed codes, one little-endian bitstream of uint32 words per row.

    [KronQ-README] opening section: weights are stored packed (int4/int2).
    READING (also for 3 bits, which the README ships unpacked): bit k of row
    r's stream is bit (k mod b) of code floor(k / b); word w holds stream bits
    32w .. 32w+31, least significant first.  Row length in * b must be a
    multiple of 32.  Written bit by bit.
    """
    codes = np.asarray(codes, dtype=np.int64)
    out_n, n = codes.shape
    nbits = n * bits
    if nbits % 32:
        raise ValueError("in * bits must be a multiple of 32")
    words = np.zeros((out_n, nbits // 32), dtype=np.int64)
    for k in range(nbits):
        bit = (codes[:, k // bits] >> (k % bits)) & 1
        words[:, k // 32] |= bit << (k % 32)
    return words.astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of pack_codes, bit by bit."""
    words = np.asarray(words, dtype=np.int64)
    codes = np.zeros((words.shape[0], n), dtype=np.int64)
    for k in range(n * bits):
        bit = (words[:, k // 32] >> (k % 32)) & 1
        codes[:, k // bits] |= bit << (k % bits)
    return codes


# ---------------------------------------------------------------------------
# Inter-layer bit allocation
# ---------------------------------------------------------------------------
def allocate_bits(sens, numel, allowed=(2, 3, 4), target_num: int = 5, target_den: int = 2,
                  report_margin: bool = False):
    """Per-sublayer bit widths from the tr(H_G) tr(H_X) sensitivities.

    [KronQ-README] opening section and flags table (mixed precision across
    sublayers, `--inter_layer_mp`); [KronQ-abstract] point (2).  The rule is
    not on the pages.  READING: a sublayer's expected loss is modelled as
    s_l * 4^-b_l (uniform-noise model: E tr(H_G dW H_X dW^T) = sigma^2 tr(H_G)
    tr(H_X), sigma^2 ~ 4^-b).  Start every sublayer at the lowest width; while
    the budget sum_l b_l n_l <= floor(target * sum_l n_l) allows, raise by one
    step the sublayer with the largest loss reduction per added bit-weight,
    gain_l = (s_l * (4^-b_l - 4^-b_next)) / n_l, ties to the smallest index.
    Integer budget; gains compared exactly in fp64 in that operation order.
    With report_margin, also returns the smallest relative gap, over all steps,
    between the chosen gain and the best gain it beat (how far the decisions
    were from a tie).
    """
    sens = [float(s) for s in sens]
    numel = [int(n) for n in numel]
    allowed = sorted(int(a) for a in allowed)
    L = len(sens)
    bits = [allowed[0]] * L
    total = sum(numel)
    budget = (total * target_num) // target_den
    used = allowed[0] * total
    margin = math.inf
    while True:
        best, best_gain = -1, -1.0
        gains = []
        for l in range(L):
            i = allowed.index(bits[l])
            if i + 1 >= len(allowed):
                continue
            nb = allowed[i + 1]
            if used + (nb - bits[l]) * numel[l] > budget:
                continue
            dq = 4.0 ** (-bits[l]) - 4.0 ** (-nb)
            gain = (sens[l] * dq) / float(numel[l] * (nb - bits[l]))
            gains.append(gain)
            if gain > best_gain:
                best, best_gain = l, gain
        if best < 0:
            break
        if len(gains) > 1 and best_gain > 0:
            runner = sorted(gains)[-2]
            margin = min(margin, (best_gain - runner) / best_gain)
        i = allowed.index(bits[best])
        used += (allowed[i + 1] - bits[best]) * numel[best]
        bits[best] = allowed[i + 1]
    return (bits, margin) if report_margin else bits


# ---------------------------------------------------------------------------
# Brute force (tiny inputs only)
# ---------------------------------------------------------------------------
def brute_force_min_loss(W: np.ndarray, HX: np.ndarray, HG: np.ndarray | None, scales: np.ndarray,
                         zeros: np.ndarray, bits: int) -> float:
    """min over every code assignment on the given per-row grid of
    tr(H_G dW H_X dW^T) (one group per row).  (2^b)^(out*in) evaluations."""
    W = np.asarray(W, np.float64)
    out_n, n = W.shape
    levels = 1 << bits
    best = math.inf
    grid = [scales[r] * (np.arange(levels) - zeros[r]) for r in range(out_n)]
    for flat in range(levels ** (out_n * n)):
        Q = np.empty((out_n, n))
        x = flat
        for r in range(out_n):
            for c in range(n):
                Q[r, c] = grid[r][x % levels]
                x //= levels
        best = min(best, proxy_loss(W - Q, HX, HG))
    return best
