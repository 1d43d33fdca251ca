"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle stage to a closed form, an invariant, a brute-force
search, a hand-derived example or a printed worked example, chosen so that a
plausible slip (dropped term, wrong sign or side, transposed operand, wrong
exponent) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as o
from synthetic import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def spd(rng, n, cond_scale=1.0):
    A = rng.standard_normal((3 * n, n)) * np.exp(cond_scale * rng.standard_normal(n))[None, :]
    return A.T @ A


# ---------------------------------------------------------------------------
# Hessian factors and sensitivity
# ---------------------------------------------------------------------------
def test_hessian_matches_triple_loop():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((7, 5))
    H = o.hessian_factor(A)
    for i in range(5):
        for j in range(5):
            s = 0.0
            for t in range(7):
                s += A[t, i] * A[t, j]
            assert H[i, j] == pytest.approx(s, rel=1e-14, abs=1e-14)


def test_hessian_symmetric_psd_and_trace_is_frobenius():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((50, 12)) * np.exp(rng.standard_normal(12))
    H = o.hessian_factor(A)
    assert np.array_equal(H, H.T) or np.allclose(H, H.T, rtol=0, atol=1e-12)
    assert np.linalg.eigvalsh(H).min() > -1e-9 * np.abs(H).max()
    assert o.trace(H) == pytest.approx(float(np.sum(A * A)), rel=1e-13)
    assert o.stream_sq_norm(A) == pytest.approx(o.trace(H), rel=1e-13)


def test_sampled_entries_match_full_factor():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((40, 9))
    H = o.hessian_factor(A)
    i = np.array([0, 3, 8, 5])
    j = np.array([0, 7, 2, 5])
    np.testing.assert_allclose(o.hessian_factor_entry(A[:, i], A[:, j]), H[i, j], rtol=1e-12, atol=1e-12)


def test_bf16_decoding_known_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x4049], dtype=np.uint16)
    # 1.0, -2.0, 1 + 2^-7, 0, 3.140625 (0x4049 -> sign 0, exp 128, mantissa 0x49)
    np.testing.assert_array_equal(o.bf16_bits_to_f64(bits), [1.0, -2.0, 1.0078125, 0.0, 3.140625])


def test_bf16_generator_rounds_to_nearest_even():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties to even (1.0);
    # 1 + 3*2^-8 lies between 1+2^-7 and 1+2^-6: ties to even (1 + 2^-6).
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    y = bf16_bits_to_f32(f32_to_bf16_bits(x))
    np.testing.assert_array_equal(y, np.array([1.0, 1 + 2 ** -6, 1 + 2 ** -7], dtype=np.float32))


def test_sensitivity_is_product_of_stream_norms():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((30, 6)) * 2.0
    G = rng.standard_normal((30, 4)) * 0.5
    tx, tg, s = o.sensitivity(o.hessian_factor(X), o.hessian_factor(G))
    assert s == pytest.approx(float(np.sum(X * X)) * float(np.sum(G * G)), rel=1e-13)
    assert tx == pytest.approx(float(np.sum(X * X)), rel=1e-13)
    assert tg == pytest.approx(float(np.sum(G * G)), rel=1e-13)


# ---------------------------------------------------------------------------
# Hadamard and rotation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 4, 16, 64, 256])
def test_sylvester_orthogonality_and_recursive_construction(b):
    H = o.sylvester_hadamard(b)
    np.testing.assert_array_equal(H @ H.T, b * np.eye(b))
    np.testing.assert_array_equal(H, H.T)
    # Sylvester's recursive construction H_2m = [[H_m, H_m], [H_m, -H_m]]
    R = np.array([[1.0]])
    while R.shape[0] < b:
        R = np.block([[R, R], [R, -R]])
    np.testing.assert_array_equal(H, R)


def test_hadamard_block_rule():
    assert o.hadamard_block_size(11008) == 256
    assert o.hadamard_block_size(28672) == 4096
    assert o.hadamard_block_size(4096) == 4096
    assert o.hadamard_block_size(8192) == 8192
    assert o.hadamard_block_size(16384) == 16384     # no cap: the whole power of 2
    assert o.hadamard_block_size(3 * 16384) == 16384
    assert o.hadamard_block_size(8192, 4096) == 4096
    with pytest.raises(ValueError):
        o.hadamard_block_size(96, 64)


@pytest.mark.parametrize("n,b", [(64, 0), (96, 32), (48, 16)])
def test_rotation_is_orthogonal_and_matches_dense(n, b):
    rng = np.random.default_rng(5)
    s = rng.choice([-1, 1], size=n)
    P = o.rotation_matrix(s, b)
    np.testing.assert_allclose(P @ P.T, np.eye(n), atol=1e-13)
    M = rng.standard_normal((5, n))
    np.testing.assert_allclose(o.rotate_rows(M, s, b), M @ P.T, atol=1e-13)
    np.testing.assert_allclose(o.rotate_cols(M.T, s, b), P @ M.T, atol=1e-13)


def _map_like_w(dW, d_in, d_out, s_in, s_out, had_in, had_out, mode):
    M = dW * d_out[:, None] * d_in[None, :]
    if mode != o.BIIP_OUT_ONLY:
        M = o.rotate_rows(M, s_in, had_in)
    if mode != o.BIIP_IN_ONLY:
        M = o.rotate_cols(M, s_out, had_out)
    return M


@pytest.mark.parametrize("mode", [o.BIIP_FULL, o.BIIP_NO_RESCALE, o.BIIP_IN_ONLY, o.BIIP_OUT_ONLY])
def test_biip_keeps_kfac_loss_invariant(mode):
    rng = np.random.default_rng(6)
    out_n, in_n = 24, 32
    W = rng.standard_normal((out_n, in_n)) * 0.02
    W[:, 3] *= 20
    HX, HG = spd(rng, in_n), spd(rng, out_n)
    s_in, s_out = rng.choice([-1, 1], in_n), rng.choice([-1, 1], out_n)
    Wt, HXt, HGt, d_in, d_out = o.biip(W, HX, HG, s_in, s_out, 0.25, mode, 16, 8)
    for k in range(3):
        dW = rng.standard_normal((out_n, in_n))
        dWt = _map_like_w(dW, d_in, d_out, s_in, s_out, 16, 8, mode)
        assert o.proxy_loss(dWt, HXt, HGt) == pytest.approx(o.proxy_loss(dW, HX, HG), rel=1e-11)
    # W itself is mapped the same way
    np.testing.assert_allclose(Wt, _map_like_w(W, d_in, d_out, s_in, s_out, 16, 8, mode), atol=1e-14)
    # traces change only through the rescale; rotation alone keeps them
    if mode == o.BIIP_NO_RESCALE:
        assert o.trace(HXt) == pytest.approx(o.trace(HX), rel=1e-12)
        assert o.trace(HGt) == pytest.approx(o.trace(HG), rel=1e-12)


def test_rescale_quarter_power_minimizes_proxy_bound():
    """With alpha = 1/4 each side's d minimizes tr(D^-1 H D^-1) * ||W D||_F^2 over
    positive diagonals (Cauchy-Schwarz); random perturbations only increase it."""
    rng = np.random.default_rng(7)
    W = rng.standard_normal((10, 12))
    W[:, 2] *= 15
    HX, HG = spd(rng, 12, 1.0), spd(rng, 10, 1.0)
    d_in, d_out = o.rescale_vectors(W, HX, HG, 0.25, o.BIIP_FULL)

    def f_in(d):
        return np.sum(np.diag(HX) / d ** 2) * np.sum((W * d[None, :]) ** 2)

    def f_out(d):
        return np.sum(np.diag(HG) / d ** 2) * np.sum((W * d[:, None]) ** 2)

    base_in, base_out = f_in(d_in), f_out(d_out)
    for _ in range(50):
        assert f_in(d_in * np.exp(0.1 * rng.standard_normal(12))) >= base_in * (1 - 1e-12)
        assert f_out(d_out * np.exp(0.1 * rng.standard_normal(10))) >= base_out * (1 - 1e-12)
    # alpha = 1/2 (or the reciprocal rule) is not the minimizer
    d_half, _ = o.rescale_vectors(W, HX, HG, 0.5, o.BIIP_FULL)
    assert f_in(d_half) > base_in
    assert f_in(1.0 / d_in) > base_in


def test_rescale_degenerate_entries_give_unit_factor():
    W = np.zeros((3, 4))
    W[:, 1:] = 1.0
    HX = np.diag([1.0, 2.0, 0.0, 4.0])
    HG = np.eye(3)
    d_in, d_out = o.rescale_vectors(W, HX, HG, 0.25)
    assert d_in[0] == 1.0 and d_in[2] == 1.0
    assert d_in[1] == pytest.approx((2.0 / 3.0) ** 0.25)


# ---------------------------------------------------------------------------
# Grid, GPTQ and losses
# ---------------------------------------------------------------------------
def test_minmax_grid_hand_example():
    # group values (-1, 0.5, 2) at 2 bits: xmin -1, xmax 2, s = 1, z = 1;
    # codes rint(w/s) + z = (0, rint(0.5) + 1 = 1 [half to even], 3); dequant (-1, 0, 2)
    g = o.AsymMinMaxGrid(2, 3)
    blk = np.array([[-1.0, 0.5, 2.0]])
    g.set_params(blk)
    assert g.scale[0] == 1.0 and g.zero[0] == 1.0
    q = g.code(g.unrounded(blk[0]))
    np.testing.assert_array_equal(q, [0, 1, 3])
    np.testing.assert_array_equal(g.dequant(q), [-1.0, 0.0, 2.0])
    # all-positive group: range forced to include 0 -> xmin 0, z 0; (0.3, 0.6, 0.9) at 2 bits: s = 0.3
    g.set_params(np.array([[0.3, 0.6, 0.9]]))
    assert g.zero[0] == 0.0 and g.scale[0] == pytest.approx(0.3)
    # all-zero group: s = 1, z = 0
    g.set_params(np.zeros((1, 3)))
    assert g.scale[0] == 1.0 and g.zero[0] == 0.0


def _textbook_rtn(W, bits, group):
    """Round-to-nearest on an asymmetric min-max grid per (row, group), no feedback."""
    maxq = 2 ** bits - 1
    Q = np.empty_like(W)
    codes = np.empty(W.shape, dtype=np.int64)
    for g0 in range(0, W.shape[1], group):
        blk = W[:, g0:g0 + group]
        lo = np.minimum(blk.min(1), 0)
        hi = np.maximum(blk.max(1), 0)
        step = np.where(hi > lo, (hi - lo) / maxq, 1.0)
        zp = np.rint(-lo / step)
        c = np.clip(np.rint(blk / step[:, None]) + zp[:, None], 0, maxq)
        codes[:, g0:g0 + group] = c
        Q[:, g0:g0 + group] = step[:, None] * (c - zp[:, None])
    return codes, Q


@pytest.mark.parametrize("bits,group", [(2, 8), (3, 16), (4, 32)])
def test_gptq_with_diagonal_hessian_is_rtn(bits, group):
    rng = np.random.default_rng(8)
    W = rng.standard_normal((16, 32)) * 0.05
    HX = np.diag(np.exp(rng.standard_normal(32)))
    r = o.quantize_layer(W, HX, None, bits, group, 0.01)
    codes, Q = _textbook_rtn(W, bits, group)
    np.testing.assert_array_equal(r["gptq"].codes, codes)
    np.testing.assert_allclose(r["gptq"].qhat, Q, atol=1e-15)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gptq_single_column_is_rtn(bits):
    rng = np.random.default_rng(9)
    W = rng.standard_normal((64, 1))
    HX = np.array([[2.5]])
    r = o.quantize_layer(W, HX, None, bits, 1, 0.01)
    codes, Q = _textbook_rtn(W, bits, 1)
    np.testing.assert_array_equal(r["gptq"].codes, codes)


@pytest.mark.parametrize("bits,group,with_hg", [(2, 8, False), (2, 8, True), (3, 16, True), (4, 32, False)])
def test_gptq_predicted_loss_equals_direct_loss(bits, group, with_hg):
    """W0 - Qhat = E U and U H_d U^T = I, so sum_j e_j^T H_G e_j = tr(H_G dW H_d dW^T)."""
    rng = np.random.default_rng(10)
    n, m = 32, 12
    W = rng.standard_normal((m, n)) * 0.02
    W[:, 5] *= 20
    HX = spd(rng, n, 1.0)
    HG = spd(rng, m) if with_hg else None
    r = o.quantize_layer(W, HX, HG, bits, group, 0.01)
    res, U, lam = r["gptq"], r["U"], r["lam"]
    dW = W - res.qhat
    np.testing.assert_allclose(dW, res.E @ U, atol=1e-12)
    Hd = HX + lam * np.eye(n)
    np.testing.assert_allclose(U @ Hd @ U.T, np.eye(n), atol=1e-9)
    assert r["loss_pred"] == pytest.approx(o.proxy_loss(dW, Hd, HG), rel=1e-10)
    # the direct loss (undamped) is the predicted loss minus lam * tr(H_G dW dW^T)
    assert r["loss_direct"] == pytest.approx(
        r["loss_pred"] - lam * o.proxy_loss(dW, np.eye(n), HG), rel=1e-9)


def test_gptq_rows_are_independent():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((20, 24))
    HX = spd(rng, 24)
    full = o.quantize_layer(W, HX, None, 2, 8, 0.01)
    rows = np.array([3, 17, 0])
    sub = o.quantize_layer(W, HX, None, 2, 8, 0.01, rows=rows)
    np.testing.assert_array_equal(sub["gptq"].codes, full["gptq"].codes[rows])


def test_gptq_whitened_errors_within_babai_box():
    """Unclamped columns: |w_j - qhat_j| <= s/2, i.e. |e_j| <= s / (2 U_jj)."""
    rng = np.random.default_rng(12)
    W = rng.standard_normal((16, 32))
    HX = spd(rng, 32)
    r = o.quantize_layer(W, HX, None, 4, 32, 0.01)
    res, U = r["gptq"], r["U"]
    s = np.repeat(res.scales, 32, axis=1)
    u = res.unrounded
    unclamped = (res.codes > 0) & (res.codes < 15)
    bound = s / (2 * np.diag(U))[None, :]
    assert np.all(np.abs(res.E)[unclamped] <= bound[unclamped] * (1 + 1e-12))
    assert unclamped.mean() > 0.5
    assert np.all((res.codes >= 0) & (res.codes <= 15))
    del u


def test_gptq_brute_force_bounds_2x4_w2():
    """Exhaustive search over all 4^8 W2 codes of a 2x4 weight bounds GPTQ's loss from below."""
    rng = np.random.default_rng(13)
    for trial in range(3):
        W = rng.standard_normal((2, 4))
        HX = spd(rng, 4, 0.5)
        HG = spd(rng, 2) if trial else None
        r = o.quantize_layer(W, HX, HG, 2, 4, 0.0)
        res = r["gptq"]
        # the grid of the one group per row is set from the original W at column 0
        g = o.AsymMinMaxGrid(2, 4)
        g.set_params(W)
        np.testing.assert_allclose(res.scales[:, 0], g.scale)
        best = o.brute_force_min_loss(W, HX, HG, g.scale, g.zero, 2)
        gl = o.proxy_loss(W - res.qhat, HX, HG)
        assert best <= gl * (1 + 1e-12)
        assert best > 0


def test_babai_fig1_worked_example():
    """[WaterKron] Figure 1: GPTQ on H = L^T L is Babai rounding on the lattice L diag(alpha) Z^2."""
    with open(os.path.join(GOLDEN, "babai_fig1.json")) as f:
        gold = json.load(f)
    L = np.array(gold["L"])
    H = L.T @ L
    np.testing.assert_array_equal(H, np.array(gold["derived_by_hand"]["H = L^T L"]))
    U, lam, dead, _ = o.damp_and_factor(H, 0.0)
    np.testing.assert_allclose(U, np.array(gold["derived_by_hand"]["U = chol_upper(H^-1) = L^-T"]), atol=1e-15)
    assert -U[0, 1] / U[0, 0] == pytest.approx(gold["derived_by_hand"]["feedback coefficient -U12/U11"])
    rng = np.random.default_rng(14)
    for key in ("alpha_rect", "alpha_square"):
        alpha = np.array(gold[key])
        half = 0.5 * np.diag(L) * alpha          # half-sides of the error cell
        w = rng.standard_normal((400, 2))        # targets L w, w ~ N(0, I_2)
        res = o.gptq(w, U, o.FixedUniformGrid(alpha))
        q = res.qhat
        e = (w - q) @ L.T                        # lattice-coordinate error L (w - q)
        np.testing.assert_allclose(res.E, e, atol=1e-12)
        assert np.all(np.abs(e) <= half * (1 + 1e-12))
        # Babai's cell is a fundamental region: exactly one lattice point per target lands in it
        for t in range(0, 400, 40):
            base = np.rint(w[t] / alpha)
            hits = []
            for a, b in itertools.product(range(-3, 4), repeat=2):
                cand = (base + np.array([a, b])) * alpha
                err = L @ (w[t] - cand)
                if np.all(np.abs(err) < half):
                    hits.append(cand)
            assert len(hits) == 1
            np.testing.assert_allclose(hits[0], q[t], atol=1e-12)
    sides = np.diag(L) * np.array(gold["alpha_square"])
    np.testing.assert_allclose(sides, gold["derived_by_hand"]["cell sides (L11 alpha1, L22 alpha2) at alpha_square"])
    assert np.prod(sides) == pytest.approx(gold["derived_by_hand"]["cell area = det L * alpha1 * alpha2"])
    assert np.prod(sides) == pytest.approx(np.linalg.det(L))


def test_not_spd_raises():
    with pytest.raises(o.NotSPDError):
        o.damp_and_factor(np.array([[1.0, 2.0], [2.0, 1.0]]), 0.01)


def test_dead_channel_rule():
    rng = np.random.default_rng(15)
    HX = spd(rng, 8)
    HX[3, :] = 0
    HX[:, 3] = 0
    W = rng.standard_normal((4, 8))
    r = o.quantize_layer(W, HX, None, 2, 8, 0.01)
    assert r["dead"][3] and r["dead"].sum() == 1
    assert np.all(r["gptq"].qhat[:, 3] == 0)


# ---------------------------------------------------------------------------
# Damping: lambda = damp * mean(diag H~_X) on the processed factor, after a dead channel's
# diagonal is set to 1 (the single-layer workload's damping of one percent of the mean
# diagonal, read as GPTQ's relative damping of the factor it factors)
# ---------------------------------------------------------------------------
def test_damping_hand_example_with_dead_channel():
    """H = diag(4, 0, 8, 12), damp 0.01.  The dead channel counts as 1, so the mean diagonal
    is (4 + 1 + 8 + 12) / 4 = 6.25 and lambda = 0.0625: not 0.06 (mean taken before the dead
    diagonal is set), not 0.25 (1 % of the trace).  For a diagonal H the factor of
    (H + lambda I)^-1 is diag(1 / sqrt(h_i + lambda)) by hand."""
    H = np.diag([4.0, 0.0, 8.0, 12.0])
    U, lam, dead, Hd = o.damp_and_factor(H, 0.01)
    assert lam == pytest.approx(0.0625, rel=1e-15)
    assert list(dead) == [False, True, False, False]
    hd = [4.0625, 1.0625, 8.0625, 12.0625]
    np.testing.assert_allclose(np.diag(Hd), hd, rtol=1e-15)
    np.testing.assert_allclose(U, np.diag([1.0 / math.sqrt(v) for v in hd]), rtol=1e-14, atol=1e-300)


def test_damping_hand_example_2x2():
    """H = [[2, 1], [1, 2]], damp 0.5: lambda = 0.5 * 2 = 1, H_d = [[3, 1], [1, 3]],
    H_d^-1 = [[3, -1], [-1, 3]] / 8, whose upper Cholesky factor is, by hand,
    U = [[sqrt(3/8), -1 / (8 sqrt(3/8))], [0, 1 / sqrt(3)]]."""
    U, lam, _, Hd = o.damp_and_factor(np.array([[2.0, 1.0], [1.0, 2.0]]), 0.5)
    assert lam == 1.0
    np.testing.assert_array_equal(Hd, [[3.0, 1.0], [1.0, 3.0]])
    a = math.sqrt(3.0 / 8.0)
    np.testing.assert_allclose(U, [[a, -1.0 / (8.0 * a)], [0.0, 1.0 / math.sqrt(3.0)]], rtol=1e-14)


def test_damping_is_taken_on_the_processed_factor():
    """After BiIP the mean diagonal of H~_X is sum_i H_ii / d_i^2 / n: the rotation keeps the
    trace, the rescale divides entry (i, i) by d_i^2, with d_i = (H_ii / c_i)^(1/4) and c_i the
    squared norm of W's column i.  Here that mean is far from the raw one, so lambda taken
    from the raw H_X (or with damp times the trace) fails; the factor GPTQ then uses must
    whiten H~_X + lambda I."""
    rng = np.random.default_rng(77)
    n, out = 16, 8
    A = rng.standard_normal((64, n)) * np.exp(1.5 * rng.standard_normal(n))[None, :]
    HX = A.T @ A
    B = rng.standard_normal((64, out))
    HG = B.T @ B
    W = rng.standard_normal((out, n)) * 0.02 * np.exp(rng.standard_normal(n))[None, :]
    c = [sum(W[r, i] ** 2 for r in range(out)) for i in range(n)]
    d = [math.sqrt(math.sqrt(HX[i, i] / c[i])) for i in range(n)]
    mean_t = sum(HX[i, i] / d[i] ** 2 for i in range(n)) / n
    mean_raw = sum(HX[i, i] for i in range(n)) / n
    assert abs(mean_t - mean_raw) > 0.5 * mean_raw      # the case tells the two apart
    s_in = rng.choice([-1, 1], n).astype(np.int8)
    s_out = rng.choice([-1, 1], out).astype(np.int8)
    Wt, HXt, HGt, _, _ = o.biip(W, HX, HG, s_in, s_out, 0.25, o.BIIP_FULL, 0, 0)
    r = o.quantize_layer(Wt, HXt, HGt, 2, n, 0.01)
    assert r["lam"] == pytest.approx(0.01 * mean_t, rel=1e-12)
    U = r["U"]
    np.testing.assert_allclose(U @ (HXt + 0.01 * mean_t * np.eye(n)) @ U.T, np.eye(n), atol=1e-9)


def test_replay_accepts_only_near_ties():
    rng = np.random.default_rng(16)
    W = rng.standard_normal((8, 16))
    HX = spd(rng, 16)
    r = o.quantize_layer(W, HX, None, 2, 16, 0.01)
    codes = r["gptq"].codes.copy()
    same = o.quantize_layer(W, HX, None, 2, 16, 0.01, replay_codes=codes)["gptq"]
    assert same.hard_mismatches == 0 and same.accepted_ties == 0
    bad = codes.copy()
    u = r["gptq"].unrounded
    far = np.abs((u - np.floor(u)) - 0.5) > 0.1
    rr, cc = np.argwhere(far & (codes > 0))[0]
    bad[rr, cc] -= 1
    out = o.quantize_layer(W, HX, None, 2, 16, 0.01, replay_codes=bad)["gptq"]
    assert out.hard_mismatches >= 1 and (int(rr), int(cc)) in out.mismatch_positions


# ---------------------------------------------------------------------------
# act_order and w_clip (the base recipe's flags; readings, see the oracle)
# ---------------------------------------------------------------------------
def test_act_order_perm_hand_example():
    # diagonal (2, 5, 0, 5, 3): the dead entry counts as 1; descending, equal values by index
    H = np.diag([2.0, 5.0, 0.0, 5.0, 3.0])
    np.testing.assert_array_equal(o.act_order_perm(H), [1, 3, 4, 0, 2])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_act_order_with_diagonal_hessian_is_rtn(bits):
    # no off-diagonal coupling: GPTQ is RTN in any column order, so the codes must land back
    # in their own columns after the permutation (a wrong inverse permutation scrambles them)
    rng = np.random.default_rng(31)
    W = rng.standard_normal((12, 40)) * 0.05
    HX = np.diag(np.exp(2.0 * rng.standard_normal(40)))
    r = o.quantize_layer(W, HX, None, bits, 40, 0.01, act_order=True)
    assert not np.array_equal(r["perm"], np.arange(40))
    codes, Q = _textbook_rtn(W, bits, 40)
    np.testing.assert_array_equal(r["gptq"].codes, codes)
    np.testing.assert_allclose(r["gptq"].qhat, Q, atol=1e-15)


def test_act_order_result_is_independent_of_input_column_order():
    # act_order processes columns in a canonical order (descending diagonal), so quantizing a
    # column-permuted layer gives the same codes, moved with the columns
    rng = np.random.default_rng(32)
    n = 24
    W = rng.standard_normal((10, n)) * 0.05
    HX = spd(rng, n)
    pi = rng.permutation(n)
    a = o.quantize_layer(W, HX, None, 3, n, 0.01, act_order=True)
    b = o.quantize_layer(W[:, pi], HX[np.ix_(pi, pi)], None, 3, n, 0.01, act_order=True)
    np.testing.assert_array_equal(b["gptq"].codes, a["gptq"].codes[:, pi])
    np.testing.assert_allclose(b["gptq"].E, a["gptq"].E[:, pi], rtol=0, atol=0)
    # and the order matters without act_order (the check above is not vacuous)
    c = o.quantize_layer(W[:, pi], HX[np.ix_(pi, pi)], None, 3, n, 0.01)
    d = o.quantize_layer(W, HX, None, 3, n, 0.01)
    assert not np.array_equal(c["gptq"].codes, d["gptq"].codes[:, pi])


def test_act_order_equal_diagonal_is_natural_order():
    rng = np.random.default_rng(33)
    n = 16
    A = spd(rng, n)
    dA = np.sqrt(np.diag(A))
    HX = A / np.outer(dA, dA)   # correlation matrix
    HX[np.arange(n), np.arange(n)] = 1.0   # exactly unit diagonal
    W = rng.standard_normal((6, n)) * 0.05
    a = o.quantize_layer(W, HX, None, 2, n, 0.01, act_order=True)
    b = o.quantize_layer(W, HX, None, 2, n, 0.01)
    np.testing.assert_array_equal(a["perm"], np.arange(n))
    np.testing.assert_array_equal(a["gptq"].codes, b["gptq"].codes)


def test_act_order_keeps_the_gptq_identity():
    # W0 - Qhat = E U in the permuted order, so sum_j |e_j|^2 = tr(dW H_d dW^T) in any order
    rng = np.random.default_rng(34)
    n = 32
    W = rng.standard_normal((8, n)) * 0.05
    HX = spd(rng, n)
    r = o.quantize_layer(W, HX, None, 3, n, 0.01, act_order=True)
    Hd = HX + r["lam"] * np.eye(n)
    dW = W - r["gptq"].qhat
    assert r["loss_pred"] == pytest.approx(o.proxy_loss(dW, Hd), rel=1e-10)


def test_clip_hand_example():
    # row (3, 3, 3, 3, 10) at 2 bits (maxq 3); xmin = 0, so z = 0 and s = 10 p / 3.  By hand,
    # sum |qhat - w|^2.4 for p = 1: 4 (1/3)^2.4 = 0.2864; 0.99: 4 (0.3)^2.4 + 0.1^2.4 = 0.2265;
    # 0.98: 4 (0.2667)^2.4 + 0.2^2.4 = 0.1886; 0.97: 4 (0.2333)^2.4 + 0.3^2.4 = 0.1773;
    # 0.96: 4 (0.2)^2.4 + 0.4^2.4 = 0.1949; 0.95: 0.243; below 0.95 the 10 loses at least 0.5 and
    # below 2/3 the 3s round to 2 s.  So p = 0.97 (candidate 3).
    g = o.ClippedMinMaxGrid(2, 5)
    g.set_params(np.array([[3.0, 3.0, 3.0, 3.0, 10.0]]))
    assert g.choice[0] == 3
    assert g.scale[0] == pytest.approx(0.97 * 10 / 3, rel=1e-15) and g.zero[0] == 0
    assert g.errors[3, 0] == pytest.approx(0.1773, abs=2e-4)
    assert g.errors[0, 0] == pytest.approx(0.2864, abs=2e-4)


def test_clip_with_one_candidate_is_the_minmax_grid():
    rng = np.random.default_rng(35)
    blk = rng.standard_normal((9, 50))
    a = o.ClippedMinMaxGrid(3, 50, maxshrink=0.01)   # only p = 1
    b = o.AsymMinMaxGrid(3, 50)
    a.set_params(blk)
    b.set_params(blk)
    np.testing.assert_array_equal(a.scale, b.scale)
    np.testing.assert_array_equal(a.zero, b.zero)


def test_clip_keeps_exactly_representable_rows_and_never_loses():
    rng = np.random.default_rng(36)
    # values on the p = 1 grid of their own range: error 0 at p = 1, which is then kept
    q = rng.integers(0, 4, size=(5, 30)).astype(float)
    q[:, 0], q[:, 1] = 0, 3
    exact = (q - 1.0) * 0.25
    g = o.ClippedMinMaxGrid(2, 30)
    g.set_params(exact)
    np.testing.assert_array_equal(g.choice, 0)
    # random rows: the chosen error never exceeds the plain grid's (p = 1 is a candidate),
    # and on Gaussian rows at 2 bits some clipping wins
    blk = rng.standard_normal((20, 256))
    g.set_params(blk)
    best = g.errors[g.choice, np.arange(20)]
    assert np.all(best <= g.errors[0])
    assert np.all(g.choice > 0)


def test_clip_is_scale_equivariant():
    # a power-of-two rescale is exact: same candidate, scale times 4, same zero and codes
    rng = np.random.default_rng(37)
    W = rng.standard_normal((7, 64)) * 0.05
    HX = spd(rng, 64)
    a = o.quantize_layer(W, HX, None, 3, 64, 0.01, act_order=True, w_clip=True)
    b = o.quantize_layer(4.0 * W, HX, None, 3, 64, 0.01, act_order=True, w_clip=True)
    np.testing.assert_array_equal(a["clip_choice"], b["clip_choice"])
    np.testing.assert_array_equal(b["gptq"].scales, 4.0 * a["gptq"].scales)
    np.testing.assert_array_equal(b["gptq"].zeros, a["gptq"].zeros)
    np.testing.assert_array_equal(b["gptq"].codes, a["gptq"].codes)


def test_clip_replay_accepts_only_near_ties():
    # another implementation's scale is adopted only when its candidate's error is within
    # the tolerance of the best one
    blk = np.array([[3.0, 3.0, 3.0, 3.0, 10.0]])
    g = o.ClippedMinMaxGrid(2, 5)
    g.set_params(blk)
    s3, s2 = g.scale[0], 0.98 * 10 / 3
    far = o.ClippedMinMaxGrid(2, 5, replay_scales=np.array([s2]))
    far.set_params(blk)      # candidate 2 is 6 % worse: kept own choice
    assert far.choice[0] == 3 and far.hard_mismatches == 1 and far.accepted_ties == 0
    near = o.ClippedMinMaxGrid(2, 5, replay_scales=np.array([s2]), tol=0.07)
    near.set_params(blk)     # within a 7 % tolerance: adopted
    assert near.choice[0] == 2 and near.accepted_ties == 1 and near.scale[0] == pytest.approx(s2)
    same = o.ClippedMinMaxGrid(2, 5, replay_scales=np.array([s3]))
    same.set_params(blk)
    assert same.choice[0] == 3 and same.hard_mismatches == 0 and same.accepted_ties == 0


# ---------------------------------------------------------------------------
# Deploy side
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out_n,in_n,bo,bi", [(32, 96, 32, 32), (48, 64, 16, 64), (8, 256, 8, 0)])
def test_deploy_undoes_biip(out_n, in_n, bo, bi):
    # an unquantized W~ = BiIP(W) in the deploy forward must give back W x: the activation's
    # rescale and rotation and the output's inverse rotation and rescale exactly undo BiIP
    rng = np.random.default_rng(out_n + in_n)
    W = rng.standard_normal((out_n, in_n))
    HX, HG = spd(rng, in_n), spd(rng, out_n)
    s_in, s_out = rng.choice([-1, 1], in_n), rng.choice([-1, 1], out_n)
    Wt, _, _, d_in, d_out = o.biip(W, HX, HG, s_in, s_out, 0.25, o.BIIP_FULL, bi, bo)
    assert np.max(np.abs(d_in - 1)) > 0.1 and np.max(np.abs(d_out - 1)) > 0.1
    x = rng.standard_normal(in_n)
    y = o.deploy_linear(Wt, d_in, d_out, s_in, s_out, bi, bo, x)
    np.testing.assert_allclose(y, W @ x, rtol=1e-10, atol=1e-10 * np.linalg.norm(W @ x))
    X = rng.standard_normal((3, in_n))
    np.testing.assert_allclose(o.deploy_linear(Wt, d_in, d_out, s_in, s_out, bi, bo, X), X @ W.T,
                               rtol=1e-10, atol=1e-9)


def test_deploy_without_processing_is_the_plain_product():
    # no rescale (d = 1), plus signs, 1-blocks (no Hadamard): y = Qhat x; and the dequantized
    # values are s (q - z) per (row, group)
    codes = np.array([[0, 1, 2, 3], [3, 2, 1, 0]])
    scales = np.array([[0.5, 2.0], [1.0, 0.25]])
    zeros = np.array([[1, 0], [2, 3]])
    Q = o.dequant(codes, scales, zeros, 2)
    np.testing.assert_array_equal(Q, [[-0.5, 0.0, 4.0, 6.0], [1.0, 0.0, -0.5, -0.75]])
    x = np.array([1.0, -2.0, 0.5, 4.0])
    y = o.deploy_linear(Q, np.ones(4), np.ones(2), np.ones(4), np.ones(2), 1, 1, x)
    np.testing.assert_array_equal(y, Q @ x)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------
def test_pack_hand_examples():
    c = np.zeros((1, 16), dtype=np.int64)
    c[0, :4] = [1, 2, 3, 0]
    assert o.pack_codes(c, 2)[0, 0] == 1 + 2 * 4 + 3 * 16          # 57
    c4 = np.zeros((1, 8), dtype=np.int64)
    c4[0, :2] = [0xF, 0x1]
    assert o.pack_codes(c4, 4)[0, 0] == 0x1F
    c4[0, 7] = 0xA
    assert o.pack_codes(c4, 4)[0, 0] == 0xA000001F
    # W3: code 10 occupies stream bits 30..32 and straddles words 0 and 1
    c3 = np.zeros((1, 32), dtype=np.int64)
    c3[0, 10] = 7
    w = o.pack_codes(c3, 3)
    assert w.shape == (1, 3)
    assert w[0, 0] == 0xC0000000 and w[0, 1] == 1 and w[0, 2] == 0
    c3[0, 31] = 5                                                 # bits 93..95 -> word 2 bits 29..31
    assert o.pack_codes(c3, 3)[0, 2] == 5 << 29


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_round_trip_and_size(bits):
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 2 ** bits, size=(5, 64))
    w = o.pack_codes(codes, bits)
    assert w.shape == (5, 64 * bits // 32)
    np.testing.assert_array_equal(o.unpack_codes(w, bits, 64), codes)
    # independent unpack through numpy's bit unpacking of little-endian words
    stream = np.unpackbits(w.astype("<u4").view(np.uint8), axis=1, bitorder="little")
    back = (stream.reshape(5, 64, bits) * (1 << np.arange(bits))).sum(-1)
    np.testing.assert_array_equal(back, codes)


# ---------------------------------------------------------------------------
# Bit allocation
# ---------------------------------------------------------------------------
def test_allocator_worked_examples():
    # gains at 2 bits are s*3/64: (3, .75, .1875, .047); after 64 -> 3 bits its gain is
    # 64*3/256 = .75, tied with 16 at 2 bits: the smallest index wins -> (4, 2, 2, 2)
    assert o.allocate_bits([64, 16, 4, 1], [1, 1, 1, 1]) == [4, 2, 2, 2]
    assert o.allocate_bits([100, 10, 1, 0.1], [1, 1, 1, 1]) == [4, 2, 2, 2]
    # budget 10 of 4 unit layers, equal sensitivities: ties go to the lowest indices
    assert o.allocate_bits([1, 1, 1, 1], [1, 1, 1, 1]) == [3, 3, 2, 2]


def test_allocator_greedy_is_optimal_for_equal_sizes():
    """For equal sizes the objective sum_l s_l 4^-b_l is separable convex with unit
    costs, so the greedy result attains the brute-force optimum under the budget."""
    rng = np.random.default_rng(18)
    for trial in range(20):
        L = int(rng.integers(2, 7))
        s = np.exp(3 * rng.standard_normal(L))
        bits = o.allocate_bits(s, [7] * L)
        budget = (7 * L * 5) // 2
        assert sum(b * 7 for b in bits) <= budget
        best = min(sum(si * 4.0 ** -bi for si, bi in zip(s, bb))
                   for bb in itertools.product((2, 3, 4), repeat=L) if 7 * sum(bb) <= budget)
        got = sum(si * 4.0 ** -bi for si, bi in zip(s, bits))
        assert got == pytest.approx(best, rel=1e-12)


def test_allocator_budget_and_monotonicity():
    rng = np.random.default_rng(19)
    numel = [4096 * 4096] * 4 + [11008 * 4096] * 3
    for trial in range(10):
        s = np.exp(2 * rng.standard_normal(7))
        bits = o.allocate_bits(s, numel)
        assert all(b in (2, 3, 4) for b in bits)
        assert sum(b * n for b, n in zip(bits, numel)) <= (sum(numel) * 5) // 2
        for a in range(4):
            for b in range(4):
                if s[a] > s[b]:
                    assert bits[a] >= bits[b]


# ---------------------------------------------------------------------------
# FlipFlop Hessian factors ([WaterKron] Table 1)
# ---------------------------------------------------------------------------
def _factorial_tokens(rng, nx, n, ng, m):
    """Every pair (x_i, g_j) of two small sets: then E[x x^T (x) g g^T] = Abar (x) Gbar."""
    xs = rng.standard_normal((nx, n)) * np.exp(rng.standard_normal(n))
    gs = rng.standard_normal((ng, m)) * np.exp(rng.standard_normal(m))
    X = np.repeat(xs, ng, axis=0)
    G = np.tile(gs, (nx, 1))
    return X, G, xs.T @ xs / nx, gs.T @ gs / ng


def test_flipflop_full_factorial_closed_form():
    """Full-factorial tokens: the iteration from B = I reaches its fixed point in one step,
    A = Abar tr(Gbar) / m and B = m Gbar / tr(Gbar) (derived by hand from the two updates)."""
    rng = np.random.default_rng(31)
    n, m = 4, 3
    X, G, Abar, Gbar = _factorial_tokens(rng, 9, n, 7, m)
    for A, B in o.flipflop(X, G, 4):
        assert np.allclose(A, Abar * np.trace(Gbar) / m, rtol=1e-12, atol=0)
        assert np.allclose(B, m * Gbar / np.trace(Gbar), rtol=1e-12, atol=0)


def test_flipflop_single_output_channel():
    """m = 1: B stays 1 and A = E[g^2 x x^T] at every iteration."""
    rng = np.random.default_rng(32)
    X = rng.standard_normal((50, 5))
    G = rng.standard_normal((50, 1)) * 3.0
    want = sum(G[t, 0] ** 2 * np.outer(X[t], X[t]) for t in range(50)) / 50
    for A, B in o.flipflop(X, G, 3):
        assert np.allclose(B, [[1.0]], rtol=1e-12)
        assert np.allclose(A, want, rtol=1e-12)


def test_flipflop_first_step_by_loops():
    """From B = I: A_1 = (1/(T m)) sum_t |g_t|^2 x_t x_t^T and B_1 from A_1, by explicit loops."""
    rng = np.random.default_rng(33)
    T, n, m = 30, 3, 4
    X, G = rng.standard_normal((T, n)), rng.standard_normal((T, m))
    A1 = np.zeros((n, n))
    for t in range(T):
        A1 += sum(G[t, j] ** 2 for j in range(m)) * np.outer(X[t], X[t])
    A1 /= T * m
    Ai = np.linalg.inv(A1)
    B1 = np.zeros((m, m))
    for t in range(T):
        B1 += sum(X[t, i] * Ai[i, k] * X[t, k] for i in range(n) for k in range(n)) * np.outer(G[t], G[t])
    B1 /= T * n
    (A, B), = o.flipflop(X, G, 1)
    assert np.allclose(A, A1, rtol=1e-12) and np.allclose(B, B1, rtol=1e-12)


def test_flipflop_objective_is_the_kronecker_fit_and_decreases():
    """The objective equals tr((A (x) B)^-1 H) + log det(A (x) B) with H = E[x x^T (x) g g^T]
    built densely; it never increases over half steps; the converged pair satisfies both
    updates and beats the marginal factors and random perturbations of itself."""
    rng = np.random.default_rng(34)
    T, n, m = 60, 3, 2
    scale_x = np.exp(rng.standard_normal(n))
    X = rng.standard_normal((T, n)) * scale_x
    G = rng.standard_normal((T, m)) * (1.0 + np.abs(X[:, :1]))   # g depends on x: H is not Kronecker
    H = sum(np.kron(np.outer(X[t], X[t]), np.outer(G[t], G[t])) for t in range(T)) / T

    def dense(A, B):
        K = np.kron(A, B)
        return float(np.trace(np.linalg.solve(K, H)) + np.linalg.slogdet(K)[1])

    A0 = np.eye(n)
    B = np.eye(m)
    prev = dense(A0, B)
    for _ in range(60):
        A = o.flipflop_input_factor(X, G, B)
        cur = dense(A, B)
        assert cur <= prev + 1e-12
        assert abs(o.flipflop_objective(X, G, A, B) - cur) < 1e-10 * max(1.0, abs(cur))
        prev = cur
        B = o.flipflop_output_factor(X, G, A)
        cur = dense(A, B)
        assert cur <= prev + 1e-12
        prev = cur
    assert np.allclose(o.flipflop_input_factor(X, G, B), A, rtol=1e-9)
    assert np.allclose(o.flipflop_output_factor(X, G, A), B, rtol=1e-9)
    Am, Bm = X.T @ X / T, G.T @ G / T
    best_marginal = min(dense(Am * c, Bm) for c in np.geomspace(1e-3, 1e3, 61))
    assert prev < best_marginal
    for _ in range(20):
        Pa = rng.standard_normal((n, n)) * 1e-3
        Pb = rng.standard_normal((m, m)) * 1e-3
        assert dense(A + Pa @ Pa.T + 1e-4 * np.eye(n), B) >= prev - 1e-12
        assert dense(A, B + Pb @ Pb.T + 1e-4 * np.eye(m)) >= prev - 1e-12


def test_flipflop_dead_channel_counts_as_one():
    """A channel whose activations are all zero: its row and column of A are zero and its
    diagonal counts as 1 in the inverse, so the other channels see the same weights as if it
    were absent."""
    rng = np.random.default_rng(35)
    T, n, m = 40, 4, 3
    X = rng.standard_normal((T, n))
    X[:, 2] = 0.0
    G = rng.standard_normal((T, m))
    (A, B), = o.flipflop(X, G, 1)
    (A3, B3), = o.flipflop(np.delete(X, 2, axis=1), G, 1)
    assert np.all(A[2] == 0) and np.all(A[:, 2] == 0)
    keep = [0, 1, 3]
    assert np.allclose(A[np.ix_(keep, keep)], A3, rtol=1e-12)
    # B is divided by n: the dead channel still counts in the dimension
    assert np.allclose(B * n, B3 * (n - 1), rtol=1e-12)


# ---------------------------------------------------------------------------
# Two-sided rounding ([BaKron] abstract: GPTQ in the vectorized weight domain)
# ---------------------------------------------------------------------------
class _StaticGrid:
    """A grid for o.gptq whose parameters are fixed per (row of its input, column)."""

    def __init__(self, scale_of_col, zero_of_col, bits):
        self.S, self.Z, self.maxq, self.group = scale_of_col, zero_of_col, (1 << bits) - 1, 1

    def starts_group(self, j):
        self.j = j
        return True

    def set_params(self, block):
        self.scale, self.zero = self.S[:, self.j], self.Z[:, self.j]

    def unrounded(self, w):
        return w / self.scale

    def code(self, u):
        return np.clip(np.rint(u) + self.zero, 0, self.maxq)

    def dequant(self, q):
        return self.scale * (q - self.zero)


def _two_sided_case(seed, m=12, n=20, corr=True):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((m, n)) * 0.1
    A = rng.standard_normal((60, n)) * np.exp(0.5 * rng.standard_normal(n))
    B = rng.standard_normal((50, m)) * np.exp(0.5 * rng.standard_normal(m))
    if corr:
        A[:, 1] += A[:, 0]
        B[:, 2] -= 0.8 * B[:, 1]
    return W, A.T @ A, B.T @ B


def _per_element(scales, zeros, group, n):
    g = np.arange(n) // group
    return scales[:, g], zeros[:, g]


def test_two_sided_with_identity_output_factor_is_row_gptq():
    """H_G = I: no feedback across rows, so every row is one-sided GPTQ with U_X (static grid)."""
    W, HX, _ = _two_sided_case(51)
    m, n = W.shape
    res = o.two_sided_gptq(W, HX, np.eye(m), 3, 4, damp=0.01)
    UX = o.damp_and_factor(HX, 0.01)[0]
    S, Z = _per_element(res.scales, res.zeros, 4, n)
    for r in range(m):
        g = o.gptq(W[r:r + 1], UX, _StaticGrid(S[r:r + 1], Z[r:r + 1], 3))
        assert np.array_equal(g.codes[0], res.codes[r])
        assert np.allclose(g.qhat[0], res.qhat[r], rtol=0, atol=1e-12)


def test_two_sided_with_identity_input_factor_is_column_gptq():
    """H_X = I: every column is GPTQ over the output channels with U_G."""
    W, _, HG = _two_sided_case(52)
    m, n = W.shape
    res = o.two_sided_gptq(W, np.eye(n), HG, 4, 5, damp=0.02)
    UG = o.damp_and_factor(HG, 0.02)[0]
    S, Z = _per_element(res.scales, res.zeros, 5, n)
    for i in range(n):
        g = o.gptq(W[:, i:i + 1].T, UG, _StaticGrid(S[:, i:i + 1].T, Z[:, i:i + 1].T, 4))
        assert np.array_equal(g.codes[0], res.codes[:, i])


def test_two_sided_with_identity_factors_is_rtn():
    W, _, _ = _two_sided_case(53)
    m, n = W.shape
    res = o.two_sided_gptq(W, np.eye(n), np.eye(m), 2, n)
    S, Z = _per_element(res.scales, res.zeros, n, n)
    assert np.array_equal(res.codes, np.clip(np.rint(W / S) + Z, 0, 3))


@pytest.mark.parametrize("order", ["antidiagonal", "rows"])
def test_two_sided_is_gptq_on_vec_w_in_any_dependency_order(order):
    """Rounding vec(W) through the explicit U = kron(U_X, U_G) in another order that respects
    the dependencies (anti-diagonals r + i, or row-major) gives the same codes: the feedback
    of (r, i) reaches exactly the coordinates (r' >= r, i' >= i)."""
    W, HX, HG = _two_sided_case(54, m=6, n=9)
    m, n = W.shape
    res = o.two_sided_gptq(W, HX, HG, 3, 3, damp=0.01)
    UX = o.damp_and_factor(HX, 0.01)[0]
    UG = o.damp_and_factor(HG, 0.01)[0]
    U = np.kron(UX, UG)                      # index c = i m + r
    w = W.T.reshape(-1).copy()
    S, Z = _per_element(res.scales, res.zeros, 3, n)
    coords = [(r, i) for i in range(n) for r in range(m)]
    key = (lambda c: (c[0] + c[1], c[0])) if order == "antidiagonal" else (lambda c: (c[0], c[1]))
    done = np.zeros(m * n, dtype=bool)
    codes = np.zeros((m, n), dtype=np.int64)
    for r, i in sorted(coords, key=key):
        c = i * m + r
        q = np.clip(np.rint(w[c] / S[r, i]) + Z[r, i], 0, 7)
        e = (w[c] - S[r, i] * (q - Z[r, i])) / U[c, c]
        done[c] = True
        w[~done] -= e * U[c, ~done]
        codes[r, i] = q
    assert np.array_equal(codes, res.codes)
