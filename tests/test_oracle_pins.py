"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these retypes the oracle's formulas: each compares it with a
different route to the same value (an SVD, a library polar decomposition,
a library AdamW, a brute-force sum, a number the pages print) so that a
dropped term, a wrong sign or index, or a transposed operand fails one of
them.
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
CFG = oracle.OracleConfig()
A5, B5, C5 = 3.4445, -4.7750, 2.0315


def _rng(seed):
    return np.random.default_rng(seed)


def phi(x, a=A5, b=B5, c=C5, iters=5):
    """The scalar quintic p(x) = a x + b x^3 + c x^5 composed iters times."""
    x = np.asarray(x, dtype=np.float64)
    for _ in range(iters):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def ns_via_svd(M, a=A5, b=B5, c=C5, iters=5, eps=1e-7):
    """Closed form of the matrix iteration: it acts on singular values alone."""
    M = np.asarray(M, dtype=np.float64)
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    scale = np.linalg.norm(M) + eps
    return (U * phi(s / scale, a, b, c, iters)) @ Vt


# ------------------------------------------------------------------ schedule
def test_schedule_numbers_printed_on_pages():
    g = json.load(open(os.path.join(GOLD, "schedule_pages.json")))
    K = g["default_K"]["value"]
    assert CFG.K == K and CFG.gamma == g["default_gamma"]["value"]
    # one refresh and K-1 RowNorm steps per cycle
    br = [oracle.branch(t, CFG) for t in range(4 * K)]
    assert br.count(oracle.BRANCH_NS5) == 4
    assert br.count(oracle.BRANCH_ROWNORM) == 4 * (K - 1)

    def refresh_fraction(k, T=1200):
        return sum(oracle.refresh_indicator(t, k) for t in range(T)) / T

    for case in g["k_ablation"]["cases"]:
        cut = 100 * (1 - refresh_fraction(case["to_K"]) / refresh_fraction(case["from_K"]))
        assert round(cut) == case["refresh_reduction_pct"]
    # Eq. (9) cycle average of the per-step volume with zero RowNorm traffic
    v = g["comm_volume_gib_per_rank_step"]
    steps = range(3 * 100)
    avg = sum(v["vanilla"] if oracle.refresh_indicator(t, K) else 0.0 for t in steps) / len(steps)
    assert abs(avg - v["periodic"]) < 0.005
    assert abs(100 * (1 - avg / v["vanilla"]) - g["logical_comm_reduction_pct"]["value"]) < 0.05


def test_branch_indexing_and_degenerate_K():
    assert [oracle.branch(t, CFG) for t in range(6)] == [1, 0, 0, 1, 0, 0]
    vanilla = oracle.OracleConfig(K=1)
    assert all(oracle.branch(t, vanilla) == oracle.BRANCH_NS5 for t in range(10))
    bp = oracle.OracleConfig(bp_blocks=8, bp_period=3)
    assert [oracle.branch(t, bp) for t in range(6)] == [1, 2, 2, 1, 2, 2]
    with pytest.raises(ValueError):
        oracle.refresh_indicator(-1, 3)
    with pytest.raises(ValueError):
        oracle.refresh_indicator(0, 0)


# ------------------------------------------------------------------ momentum
def test_momentum_constant_gradient_closed_form():
    G = _rng(0).standard_normal((5, 7))
    M = np.zeros_like(G)
    for t in range(20):
        M = oracle.momentum_update(M, G, 0.95)
        np.testing.assert_allclose(M, G * (1 - 0.95 ** (t + 1)) / (1 - 0.95), rtol=1e-13)


def test_momentum_equals_discounted_sum():
    rng = _rng(1)
    Gs = [rng.standard_normal((3, 4)) for _ in range(9)]
    M = np.zeros((3, 4))
    for t, G in enumerate(Gs):
        M = oracle.momentum_update(M, G, 0.9)
        brute = np.zeros((3, 4))
        for s in range(t + 1):
            brute += 0.9 ** (t - s) * Gs[s]
        np.testing.assert_allclose(M, brute, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ NS5
@pytest.mark.parametrize("shape", [(8, 8), (6, 17), (17, 6), (32, 96), (96, 32), (64, 64), (1, 9), (9, 1)])
def test_ns5_matches_svd_closed_form(shape):
    M = _rng(hash(shape) % 1000).standard_normal(shape)
    np.testing.assert_allclose(oracle.newton_schulz(M), ns_via_svd(M), atol=5e-13)


def test_ns5_rank_deficient_and_zero():
    rng = _rng(2)
    M = rng.standard_normal((12, 3)) @ rng.standard_normal((3, 20))  # rank 3
    np.testing.assert_allclose(oracle.newton_schulz(M), ns_via_svd(M), atol=5e-13)
    Z = np.zeros((4, 9))
    assert not np.any(oracle.newton_schulz(Z))


def test_ns5_spectrum_band_and_shared_singular_vectors():
    """NS5(M) = U phi(Sigma/s) V^T: same singular vectors as the polar factor
    U V^T, singular values in the quintic's band once converged."""
    M = _rng(3).standard_normal((48, 160))
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    Y = oracle.newton_schulz(M)
    D = U.T @ Y @ Vt.T
    off = D - np.diag(np.diag(D))
    assert np.max(np.abs(off)) < 1e-12
    x = s / (np.linalg.norm(M) + 1e-7)
    np.testing.assert_allclose(np.diag(D), phi(x), atol=1e-12)
    conv = x >= 1.505e-3
    assert np.all(np.diag(D)[conv] > 0.68) and np.all(np.diag(D)[conv] < 1.21)
    # the approximation is not the polar factor itself
    P = U @ Vt
    assert 0.01 < np.linalg.norm(Y - P) / np.linalg.norm(P) < 0.5


def test_textbook_quintic_reaches_library_polar_factor():
    """With the convergent quintic (15/8, -5/4, 3/8) the same iteration must
    reproduce the polar factor of a well-conditioned matrix."""
    rng = _rng(4)
    for shape in [(10, 30), (30, 10), (16, 16)]:
        r = min(shape)
        Q1, _ = np.linalg.qr(rng.standard_normal((shape[0], r)))
        Q2, _ = np.linalg.qr(rng.standard_normal((shape[1], r)))
        M = (Q1 * np.linspace(0.5, 1.0, r)) @ Q2.T
        Y = oracle.newton_schulz(M, iters=40, a=15 / 8, b=-5 / 4, c=3 / 8, eps=0.0)
        u, _ = scipy.linalg.polar(M, side="right")
        np.testing.assert_allclose(Y, u, atol=1e-12)


def test_ns5_tiny_closed_forms():
    rng = _rng(5)
    # single row: phi(||x||/(||x||+eps)) x/||x||
    x = rng.standard_normal((1, 11))
    nx = np.linalg.norm(x)
    np.testing.assert_allclose(oracle.newton_schulz(x), phi(nx / (nx + 1e-7)) * x / nx, atol=1e-14)
    # c Q with orthonormal rows: phi(c / (c sqrt(r) + eps)) Q
    r, n, c = 4, 10, 3.0
    Q = np.linalg.qr(rng.standard_normal((n, r)))[0].T
    np.testing.assert_allclose(oracle.newton_schulz(c * Q),
                               phi(c / (c * np.sqrt(r) + 1e-7)) * Q, atol=1e-13)
    # diagonal
    d = np.array([3.0, 1.0, 0.5, 0.25])
    np.testing.assert_allclose(oracle.newton_schulz(np.diag(d)),
                               np.diag(phi(d / (np.linalg.norm(d) + 1e-7))), atol=1e-14)


def test_ns5_transpose_and_orthogonal_covariance():
    rng = _rng(6)
    M = rng.standard_normal((7, 19))
    np.testing.assert_allclose(oracle.newton_schulz(M.T), oracle.newton_schulz(M).T, atol=1e-13)
    Q = np.linalg.qr(rng.standard_normal((7, 7)))[0]
    P = np.linalg.qr(rng.standard_normal((19, 19)))[0]
    np.testing.assert_allclose(oracle.newton_schulz(Q @ M @ P),
                               Q @ oracle.newton_schulz(M) @ P, atol=1e-12)


# ------------------------------------------------------------------ RowNorm
def test_rownorm_unit_zero_and_subthreshold_rows():
    M = _rng(7).standard_normal((6, 20))
    M[2] = 0.0
    M[4] *= 1e-10                       # norm below eps = 1e-8
    R = oracle.row_normalize(M, 1e-8)
    norms = np.linalg.norm(R, axis=1)
    for i in (0, 1, 3, 5):
        assert abs(norms[i] - 1.0) < 1e-14
    assert not np.any(R[2])
    np.testing.assert_allclose(R[4], M[4] / 1e-8, rtol=1e-14)


def test_rownorm_long_axis_for_tall_matrices():
    M = _rng(8).standard_normal((40, 9))       # tall: columns are the long axis
    R = oracle.row_normalize(M, 1e-8, 0)
    np.testing.assert_allclose(np.linalg.norm(R, axis=0), 1.0, atol=1e-14)
    np.testing.assert_allclose(R, M / np.linalg.norm(M, axis=0, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(oracle.row_normalize(M.T, 1e-8, 0), R.T, rtol=1e-14)
    # stored-row mode normalises rows of every shape
    R1 = oracle.row_normalize(M, 1e-8, 1)
    np.testing.assert_allclose(np.linalg.norm(R1, axis=1), 1.0, atol=1e-14)


def test_frobenius_sqrt_r_from_pages():
    g = json.load(open(os.path.join(GOLD, "frobenius_pages.json")))
    rng = _rng(9)
    for m, n in g["cases"]:
        M = rng.standard_normal((m, n))
        r = min(m, n)
        assert abs(np.linalg.norm(oracle.row_normalize(M)) - np.sqrt(r)) < 1e-12
        u = scipy.linalg.polar(M, side="right")[0]
        assert abs(np.linalg.norm(u) - np.sqrt(r)) < 1e-10


def test_rownorm_scale_invariance():
    M = _rng(10).standard_normal((5, 12))
    np.testing.assert_allclose(oracle.row_normalize(37.5 * M), oracle.row_normalize(M), rtol=1e-14)


def test_eq8_row_shard_statistics():
    """Paper Eq. (8): per-shard column sums of squares add up to the global
    column norm that normalises a tall matrix."""
    X = _rng(11).standard_normal((103, 17))
    perm = _rng(12).permutation(103)
    shards = [perm[:10], perm[10:50], perm[50:51], perm[51:]]
    nu = oracle.column_norms_from_row_shards(X, shards)
    np.testing.assert_allclose(nu, np.linalg.norm(X, axis=0), rtol=1e-14)
    np.testing.assert_allclose(oracle.row_normalize(X), X / nu, rtol=1e-14)


# ------------------------------------------------------------------ full step
def test_direction_per_branch_and_weight_accumulation():
    rng = _rng(13)
    for shape in [(16, 40), (40, 16)]:
        W0 = rng.standard_normal(shape) * 0.02
        W, M = W0.copy(), np.zeros(shape)
        Us, Mref = [], np.zeros(shape)
        for t in range(6):
            G = rng.standard_normal(shape)
            W, M, U = oracle.muon_matrix_step(W, M, G, t, CFG)
            Mref = 0.95 * Mref + G
            if t % 3 == 0:
                np.testing.assert_allclose(U, ns_via_svd(Mref), atol=1e-12)
            else:
                long_axis = 0 if shape[0] > shape[1] else 1
                np.testing.assert_allclose(np.linalg.norm(U, axis=long_axis), CFG.gamma, rtol=1e-13)
                np.testing.assert_allclose(np.sign(U), np.sign(Mref))
            Us.append(U)
        np.testing.assert_allclose(W, W0 - CFG.lr * np.sum(Us, axis=0), atol=1e-15)


def test_weight_decay_term():
    cfg = oracle.OracleConfig(muon_wd=0.1)
    rng = _rng(14)
    W, G = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    Wn, _, U = oracle.muon_matrix_step(W, np.zeros_like(W), G, 1, cfg)
    np.testing.assert_allclose(Wn, W * (1 - cfg.lr * 0.1) - cfg.lr * U, rtol=1e-14)


# ------------------------------------------------------------------ MuonBP
def test_muonbp_single_block_equals_vanilla_muon():
    rng = _rng(15)
    bp = oracle.OracleConfig(bp_blocks=1, bp_period=3, bp_lr_ratio=1.0)
    van = oracle.OracleConfig(K=1)
    W1 = W2 = rng.standard_normal((12, 20)) * 0.02
    M1 = M2 = np.zeros((12, 20))
    for t in range(5):
        G = rng.standard_normal((12, 20))
        W1, M1, _ = oracle.muon_matrix_step(W1, M1, G, t, bp)
        W2, M2, _ = oracle.muon_matrix_step(W2, M2, G, t, van)
    np.testing.assert_allclose(W1, W2, atol=1e-15)


def test_muonbp_blocks_are_independent_ns5():
    cfg = oracle.OracleConfig(bp_blocks=4, bp_period=3, bp_lr_ratio=0.5)
    M = _rng(16).standard_normal((24, 32))
    U, lr = oracle.direction(M, 1, cfg)
    assert lr == cfg.lr * 0.5
    for j in range(4):
        np.testing.assert_allclose(U[:, 8 * j:8 * j + 8], ns_via_svd(M[:, 8 * j:8 * j + 8]), atol=1e-12)
    Uf, lrf = oracle.direction(M, 3, cfg)
    assert lrf == cfg.lr
    np.testing.assert_allclose(Uf, ns_via_svd(M), atol=1e-12)
    with pytest.raises(ValueError):
        oracle.block_newton_schulz(M, 5)


# ------------------------------------------------------------------ AdamW
@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_adamw_matches_library(wd):
    cfg = oracle.OracleConfig(adam_lr=3e-3, adam_wd=wd)
    rng = _rng(17)
    p0 = rng.standard_normal(50)
    p = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=cfg.adam_lr, betas=(cfg.adam_b1, cfg.adam_b2),
                            eps=cfg.adam_eps, weight_decay=wd)
    q, m, v = p0.copy(), np.zeros(50), np.zeros(50)
    for t in range(7):
        g = rng.standard_normal(50)
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        q, m, v = oracle.adamw_step(q, g, m, v, t, cfg)
    np.testing.assert_allclose(q, p.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_constant_gradient_is_signed_step():
    cfg = oracle.OracleConfig(adam_lr=1e-2, adam_eps=0.0)
    g = np.array([2.0, -0.5, 1e-3])
    p, m, v = np.zeros(3), np.zeros(3), np.zeros(3)
    for t in range(4):
        p, m, v = oracle.adamw_step(p, g, m, v, t, cfg)
        np.testing.assert_allclose(p, -cfg.adam_lr * (t + 1) * np.sign(g), rtol=1e-12)


# ------------------------------------------------------------------ whole parameter list
def test_oracle_step_on_a_mixed_list():
    """oracle_step over a list that mixes a wide and a tall Muon matrix with
    two AdamW vectors, for two K-cycles.  Each entry is checked against a
    route that does not go through the oracle: the matrices against the
    discounted gradient sum put through the SVD closed form (refresh steps)
    or divided by its long-axis slice norms (RowNorm steps), the vectors
    against torch.optim.AdamW; the returned state keeps the per-entry kind
    (momentum array, or the AdamW (m, v) pair in that order)."""
    rng = _rng(19)
    cfg = oracle.OracleConfig(adam_lr=2e-3, adam_wd=0.01)
    shapes = [(9, 21), None, (30, 8), None]
    kinds = ["matrix", "adamw", "matrix", "adamw"]
    sizes = {1: 13, 3: 40}
    params = [rng.standard_normal(s) * 0.02 if k == "matrix" else rng.standard_normal(sizes[i])
              for i, (s, k) in enumerate(zip(shapes, kinds))]
    state = [np.zeros(s) if k == "matrix" else (np.zeros(sizes[i]), np.zeros(sizes[i]))
             for i, (s, k) in enumerate(zip(shapes, kinds))]
    torch_p = {i: torch.tensor(params[i], dtype=torch.float64, requires_grad=True) for i in sizes}
    opts = {i: torch.optim.AdamW([torch_p[i]], lr=cfg.adam_lr, betas=(cfg.adam_b1, cfg.adam_b2),
                                 eps=cfg.adam_eps, weight_decay=cfg.adam_wd) for i in sizes}
    W0 = [p.copy() for p in params]
    gsum = {0: [], 2: []}
    for t in range(2 * cfg.K):
        grads = [rng.standard_normal(s) if k == "matrix" else rng.standard_normal(sizes[i])
                 for i, (s, k) in enumerate(zip(shapes, kinds))]
        before = [np.copy(p) for p in params]
        params, state = oracle.oracle_step(params, grads, state, kinds, t, cfg)
        for i in sizes:
            torch_p[i].grad = torch.tensor(grads[i], dtype=torch.float64)
            opts[i].step()
            np.testing.assert_allclose(params[i], torch_p[i].detach().numpy(), rtol=1e-13, atol=1e-15)
            # (m, v) in that order: discounted sums of the gradients and of their squares
            gsum.setdefault(i, []).append(grads[i])
            m_ref = sum((1 - cfg.adam_b1) * cfg.adam_b1 ** (t - s) * g for s, g in enumerate(gsum[i]))
            v_ref = sum((1 - cfg.adam_b2) * cfg.adam_b2 ** (t - s) * g * g
                        for s, g in enumerate(gsum[i]))
            np.testing.assert_allclose(state[i][0], m_ref, rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(state[i][1], v_ref, rtol=1e-12, atol=1e-15)
        for i in (0, 2):
            gsum[i].append(grads[i])
            Mref = sum(0.95 ** (t - s) * g for s, g in enumerate(gsum[i]))
            np.testing.assert_allclose(state[i], Mref, rtol=1e-12, atol=1e-14)
            U = (before[i] - params[i]) / cfg.lr
            if t % cfg.K == 0:
                np.testing.assert_allclose(U, ns_via_svd(Mref), atol=1e-12)
            else:
                axis = 0 if shapes[i][0] > shapes[i][1] else 1
                norms = np.linalg.norm(Mref, axis=axis, keepdims=True)
                np.testing.assert_allclose(U, cfg.gamma * Mref / norms, rtol=1e-12, atol=1e-15)
    for i in (0, 2):
        assert not np.allclose(params[i], W0[i])
    # the inputs are not modified
    p_in = [np.ones((3, 5)), np.ones(4)]
    s_in = [np.zeros((3, 5)), (np.zeros(4), np.zeros(4))]
    oracle.oracle_step(p_in, [np.ones((3, 5)), np.ones(4)], s_in, ["matrix", "adamw"], 1, cfg)
    assert np.all(p_in[0] == 1) and np.all(s_in[0] == 0) and np.all(s_in[1][0] == 0)


# ------------------------------------------------------------------ planted mistakes
def test_pins_catch_planted_mistakes():
    """Mistakes planted in copies of the oracle's arithmetic are caught by
    the pins above: the NS5 variants by the SVD closed form, the RowNorm
    variants by the pages' sqrt(r) Frobenius norm, the long-axis unit norms
    and the Eq. (8) column statistics."""
    rng = _rng(18)
    M = rng.standard_normal((12, 30))
    S = rng.standard_normal((16, 16))          # square: transposed operands type-check

    def ns_variant(M, swap=False, iters=5, sign=1.0, normalise=True, right=False, gram_t=False):
        X = M / (np.linalg.norm(M) + 1e-7) if normalise else M
        for _ in range(iters):
            A = X.T @ X if gram_t else X @ X.T
            B = (C5 * A + B5 * (A @ A)) if swap else (B5 * A + sign * C5 * (A @ A))
            X = A5 * X + (X @ B if right else B @ X)
        return X

    for inp in (M, S):
        assert np.allclose(ns_variant(inp), ns_via_svd(inp), atol=1e-12)
    for inp, kw in [(M, dict(swap=True)), (M, dict(iters=4)), (M, dict(sign=-1.0)),
                    (M, dict(normalise=False)), (S, dict(right=True)), (S, dict(gram_t=True))]:
        with np.errstate(all="ignore"):
            bad = ns_variant(inp, **kw)
        assert not np.allclose(bad, ns_via_svd(inp), atol=1e-3), kw

    # RowNorm of a tall matrix along the wrong (stored-row) axis, without the
    # eps floor's max, or with the norm squared
    T = rng.standard_normal((40, 9))
    r = min(T.shape)

    def rn_variant(X, axis=0, floor=True, power=0.5):
        s = np.sum(X * X, axis=axis, keepdims=True) ** power
        return X / (np.maximum(s, 1e-8) if floor else s)

    def pins_hold(R, X):
        unit = np.allclose(np.linalg.norm(R, axis=0), 1.0, atol=1e-12)
        frob = abs(np.linalg.norm(R) - np.sqrt(r)) < 1e-12
        nu = oracle.column_norms_from_row_shards(X, [np.arange(0, 17), np.arange(17, 40)])
        eq8 = np.allclose(R, X / nu, rtol=1e-12)
        return unit and frob and eq8

    assert pins_hold(rn_variant(T), T) and pins_hold(oracle.row_normalize(T), T)
    for kw in (dict(axis=1), dict(power=1.0)):
        assert not pins_hold(rn_variant(T, **kw), T), kw
    Z = T.copy()
    Z[:, 4] = 0.0
    with np.errstate(all="ignore"):
        no_floor = rn_variant(Z, floor=False)
    assert not np.all(np.isfinite(no_floor))          # the zero-slice pin fails
    assert not np.any(oracle.row_normalize(Z)[:, 4])
