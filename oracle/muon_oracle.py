"""Plain fp64 CPU oracle for the Periodic Row-wise Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code, tables or constants with the HIP
library: every number it uses is either an argument or a default written out
here from the pages' text.

Sources (each function names the passage it follows):

* "Scaling Muon for Diffusion Transformers" (paperdance.org card), English
  abstract: momentum is materialised in full; a full NS5 spectral update every
  K steps and a row-wise constrained update of the current momentum on the
  other steps.
* PaperDaily post on the same paper ("告别每步都算谱分解！Meta让Muon在15B
  DiT上跑出性价比"):
    - section "周期性行式Muon" (Periodic Row-wise Muon), blog fig. 3: the
      update rule with refresh indicator rho_t (NS5 when t is a multiple of K,
      gamma times RowNorm otherwise, both acting on the current momentum);
      blog fig. 4: RowNorm divides row i by max(||X_i:||, eps);
      text under fig. 3: NS5 approximates the polar factor without an SVD
      using five rounds of matrix products and scaling; both maps have
      Frobenius norm sqrt(r); defaults K=3, gamma=0.15.
    - section "分布式协同设计" (distributed co-design), paper Eq. (8) / blog
      fig. 8: for tall (m>n) matrices the normalising statistic is a column
      sum of squares over rows, i.e. the norm is taken along the long axis.
    - section "从1.3B到15B": biases and normalisation parameters stay on AdamW.
* "MuonBP: Faster Muon via Block-Periodic Orthogonalization", English
  abstract: orthogonalise each shard (block) independently, run a full
  orthogonalisation periodically, with separate step sizes for the two.

Readings where the pages are silent (each one is a parameter here):
* NS5 polynomial coefficients (a, b, c) = (3.4445, -4.7750, 2.0315), 5
  iterations, X0 = X / (||X||_F + 1e-7): the Muon reference the post cites
  (Muon: an optimizer for hidden layers in neural networks, 2024).  The pages
  name NS5 but print no coefficients.
* Tall matrices (m > n) are orthogonalised in their transposed (wide)
  orientation; square counts as wide.
* RowNorm normalises slices of the long axis (rows if m <= n, columns if
  m > n); ``rownorm_axis=1`` selects stored rows for every shape instead.
* No Nesterov, no shape-dependent learning-rate scale, Muon weight decay 0.
* t starts at 0, so t = 0 is a refresh step.
* MuonBP: ``bp_blocks`` equal contiguous splits of the stored column axis;
  full NS5 when t mod ``bp_period`` == 0 with ``lr``; otherwise each block is
  orthogonalised on its own with ``lr * bp_lr_ratio``.
* AdamW: decoupled weight decay with bias correction by (t + 1).
"""

from __future__ import annotations

import dataclasses

import numpy as np

BRANCH_ROWNORM = 0
BRANCH_NS5 = 1
BRANCH_BLOCK_NS5 = 2


@dataclasses.dataclass
class OracleConfig:
    lr: float = 0.02
    beta: float = 0.95
    gamma: float = 0.15
    eps_row: float = 1e-8
    K: int = 3
    ns_iters: int = 5
    ns_a: float = 3.4445
    ns_b: float = -4.7750
    ns_c: float = 2.0315
    ns_eps: float = 1e-7
    rownorm_axis: int = 0          # 0: long axis, 1: stored rows
    bp_blocks: int = 0             # 0: MuonBP off
    bp_period: int = 3
    bp_lr_ratio: float = 0.5
    muon_wd: float = 0.0
    adam_lr: float = 1e-3
    adam_b1: float = 0.9
    adam_b2: float = 0.999
    adam_eps: float = 1e-8
    adam_wd: float = 0.0


# ---------------------------------------------------------------- schedule
def refresh_indicator(t: int, K: int) -> bool:
    """rho_t: true exactly when t is a multiple of K.

    PaperDaily post, section "Periodic Row-wise Muon", blog fig. 3.
    """
    if K < 1 or t < 0:
        raise ValueError("need K >= 1 and t >= 0")
    return t % K == 0


def branch(t: int, cfg: OracleConfig) -> int:
    """Which direction map step t uses.

    Without MuonBP: NS5 on refresh steps, RowNorm otherwise (PaperDaily post,
    blog fig. 3).  With MuonBP: a full orthogonalisation every ``bp_period``
    steps and block-wise orthogonalisation on the others (MuonBP abstract).
    """
    if cfg.bp_blocks > 0:
        return BRANCH_NS5 if refresh_indicator(t, cfg.bp_period) else BRANCH_BLOCK_NS5
    return BRANCH_NS5 if refresh_indicator(t, cfg.K) else BRANCH_ROWNORM


# ---------------------------------------------------------------- momentum
def momentum_update(M: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """M <- beta * M + G, kept explicitly for every 2-D weight.

    "Scaling Muon for Diffusion Transformers", abstract (full-momentum
    materialisation); PaperDaily post, blog fig. 3 (maps act on the current
    momentum).
    """
    return beta * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)


# ---------------------------------------------------------------- NS5
def newton_schulz(M: np.ndarray, iters: int = 5, a: float = 3.4445,
                  b: float = -4.7750, c: float = 2.0315,
                  eps: float = 1e-7) -> np.ndarray:
    """Newton-Schulz approximation of the polar factor of M.

    PaperDaily post, section "Periodic Row-wise Muon" (text under blog fig. 3):
    NS5 corrects the momentum towards an approximately orthogonal direction
    with five rounds of matrix products and scaling, no SVD.  The iteration is
    run on the wide orientation (r x c, r <= c) so the Gram matrix is r x r,
    which is what the Theta(5 r^2 c) cost in the post's review section implies.

        X  <- X / (||X||_F + eps)
        repeat iters times:
            A <- X X^T
            B <- b A + c A A
            X <- a X + B X
    """
    M = np.asarray(M, dtype=np.float64)
    tall = M.shape[0] > M.shape[1]
    X = M.T if tall else M
    X = X / (np.linalg.norm(X) + eps)
    for _ in range(iters):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T.copy() if tall else X


# ---------------------------------------------------------------- RowNorm
def row_normalize(M: np.ndarray, eps: float = 1e-8, axis_mode: int = 0) -> np.ndarray:
    """RowNorm_eps: each row divided by max(||row||_2, eps).

    PaperDaily post, blog fig. 4 (the RowNorm formula).  ``axis_mode`` 0 takes
    the rows of the wide orientation, so a tall (m > n) matrix is normalised
    per column: paper Eq. (8) (blog fig. 8, section "distributed co-design")
    builds exactly that statistic, a column sum of squares over the rows.
    ``axis_mode`` 1 normalises stored rows for every shape.
    """
    M = np.asarray(M, dtype=np.float64)
    if axis_mode == 0 and M.shape[0] > M.shape[1]:
        return row_normalize(M.T, eps, 1).T.copy()
    norms = np.sqrt(np.sum(M * M, axis=1, keepdims=True))
    return M / np.maximum(norms, eps)


def column_norms_from_row_shards(X: np.ndarray, shards) -> np.ndarray:
    """nu_j = sqrt(sum_p q_j^(p)), q_j^(p) = sum_{i in S_p} X_ij^2.

    Paper Eq. (8) (blog fig. 8): each owner of a row set S_p forms the column
    sums of squares of its rows; their sum is the global column norm.
    ``shards`` is a list of row-index arrays that partition the rows.
    """
    X = np.asarray(X, dtype=np.float64)
    q = [np.sum(X[np.asarray(S)] ** 2, axis=0) for S in shards]
    return np.sqrt(np.sum(q, axis=0))


# ---------------------------------------------------------------- MuonBP
def block_newton_schulz(M: np.ndarray, blocks: int, **ns) -> np.ndarray:
    """Orthogonalise each of ``blocks`` equal column splits independently.

    MuonBP abstract: each device-local shard is orthogonalised on its own.
    The shards are read as equal contiguous splits of the stored column axis.
    """
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[1]
    if blocks < 1 or n % blocks:
        raise ValueError("columns must split evenly into blocks")
    w = n // blocks
    return np.concatenate(
        [newton_schulz(M[:, j * w:(j + 1) * w], **ns) for j in range(blocks)], axis=1)


# ---------------------------------------------------------------- one matrix
def _ns_kwargs(cfg: OracleConfig) -> dict:
    return dict(iters=cfg.ns_iters, a=cfg.ns_a, b=cfg.ns_b, c=cfg.ns_c, eps=cfg.ns_eps)


def direction(M: np.ndarray, t: int, cfg: OracleConfig):
    """U_t and its learning rate for one momentum matrix at step t.

    PaperDaily post, blog fig. 3: rho_t NS5(M) + (1 - rho_t) gamma RowNorm(M)
    with the Muon learning rate for both; MuonBP abstract for the block branch
    and its second step size.
    """
    br = branch(t, cfg)
    if br == BRANCH_NS5:
        return newton_schulz(M, **_ns_kwargs(cfg)), cfg.lr
    if br == BRANCH_BLOCK_NS5:
        return block_newton_schulz(M, cfg.bp_blocks, **_ns_kwargs(cfg)), cfg.lr * cfg.bp_lr_ratio
    return cfg.gamma * row_normalize(M, cfg.eps_row, cfg.rownorm_axis), cfg.lr


def muon_matrix_step(W: np.ndarray, M: np.ndarray, G: np.ndarray, t: int,
                     cfg: OracleConfig):
    """One optimizer step of a 2-D weight: returns (W_new, M_new, U_t).

    Momentum, then the branch direction on the current momentum, then
    W <- W - lr * U_t (minus lr * wd * W when weight decay is set).
    """
    M_new = momentum_update(M, G, cfg.beta)
    U, lr = direction(M_new, t, cfg)
    W = np.asarray(W, dtype=np.float64)
    W_new = W - lr * U
    if cfg.muon_wd:
        W_new = W_new - lr * cfg.muon_wd * W
    return W_new, M_new, U


# ---------------------------------------------------------------- AdamW
def adamw_step(p, g, m, v, t: int, cfg: OracleConfig):
    """AdamW with decoupled weight decay (the post's reference [3]).

    The post's section "从1.3B到15B" keeps non-matrix parameters (biases,
    normalisation scales) on AdamW.  Bias correction uses step count t + 1.
    Returns (p_new, m_new, v_new).
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = cfg.adam_b1 * np.asarray(m, dtype=np.float64) + (1.0 - cfg.adam_b1) * g
    v = cfg.adam_b2 * np.asarray(v, dtype=np.float64) + (1.0 - cfg.adam_b2) * g * g
    n = t + 1
    m_hat = m / (1.0 - cfg.adam_b1 ** n)
    v_hat = v / (1.0 - cfg.adam_b2 ** n)
    p = p * (1.0 - cfg.adam_lr * cfg.adam_wd) - cfg.adam_lr * m_hat / (np.sqrt(v_hat) + cfg.adam_eps)
    return p, m, v


# ---------------------------------------------------------------- whole set
def oracle_step(params, grads, state, kinds, t: int, cfg: OracleConfig):
    """One step over a parameter list, one tensor at a time.

    ``kinds[i]`` is "matrix" (Muon) or "adamw".  ``state[i]`` is the momentum
    array for a matrix and a (m, v) pair for an AdamW tensor.  Returns new
    (params, state) lists; inputs are not modified.
    """
    new_p, new_s = [], []
    for P, G, S, kind in zip(params, grads, state, kinds):
        if kind == "matrix":
            Wn, Mn, _ = muon_matrix_step(P, S, G, t, cfg)
            new_p.append(Wn)
            new_s.append(Mn)
        else:
            pn, mn, vn = adamw_step(P, G, S[0], S[1], t, cfg)
            new_p.append(pn)
            new_s.append((mn, vn))
    return new_p, new_s


__all__ = [
    "OracleConfig", "BRANCH_ROWNORM", "BRANCH_NS5", "BRANCH_BLOCK_NS5",
    "refresh_indicator", "branch", "momentum_update", "newton_schulz",
    "row_normalize", "column_norms_from_row_shards", "block_newton_schulz",
    "direction", "muon_matrix_step", "adamw_step", "oracle_step",
]

