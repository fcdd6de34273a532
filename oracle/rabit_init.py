"""Plain float64 CPU oracle for the initialisation of the scales: iterative
residual SVID with optional I/O channel importance preconditioning.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (the pages about "RaBiT: Residual-Aware Binarization Training for
Accurate and Efficient LLMs"):

* paper §4.3 "Iterative Residual SVID", eq.: in sweep t, path i is re-fitted
  to R_i^(t) = W_FP − Σ_{j<i} W_hat_j^(t) − Σ_{j>i} W_hat_j^(t−1) (paths before
  i already re-fitted in this sweep, paths after i from the previous sweep),
  (B_i, g_i, h_i) = SVID(R_i), W_hat_i = g_i ⊙ B_i ⊙ h_i.
* App. F.3: the first sweep is the greedy SVID; Table 11 and F.1: T_max = 20
  sweeps.
* paper §4.3 "I/O Channel Importance-Scaled Preconditioning", eqs.: the
  decomposition runs on W' = s_out^a_out ⊙ W_FP ⊙ s_in^a_in and the scales are
  mapped back with g_i = s_out^-a_out ⊙ g_i', h_i = s_in^-a_in ⊙ h_i'.

Readings:

* SVID (not defined on the pages; the pages cite OneBit for it): B = sign(R)
  (+1 unless R < 0) and g hᵀ the best rank-1 approximation of |R| in the
  Frobenius norm, i.e. sqrt(σ_1) times the leading singular vectors, taken
  non-negative (|R| is non-negative, so its leading singular vectors can be).
  With g, h >= 0 this (B, g, h) minimises ||R − g ⊙ B ⊙ h||_F exactly.
* W_hat_j^(0) = 0 for every path before the first sweep (so sweep 1 is greedy).
* The preconditioning factors are given as f_out = s_out^a_out and
  f_in = s_in^a_in (positive; the calibration statistics that produce s_in and
  s_out are outside the decomposition); W' = f_out ⊙ W ⊙ f_in,
  g_i = g_i' / f_out, h_i = h_i' / f_in.
* The leading singular triple is numpy's SVD of |R| in float64 (a library
  step).

Pins (tests/test_oracle_init.py): exact recovery of a matrix that is a sign
pattern times a positive rank-1 matrix; the 2x2 leading singular value in
closed form; SVID optimality against perturbed candidates; the residual norm
never rises across a sweep (each re-fit is an exact block minimisation);
sweep 1 equals two greedy SVIDs; at unit preconditioning factors the result
is unchanged, and the mapped-back scales reproduce the preconditioned fit.
"""
from __future__ import annotations

import numpy as np

__all__ = ["svid", "svid_leading", "residual_svid", "svid_objective"]


def svid(r: np.ndarray):
    """(s, g, h): s = (R < 0) (True = -1), g hᵀ the best rank-1 fit of |R|,
    with g, h >= 0 and ||g|| = ||h|| (both sqrt(σ_1) times unit vectors)."""
    r = np.asarray(r, dtype=np.float64)
    s = r < 0
    a = np.abs(r)
    u, sig, vt = np.linalg.svd(a, full_matrices=False)
    u0, v0 = u[:, 0], vt[0]
    if u0.sum() < 0:               # the sign of a singular pair is arbitrary
        u0, v0 = -u0, -v0
    root = np.sqrt(sig[0])
    return s, root * np.maximum(u0, 0.0), root * np.maximum(v0, 0.0)


def svid_leading(r: np.ndarray):
    """The same (s, g, h) as ``svid`` for large matrices: the leading singular
    triple from scipy's sparse SVD (ARPACK, k = 1) instead of the full SVD (a
    library step; pinned against ``svid`` on small matrices)."""
    from scipy.sparse.linalg import svds
    r = np.asarray(r, dtype=np.float64)
    s = r < 0
    u, sig, vt = svds(np.abs(r), k=1, tol=1e-12)
    u0, v0 = u[:, 0], vt[0]
    if u0.sum() < 0:
        u0, v0 = -u0, -v0
    root = np.sqrt(sig[0])
    return s, root * np.maximum(u0, 0.0), root * np.maximum(v0, 0.0)


def _what(s, g, h):
    return g[:, None] * np.where(s, -1.0, 1.0) * h[None, :]


def svid_objective(w, paths) -> float:
    """||W − Σ_i g_i ⊙ B_i ⊙ h_i||_F for paths [(s, g, h)]."""
    w = np.asarray(w, dtype=np.float64)
    res = w.copy()
    for s, g, h in paths:
        res -= _what(s, g, h)
    return float(np.linalg.norm(res))


def residual_svid(w, n_paths: int = 2, sweeps: int = 20, f_out=None, f_in=None,
                  history: list | None = None):
    """Iterative residual SVID (paper §4.3 eq.), optionally on the
    preconditioned matrix; returns [(s_i, g_i, h_i)] with the scales mapped
    back to the original domain. ``history`` (if given) receives the
    objective on the preconditioned matrix after every re-fit."""
    w = np.asarray(w, dtype=np.float64)
    out, inp = w.shape
    fo = np.ones(out) if f_out is None else np.asarray(f_out, dtype=np.float64)
    fi = np.ones(inp) if f_in is None else np.asarray(f_in, dtype=np.float64)
    wp = fo[:, None] * w * fi[None, :]
    paths = [(np.zeros((out, inp), dtype=bool), np.zeros(out), np.zeros(inp))
             for _ in range(n_paths)]
    for _t in range(sweeps):
        for i in range(n_paths):
            r = wp.copy()
            for j in range(n_paths):
                if j != i:
                    r -= _what(*paths[j])
            paths[i] = svid(r)
            if history is not None:
                history.append(svid_objective(wp, paths))
    return [(s, g / fo, h / fi) for s, g, h in paths]
