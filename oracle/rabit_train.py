"""Plain float64 CPU oracle for the training side of one RaBiT linear layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (the pages about "RaBiT: Residual-Aware Binarization Training for
Accurate and Efficient LLMs"):

* paper §4.2 "The Coupled Forward Pass", steps 1-3: in every training step the
  binary cores are derived from the one shared weight W_FP with the current
  learnable scales, and the forward uses W_hat^(k) = Σ_i g_i ⊙ B_i ⊙ h_i.
* paper §4.2 "Backward Pass and Parameter Updates", first item: the gradient
  with respect to the effective weight W_hat^(k) is handed to W_FP unchanged
  (a straight-through estimator over the whole derivation); the update is
  shaped d_out x d_in.
* same section, second item: g_i and h_i get chain-rule gradients summed over
  the samples of the mini-batch, with the cores B_i held constant.
* paper §4.2 last paragraph and §5.4: inference (and the gradient to the
  layer input) uses the same effective weight.

Readings (the formulas of both items are missing from the pages' text):

* The loss gradient at the layer output is dY [N][d_out] (row n = sample n);
  the layer computes Y = X W_hatᵀ (X is [N][d_in], the inference convention
  y = W_hat x per sample).
* dW_FP = Σ_n dY[n] X[n]ᵀ  (the gradient of W_hat^(k), d_out x d_in).
* dg_i = Σ_n dY[n] ⊙ (B_i (h_i ⊙ X[n])),  dh_i = Σ_n X[n] ⊙ (B_iᵀ (g_i ⊙ dY[n]))
  (chain rule through W_hat_i = g_i ⊙ B_i ⊙ h_i with B_i constant).
* dX[n] = W_hatᵀ dY[n]  (the gradient passed to the layer below).
* The forward takes the scales as stored for inference (fp16); the
  derivation is ``rabit_oracle.derive(..., mode="given")``.
* The sum over samples is written as one float64 matrix product per term (a
  library step; no other reordering).

Pins (tests/test_oracle_train.py): torch.autograd in float64 on the same
graph; exact finite differences in Fraction on a tiny case; one-hot closed
forms; the Euler identities <g_i, dg_i> = <h_i, dh_i> = <dW, W_hat_i> and
Σ_i <dW, W_hat_i> = <dY, Y>; the transposed layer's bit positions by hand.
"""
from __future__ import annotations

import numpy as np

from .rabit_oracle import Derived, derive, weff

__all__ = [
    "train_forward", "transposed", "grad_weight", "grad_scales", "grad_input",
    "grad_weight_entries", "grad_g_rows", "grad_h_cols", "grad_input_cols",
]


def _signs(s: np.ndarray) -> np.ndarray:
    return np.where(s, -1.0, 1.0)


def train_forward(w, x, g1, h1, g2=None, h2=None, n_paths: int = 2, g3=None, h3=None):
    """Coupled forward of one training step (paper §4.2 steps 1-3): derive the
    cores from W_FP with the current scales, then Y = X W_hatᵀ in float64.
    Returns (Derived, Y)."""
    d = derive(w, "given", g1=g1, h1=h1, g2=g2, h2=h2, n_paths=n_paths, g3=g3, h3=h3)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return d, x @ weff(d).T


def transposed(d: Derived) -> Derived:
    """The layer of W_hatᵀ: cores B_iᵀ, output scales h_i, input scales g_i
    (W_hatᵀ = Σ_i h_i ⊙ B_iᵀ ⊙ g_i)."""
    ps = d.paths
    s = [p[0].T.copy() for p in ps]
    g = [p[2] for p in ps]
    h = [p[1] for p in ps]
    if len(ps) == 2:
        return Derived(s[0], s[1], g[0], h[0], g[1], h[1])
    return Derived(s[0], s[1], g[0], h[0], g[1], h[1], None, s[2], g[2], h[2])


def grad_weight(x, dy) -> np.ndarray:
    """Straight-through gradient to W_FP: Σ_n dY[n] X[n]ᵀ, [d_out][d_in]."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
    return dy.T @ x


def grad_scales(d: Derived, x, dy):
    """[(dg_i, dh_i)] per path: Σ_n dY[n] ⊙ (B_i (h_i ⊙ X[n])) and
    Σ_n X[n] ⊙ (B_iᵀ (g_i ⊙ dY[n])) with B_i constant."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
    res = []
    for s, g, h in d.paths:
        b = _signs(s)
        t_out = (x * h.astype(np.float64)[None, :]) @ b.T       # [N][out]: B (h ⊙ x_n)
        t_in = (dy * g.astype(np.float64)[None, :]) @ b         # [N][in]:  Bᵀ (g ⊙ dy_n)
        res.append(((dy * t_out).sum(axis=0), (x * t_in).sum(axis=0)))
    return res


def grad_input(d: Derived, dy) -> np.ndarray:
    """dX[n] = W_hatᵀ dY[n]; [N][d_in]."""
    dy = np.atleast_2d(np.asarray(dy, dtype=np.float64))
    return dy @ weff(d)


# --- sampled forms (the same sums, for a subset of outputs at full size) ---
def grad_weight_entries(x, dy, rows, cols) -> np.ndarray:
    """dW[rows[k], cols[k]] = Σ_n dY[n, rows[k]] X[n, cols[k]]."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    return np.einsum("nk,nk->k", dy[:, rows], x[:, cols])


def grad_g_rows(s_rows: np.ndarray, h: np.ndarray, x, dy_rows) -> np.ndarray:
    """dg for the output rows whose sign rows are s_rows ([R][in]) and whose
    output gradients are dy_rows ([N][R])."""
    x = np.asarray(x, dtype=np.float64)
    t = (x * h.astype(np.float64)[None, :]) @ _signs(s_rows).T     # [N][R]
    return (np.asarray(dy_rows, dtype=np.float64) * t).sum(axis=0)


def grad_h_cols(s_cols: np.ndarray, g: np.ndarray, dy, x_cols) -> np.ndarray:
    """dh for the input columns whose sign columns are s_cols ([out][C]) and
    whose inputs are x_cols ([N][C])."""
    dy = np.asarray(dy, dtype=np.float64)
    t = (dy * g.astype(np.float64)[None, :]) @ _signs(s_cols)      # [N][C]
    return (np.asarray(x_cols, dtype=np.float64) * t).sum(axis=0)


def grad_input_cols(cols_weff: np.ndarray, dy) -> np.ndarray:
    """dX[:, cols] from the W_hat columns cols_weff ([out][C])."""
    return np.asarray(dy, dtype=np.float64) @ cols_weff
