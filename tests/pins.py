"""Independent fp64 formulations used to pin the oracle (test helpers).

None of these re-types the oracle's four-line loop.  Each is a different
statement of the same mathematics, taken from the pages or from textbook
linear algebra, so that a slip in the oracle (a dropped term, a wrong sign, a
transposed operand, an off-by-one in the decay) shows up as a disagreement.

* ``chunk_form`` -- the chunkwise-parallel prompt form of the Qwen3.5-9B-npu
  model page ("How it works" -> "Gated DeltaNet on the NPU": G = cumsum g,
  strictly lower N, the deltas D through (I+N)^-1, the block output O and the
  carried state S_T), with the partial last block padded by g = 0, beta = 0
  rows as the page's token_valid input does.
* ``matrix_step`` -- the same page's one-token matrix form ([q;k]^T S in one
  product, o = d q^T S + (q.k) delta, S' = d S + k delta^T).
* ``transition_form`` -- the state as an affine map per token,
  S_t = e^{g_t} (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, built from
  explicit dk x dk matrices (with beta = 1 and unit keys each factor is the
  orthogonal projector of the Kaczmarz method).
* ``block_doubling_inverse`` -- the page's exact block-doubling inverse of a
  unit lower triangular matrix, (D + C)^-1 = D^-1 - D^-1 C D^-1.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_form_unit(q, k, v, g, beta, S0, C):
    """One (sequence, head): q, k [L, dk], v [L, dv], g, beta [L], S0 [dk, dv]."""
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((L, dv))
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        # token_valid padding: pad rows carry g = 0, beta = 0 and zero q/k/v
        Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
        gg = np.zeros(C); bb = np.zeros(C)
        Q[:n], K[:n], V[:n] = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n]
        gg[:n], bb[:n] = g[c0:c0 + n], beta[c0:c0 + n]
        G = np.cumsum(gg)
        Ediff = np.exp(G[:, None] - G[None, :])          # exp(G_t - G_j)
        N = np.diag(bb) @ np.tril(Ediff * (K @ K.T), -1)  # strictly lower
        rhs = np.diag(bb) @ (V - np.diag(np.exp(G)) @ K @ S)
        D = solve_triangular(np.eye(C) + N, rhs, lower=True, unit_diagonal=True)
        Ablk = np.tril(Ediff * (Q @ K.T), 0)                # j <= t
        Oc = np.diag(np.exp(G)) @ Q @ S + Ablk @ D
        S = np.exp(G[-1]) * S + K.T @ np.diag(np.exp(G[-1] - G)) @ D
        O[c0:c0 + n] = Oc[:n]
    return O, S


def chunk_form(q, k, v, g, beta, S0, C, cu_seqlens=None):
    """Whole-call chunk form with the same layouts as the oracle."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        spans = [(b, 0, T) for b in range(B)]
    else:
        cu = list(np.asarray(cu_seqlens))
        spans = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    O = np.zeros((B, T, H, dv))
    S_T = np.zeros((len(spans), H, dk, dv))
    for n, (b, s, e) in enumerate(spans):
        for h in range(H):
            s0 = None if S0 is None else np.asarray(S0, dtype=np.float64)[n, h]
            o, st = chunk_form_unit(q[b, s:e, h], k[b, s:e, h], v[b, s:e, h],
                                    g[b, s:e, h], beta[b, s:e, h], s0, C)
            O[b, s:e, h] = o
            S_T[n, h] = st
    return O, S_T


def matrix_step(q, k, v, g, beta, S):
    """One token for one head in the page's matrix form. Returns (o, S')."""
    qk = np.stack([q, k])                    # [2, dk]
    P = qk @ S                               # [q;k]^T S in one product: [2, dv]
    d = np.exp(g)
    delta = beta * (v - d * P[1])
    o = d * P[0] + float(q @ k) * delta
    S_new = d * S + np.outer(k, delta)
    return o, S_new


def transition_form_unit(q, k, v, g, beta, S0):
    """Explicit affine transition matrices per token, for one head."""
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    I = np.eye(dk)
    O = np.zeros((L, dv))
    for t in range(L):
        A = np.exp(g[t]) * (I - beta[t] * np.outer(k[t], k[t]))
        S = A @ S + beta[t] * np.outer(k[t], v[t])
        O[t] = S.T @ q[t]
    return O, S


def block_doubling_inverse(M, base=1):
    """Inverse of a unit lower triangular matrix by exact block doubling."""
    n = M.shape[0]
    if n <= base:
        return solve_triangular(M, np.eye(n), lower=True)
    h = n // 2
    Ainv = block_doubling_inverse(M[:h, :h], base)
    Binv = block_doubling_inverse(M[h:, h:], base)
    Dinv = np.zeros_like(M)
    Dinv[:h, :h], Dinv[h:, h:] = Ainv, Binv
    Cm = np.zeros_like(M)
    Cm[h:, :h] = M[h:, :h]
    return Dinv - Dinv @ Cm @ Dinv


def rel_err(x, r):
    """Normwise max|x - r| / max|r| over the whole array."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / (den if den > 0 else 1.0))
