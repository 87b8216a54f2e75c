"""Independent float64 chunkwise KDA -- TEST INFRASTRUCTURE ONLY (pins the token oracle).

A second, structurally different CPU algorithm for the same operator, used only to pin
``oracle/kda_oracle.py``: the chunkwise parallel form (Kimi K3: Open Frontier Intelligence,
§2.1.1, eqs. (3)-(4)) must reproduce the token recurrence of eq. (1) exactly (up to rounding)
for every chunk size C.  It never runs on the product path and shares no code with the HIP
library.

Within a chunk with entering state S (positions r = 1..C), G_r = sum_{i<=r} g_i per key channel
(the log of the cumulative decay gamma^r of eq. (3)).  The pages defer the UT transform to the
Kimi Linear paper; unrolling eq. (1) over the chunk gives it directly:

    the effective write of token r is u_r = beta_r (v_r - S_{r-1}^T Diag(alpha_r) k_r), and
    substituting S_{r-1} = Diag(gamma^{r-1}) S + sum_{i<r} Diag(gamma^{i+1->r-1}) k_i u_i^T gives
    (I + A_kk) U_true = Diag(beta) V - Diag(beta) (K * Gamma) S,
    A_kk[r, i] = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)   for i < r  (strictly lower).

Hence, with T = (I + A_kk)^{-1}: U = T Diag(beta) V, W = T Diag(beta) (K * Gamma) and the
pseudo-value V~ = U - W S (the quantity §2.1.1 names).  The outputs are eq. (4),
O = (Q * Gamma) S + Tril[(Q * Gamma)(K / Gamma)^T] V~ with the diagonal kept, and the state
leaving the chunk is S' = Diag(gamma^C) S + (K * gamma^C / Gamma)^T V~.

The decayed products use exp(G_r - G_i) directly (log-space), so no reciprocal of a long
cumulative product is ever formed.  T is obtained with a library triangular solve.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_intermediates(q, k, v, g, beta, scale=1.0):
    """Per-chunk quantities for one head: q, k, g [C, dk]; v [C, dv]; beta [C].

    Returns dict with G [C, dk], A_kk, T (inverse of I + A_kk), W [C, dk], U [C, dv],
    A_qk [C, C] (lower incl. diagonal), Qg = Q * Gamma, Kend = K * gamma^C / Gamma,
    gammaC [dk]."""
    q = scale * np.asarray(q, np.float64)
    k, v, g, beta = (np.asarray(a, np.float64) for a in (k, v, g, beta))
    C = k.shape[0]
    G = np.cumsum(g, axis=0)
    rel = np.exp(G[:, None, :] - G[None, :, :])          # [r, i, c] = exp(G_rc - G_ic)
    lower_strict = np.tril(np.ones((C, C)), -1)
    lower_incl = np.tril(np.ones((C, C)), 0)
    with np.errstate(over="ignore", invalid="ignore"):
        A_kk = np.einsum("rc,ic,ric->ri", k, k, np.where(lower_strict[:, :, None] > 0, rel, 0.0))
        A_qk = np.einsum("rc,ic,ric->ri", q, k, np.where(lower_incl[:, :, None] > 0, rel, 0.0))
    A_kk = beta[:, None] * A_kk * lower_strict
    A_qk = A_qk * lower_incl
    eye = np.eye(C)
    Tm = solve_triangular(eye + A_kk, eye, lower=True, unit_diagonal=True)
    Gamma = np.exp(G)
    W = Tm @ (beta[:, None] * (k * Gamma))
    U = Tm @ (beta[:, None] * v)
    gammaC = np.exp(G[-1])
    Kend = k * np.exp(G[-1][None, :] - G)
    return dict(G=G, A_kk=A_kk, T=Tm, W=W, U=U, A_qk=A_qk, Qg=q * Gamma, Kend=Kend,
                gammaC=gammaC)


def chunk_step(S, q, k, v, g, beta, scale=1.0):
    """Advance one chunk: returns (O [C, dv], S_next [dk, dv])."""
    c = chunk_intermediates(q, k, v, g, beta, scale)
    Vt = c["U"] - c["W"] @ S
    O = c["Qg"] @ S + c["A_qk"] @ Vt
    S_next = c["gammaC"][:, None] * S + c["Kend"].T @ Vt
    return O, S_next


def kda_forward_chunkwise(q, k, v, g, beta, S0=None, chunk=64, scale=1.0):
    """Chunkwise KDA for one sequence (all heads): q, k, g [T, H, dk]; v [T, H, dv];
    beta [T, H]; S0 [H, dk, dv] or None.  The last chunk may be partial.
    Returns (o [T, H, dv], S_T [H, dk, dv]) float64."""
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((T, H, dv))
    ST = np.zeros((H, dk, dv))
    for h in range(H):
        S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[h], np.float64).copy()
        for s in range(0, T, chunk):
            e = min(T, s + chunk)
            o[s:e, h], S = chunk_step(S, q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h],
                                      beta[s:e, h], scale)
        ST[h] = S
    return o, ST
