"""Reference (oracle) for the Kimi Delta Attention operator -- TEST INFRASTRUCTURE ONLY.

This module is the slow, obviously-correct CPU definition that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path never does.  It shares no code with the HIP
library (the two meet only in the seeded input generators, which hold none of the method's
arithmetic).

What it computes (Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (1)): for every sequence n
and head h independently, starting from the entering state S0[n, h] (zeros when absent), every
token t applies

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,

with alpha_t = exp(g_t) per key channel (§2.1.1, eq. (5): g is a natural-log decay).  The
channel-wise decay acts before the delta-rule erase/write (the text right above eq. (1)), and
the output reads the state after the current token's update (the remark under eq. (4) that the
causal mask keeps its diagonal for this reason).  The loop below is the same update written
without the dense dk x dk matrix: decay the rows of S, form the delta-rule residual
u = beta (v - S^T k) against the decayed state, add the rank-one write k u^T, read out S^T q.

Every input is upcast from its stored dtype to float64; the arithmetic is float64 throughout.
``scale`` multiplies q (eq. (1) has no scale; tests pass 1.0).

Pinned by tests/test_oracle_pins.py: closed forms (beta = 0, a single token, orthonormal keys
with g = 0), exact rational brute force on tiny shapes, read-after-write, linearity/affinity in
(V, S0) (§5.1.2, eq. (17)), resume, varlen independence, and agreement with the independent
chunkwise algorithm in ``oracle/chunkwise.py`` for every chunk size.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """Stored values -> float64 numpy (accepts numpy arrays or CPU torch tensors)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: go through float32 first (bf16 is exact in fp32)
        x = x.detach().cpu()
        if x.dtype != x.new_zeros(()).double().dtype:
            x = x.float()
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def kda_token_step(S, q, k, v, g, beta, scale=1.0):
    """One token of eq. (1) on one head.  S: [dk, dv] float64 (not modified).

    Returns (o [dv], S_new [dk, dv])."""
    S = np.exp(g)[:, None] * S                # Diag(alpha_t) S_{t-1}
    u = beta * (v - S.T @ k)                  # delta-rule residual against the decayed state
    S = S + np.outer(k, u)                    # (I - beta k k^T) Diag(alpha) S + beta k v^T
    o = S.T @ (scale * q)                     # read-out after the update
    return o, S


def _sequence_bounds(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    if B != 1:
        raise ValueError("packed (cu_seqlens) inputs have batch dimension 1")
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu[:-1], cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def kda_forward(q, k, v, g, beta, S0=None, cu_seqlens=None, scale=1.0, heads=None):
    """Token-by-token KDA over whole sequences.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; g: [B, T, H, dk] (natural-log decay);
    beta: [B, T, H]; S0: [N, H, dk, dv] or None (zeros); cu_seqlens: None (N = B, one
    sequence per row) or int array [N + 1] with B = 1 (packed sequences).
    ``heads``: optional list of head indices to evaluate (others are left zero).

    Returns (o [B, T, H, dv] float64, S_T [N, H, dk, dv] float64)."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    seqs = _sequence_bounds(B, T, cu_seqlens)
    N = len(seqs)
    S0 = np.zeros((N, H, dk, dv)) if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    for n, (b, bos, eos) in enumerate(seqs):
        for h in (range(H) if heads is None else heads):
            S = S0[n, h].copy()
            for t in range(bos, eos):
                o[b, t, h], S = kda_token_step(S, q[b, t, h], k[b, t, h], v[b, t, h],
                                               g[b, t, h], beta[b, t, h], scale)
            ST[n, h] = S
    return o, ST


def kda_decode_step(q, k, v, g, beta, S, scale=1.0):
    """One decode token per (sequence, head): eq. (1) with T = 1 (§5.4.2: the state is updated
    in place every step; here the new state is returned).

    q, k: [N, H, dk]; v: [N, H, dv]; g: [N, H, dk]; beta: [N, H]; S: [N, H, dk, dv].
    Returns (o [N, H, dv], S_new [N, H, dk, dv]) in float64."""
    q, k, v, g, beta, S = (_f64(a) for a in (q, k, v, g, beta, S))
    N, H = q.shape[:2]
    o = np.zeros(v.shape)
    Snew = np.zeros(S.shape)
    for n in range(N):
        for h in range(H):
            o[n, h], Snew[n, h] = kda_token_step(S[n, h], q[n, h], k[n, h], v[n, h],
                                                 g[n, h], beta[n, h], scale)
    return o, Snew


G_MIN = -5.0   # §2.1.1, eq. (5): the lower bound of the log-decay is fixed at -5


def kda_gate(z, A_log, g_min=G_MIN):
    """The bounded decay map of §2.1.1, eq. (5): g = g_min * Sigmoid(exp(A_h) * z), per head h
    (A_h is the per-head log-scale) and per key channel.

    z: [..., H, dk] (any leading shape); A_log: [H].  Returns g in float64, in [g_min, 0].
    Sigmoid(x) = 1 / (1 + exp(-x)); exp(-x) overflowing to +inf for very negative x gives the
    limit 0 exactly."""
    z, A = _f64(z), _f64(A_log)
    x = np.exp(A)[:, None] * z
    with np.errstate(over="ignore"):
        return g_min / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------- around the operator
# The steps that eq. (2) and eq. (6) of §2.1.1 apply around the recurrence, for the fused decode:
# the short convolution (caller taps) and Swish of the projections, L2-normalised q and k,
# beta = Sigmoid of its logit, and the output gate y = Sigmoid(G) * RMSNorm(o~) with G = W_g x
# given (the projections themselves and W_o need trained weights and stay outside).

L2NORM_FLOOR = 1e-12   # the norm is floored so that a zero vector stays zero


def l2norm(x):
    """x / max(||x||_2, 1e-12) over the last axis, float64 (eq. (2): L2Norm of q and k)."""
    x = _f64(x)
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    return x / np.maximum(n, L2NORM_FLOOR)


def sigmoid(x):
    """1 / (1 + exp(-x)), float64 (eq. (2) for beta, eq. (6) for the output gate)."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def gated_rmsnorm(o, G, weight=None, eps=1e-6):
    """Sigmoid(G) * RMSNorm(o) over the last axis (per head), eq. (6) without W_o:
    RMSNorm(o) = o / sqrt(mean(o^2) + eps) * weight (weight None: ones).  float64."""
    o, G = _f64(o), _f64(G)
    r = o / np.sqrt((o * o).mean(-1, keepdims=True) + eps)
    if weight is not None:
        r = r * _f64(weight)
    return sigmoid(G) * r


def swish(x):
    """x * Sigmoid(x), float64 (eq. (2): the activation after the short convolution)."""
    x = _f64(x)
    return x * sigmoid(x)


def short_conv(x, w, state=None):
    """Causal depthwise convolution along the token axis (eq. (2): ShortConv of a projection).

    x: [N, K, H, C], K consecutive tokens per sequence; w: [H, C, W] taps per (head, channel),
    w[..., W-1] weighting the current token and w[..., 0] the token W-1 steps back; state:
    [N, H, C, W-1], the W-1 inputs that precede token 0, oldest first (None: zeros).  With xx the
    state followed by x along the tokens,

        y[n, t, h, c] = sum_j w[h, c, j] * xx[n, h, c, t + j].

    Returns (y [N, K, H, C], xx [N, H, C, W - 1 + K]) in float64; the window after the first m
    tokens is xx[..., m : m + W - 1]."""
    x, w = _f64(x), _f64(w)
    N, K, H, C = x.shape
    W = w.shape[-1]
    st = np.zeros((N, H, C, W - 1)) if state is None else _f64(state)
    xx = np.concatenate([st, np.transpose(x, (0, 2, 3, 1))], axis=-1)
    y = np.zeros((N, K, H, C))
    for t in range(K):
        y[:, t] = (xx[..., t:t + W] * w[None]).sum(-1)
    return y, xx


def kda_fused_decode(q, k, v, z, A_log, b, S, G, weight=None, eps=1e-6, scale=1.0, n_commit=None,
                     conv_w=None, conv_state=None):
    """K decode tokens per (sequence, head) with the fused prologue and epilogue: q, k
    L2-normalised, beta = Sigmoid(b), g = kda_gate(z, A_log), the recurrence (eq. (1)) from S,
    outputs gated_rmsnorm(o~, G, weight, eps).  q, k, z [N, K, H, dk]; v, G [N, K, H, dv];
    b [N, K, H]; S [N, H, dk, dv].  Returns (y [N, K, H, dv], state after n_commit[n] tokens)
    in float64 (n_commit None: all K).

    With conv_w ([H, 2 dk + dv, W]: the taps of q's channels, then k's, then v's) q, k, v are the
    projections before eq. (2)'s ShortConv, and the operator's inputs are
    L2Norm(Swish(ShortConv(q))), L2Norm(Swish(ShortConv(k))), Swish(ShortConv(v)), the window
    entering from conv_state ([N, H, 2 dk + dv, W - 1], oldest first; None: zeros).  The result
    then also holds the window after the n_commit[n] committed tokens."""
    conv_out = None
    if conv_w is not None:
        q, k, v = _f64(q), _f64(k), _f64(v)
        dk, dv = q.shape[-1], v.shape[-1]
        cw = _f64(conv_w)
        st = None if conv_state is None else _f64(conv_state)
        parts = []
        for x, lo, hi in ((q, 0, dk), (k, dk, 2 * dk), (v, 2 * dk, 2 * dk + dv)):
            y, xx = short_conv(x, cw[:, lo:hi], None if st is None else st[:, :, lo:hi])
            parts.append((swish(y), xx))
        (q, xq), (k, xk), (v, xv) = parts
        W = cw.shape[-1]
        N, K = q.shape[:2]
        xx = np.concatenate([xq, xk, xv], axis=2)
        conv_out = np.zeros(xx.shape[:3] + (W - 1,))
        for n in range(N):
            c = K if n_commit is None else max(0, min(K, int(n_commit[n])))
            conv_out[n] = xx[n, :, :, c:c + W - 1]
    qn, kn = l2norm(q), l2norm(k)
    beta = sigmoid(b)
    g = kda_gate(z, A_log)
    S = _f64(S)
    N, K = qn.shape[:2]
    o, _ = kda_forward(qn, kn, v, g, beta, S, scale=scale)
    y = gated_rmsnorm(o, G, weight, eps)
    S_out = S.copy()
    for n in range(N):
        c = K if n_commit is None else max(0, min(K, int(n_commit[n])))
        if c > 0:
            _, s = kda_forward(qn[n:n + 1, :c], kn[n:n + 1, :c], _f64(v)[n:n + 1, :c], g[n:n + 1, :c],
                               beta[n:n + 1, :c], S[n:n + 1], scale=scale)
            S_out[n] = s[0]
    if conv_out is not None:
        return y, S_out, conv_out
    return y, S_out
