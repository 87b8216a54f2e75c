"""Seeded synthetic inputs for the KDA operator (shared by tests, the oracle calls and bench.py).

This module only draws random numbers and shapes them; it holds none of the operator's
arithmetic.  The recipe follows the workloads the operator is specified on:

- q, k ~ N(0, 1), L2-normalised over the key dimension per (token, head), then stored in the
  input dtype (the projections of Kimi K3: Open Frontier Intelligence, §2.1.1, eq. (2) end in an
  L2 normalisation);
- v ~ N(0, 1), stored in the input dtype;
- z ~ N(0, 1) per (token, head, key channel); A_h ~ N(0, A_std) per head; the log-decay input is
  g = g_min * sigmoid(exp(A_h) * z) with g_min = -5 (§2.1.1, eq. (5)), stored as float32;
  optionally a seeded fraction of channels per head has z fixed at +3 (decay close to g_min);
- beta = sigmoid(N(0, 1)), stored in the input dtype;
- S0 ~ N(0, S0_std), float32 (or absent).

Second arguments of N(.,.) are standard deviations.  Packed variable-length batches draw their
lengths from a lognormal (median 1024, sigma 1.0), clipped to [1, 65536], with the longest forced
to 65536.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

G_MIN = -5.0


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype = torch.bfloat16
    A_std: float = 0.5
    S0_std: float | None = 0.1
    near_gmin_frac: float = 0.0
    n_varlen: int = 0            # > 0: packed lognormal lengths (B = 1, T = total)
    note: str = ""


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype = torch.bfloat16
    A_std: float = 0.5
    S_std: float = 0.1


# The five workloads the operator is specified on (sizes as stated there).
CONFIGS = {
    "tiny_fp32_t256_d64": PrefillConfig("tiny_fp32_t256_d64", B=1, T=256, H=1, dk=64, dv=64,
                                        dtype=torch.float32, A_std=0.0, S0_std=None),
    "h16_t4096_d128": PrefillConfig("h16_t4096_d128", B=1, T=4096, H=16, dk=128, dv=128),
    "prefill_b4_h32_t32k_d128": PrefillConfig("prefill_b4_h32_t32k_d128", B=4, T=32768, H=32,
                                              dk=128, dv=128),
    "long_b1_h32_t1m_d128": PrefillConfig("long_b1_h32_t1m_d128", B=1, T=1 << 20, H=32, dk=128,
                                          dv=128, near_gmin_frac=0.1),
    "varlen64_h32_d128": PrefillConfig("varlen64_h32_d128", B=1, T=0, H=32, dk=128, dv=128,
                                       n_varlen=64),
}
DECODE_CONFIG = DecodeConfig("decode_n1024_h32_d128", N=1024, H=32, dk=128, dv=128)


def varlen_lengths(n: int, seed: int, median: int = 1024, sigma: float = 1.0,
                   max_len: int = 65536) -> list[int]:
    """Lognormal sequence lengths, clipped to [1, max_len], longest forced to max_len."""
    rng = np.random.default_rng(seed + 7919)
    lens = np.clip(np.round(np.exp(rng.normal(math.log(median), sigma, size=n))), 1, max_len)
    lens = lens.astype(np.int64)
    lens[int(np.argmax(lens))] = max_len
    return [int(x) for x in lens]


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def _gen(device, seed):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _l2norm_last(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-12)


def make_prefill_inputs(B, T, H, dk, dv, *, dtype=torch.bfloat16, seed=0, device="cpu",
                        A_std=0.5, S0_std=0.1, near_gmin_frac=0.0, cu_seqlens=None,
                        beta_dtype=None, with_logits=False):
    """Draw one prefill batch.  Returns a dict with q, k, v, g, beta, S0 (or None),
    cu_seqlens (int32 tensor on ``device`` or None) and N (number of sequences).  With
    ``with_logits`` it also holds the decay logits z ([B, T, H, dk], stored in ``dtype``) and the
    per-head log-scales A_log ([H] float32) that g was synthesised from (g itself comes from the
    float32 logits, before z is rounded to ``dtype``)."""
    device = torch.device(device)
    gen = _gen(device, seed)
    q = _l2norm_last(_randn((B, T, H, dk), gen, device)).to(dtype)
    k = _l2norm_last(_randn((B, T, H, dk), gen, device)).to(dtype)
    v = _randn((B, T, H, dv), gen, device).to(dtype)
    z = _randn((B, T, H, dk), gen, device)
    A = _randn((H,), gen, device) * A_std
    if near_gmin_frac > 0:
        nb = int(round(near_gmin_frac * dk))
        chans = torch.stack([torch.randperm(dk, generator=gen, device=device)[:nb]
                             for _ in range(H)])                      # [H, nb]
        mask = torch.zeros((H, dk), dtype=torch.bool, device=device)
        mask.scatter_(1, chans, True)
        z = torch.where(mask, torch.full_like(z, 3.0), z)
    g = (G_MIN * torch.sigmoid(torch.exp(A)[None, None, :, None] * z)).float()
    zs = z.to(dtype) if with_logits else None
    del z
    beta = torch.sigmoid(_randn((B, T, H), gen, device)).to(beta_dtype or dtype)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    S0 = None if S0_std is None else _randn((N, H, dk, dv), gen, device) * S0_std
    cu = None if cu_seqlens is None else torch.as_tensor(cu_seqlens, dtype=torch.int32).to(device)
    out = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, cu_seqlens=cu, N=N)
    if with_logits:
        out.update(z=zs, A_log=A.float().contiguous())
    return out


def make_config_inputs(cfg: PrefillConfig, seed=0, device="cpu"):
    """Inputs for one of the named workloads."""
    if cfg.n_varlen:
        lens = varlen_lengths(cfg.n_varlen, seed)
        cu = cu_from_lengths(lens)
        return make_prefill_inputs(1, int(cu[-1]), cfg.H, cfg.dk, cfg.dv, dtype=cfg.dtype,
                                   seed=seed, device=device, A_std=cfg.A_std, S0_std=cfg.S0_std,
                                   near_gmin_frac=cfg.near_gmin_frac, cu_seqlens=cu)
    return make_prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, dtype=cfg.dtype, seed=seed,
                               device=device, A_std=cfg.A_std, S0_std=cfg.S0_std,
                               near_gmin_frac=cfg.near_gmin_frac)


def make_decode_inputs(N, H, dk, dv, *, dtype=torch.bfloat16, seed=0, device="cpu", A_std=0.5,
                       S_std=0.1):
    """One decode token per (sequence, head) plus the states it updates."""
    device = torch.device(device)
    gen = _gen(device, seed)
    q = _l2norm_last(_randn((N, H, dk), gen, device)).to(dtype)
    k = _l2norm_last(_randn((N, H, dk), gen, device)).to(dtype)
    v = _randn((N, H, dv), gen, device).to(dtype)
    z = _randn((N, H, dk), gen, device)
    A = _randn((H,), gen, device) * A_std
    g = (G_MIN * torch.sigmoid(torch.exp(A)[None, :, None] * z)).float()
    beta = torch.sigmoid(_randn((N, H), gen, device)).to(dtype)
    S = _randn((N, H, dk, dv), gen, device) * S_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, S=S)


def make_fused_decode_inputs(N, K, H, dk, dv, *, dtype=torch.bfloat16, seed=0, device="cpu",
                             A_std=0.5, S_std=0.1):
    """K decode tokens per (sequence, head) as the fused decode takes them: the raw projections
    q, k, v ~ N(0, 1) (not normalised), decay logits z ~ N(0, 1) and per-head log-scales
    A_log ~ N(0, A_std), beta logits ~ N(0, 1), output-gate pre-activations G ~ N(0, 1), an RMSNorm
    weight 1 + 0.1 N(0, 1) (float32 [dv]) and states S ~ N(0, S_std)."""
    device = torch.device(device)
    gen = _gen(device, seed)
    q = _randn((N, K, H, dk), gen, device).to(dtype)
    k = _randn((N, K, H, dk), gen, device).to(dtype)
    v = _randn((N, K, H, dv), gen, device).to(dtype)
    z = _randn((N, K, H, dk), gen, device).to(dtype)
    A_log = (_randn((H,), gen, device) * A_std).float()
    b = _randn((N, K, H), gen, device).to(dtype)
    G = _randn((N, K, H, dv), gen, device).to(dtype)
    w = (1.0 + 0.1 * _randn((dv,), gen, device)).float()
    S = _randn((N, H, dk, dv), gen, device) * S_std
    return dict(q=q, k=k, v=v, z=z, A_log=A_log, beta_logit=b, G=G, norm_weight=w, S=S)


def make_conv_inputs(N, H, dk, dv, W, *, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Taps and entering windows for the short convolution in front of the fused decode: weights
    [H, 2 dk + dv, W] float32 ~ N(0, 1 / W) (channels of q, then k, then v; the last tap weights
    the current token) and windows [N, H, 2 dk + dv, W - 1] ~ N(0, 1) in dtype, oldest first,
    standing for the previous projections."""
    device = torch.device(device)
    gen = _gen(device, seed)
    C = 2 * dk + dv
    w = (_randn((H, C, W), gen, device) / W ** 0.5).float()
    st = _randn((N, H, C, max(W - 1, 0)), gen, device).to(dtype)
    return dict(conv_weight=w, conv_state=st)
