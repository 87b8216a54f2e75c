"""Pins of the reference implementations against what the pages and the mathematics fix.

Each pin is a function of a forward callable ``fwd(q, k, v, g, beta, S0, cu_seqlens) -> (o, S_T)``
that returns an error; the numpy oracle and the C oracle must both pass every pin, and planted
mistakes (in copies of the oracle, on the CPU) must each fail at least one pin.

Sources (Kimi K3: Open Frontier Intelligence):
- §2.1.1 eq. (1): the recurrence, decay before the delta update, output after the update;
- §2.1.1 eqs. (3)-(4): the chunkwise form (exact algebra, so chunk-size invariant);
- §2.1.1 eq. (5) and the paragraph after it: g in (g_min, 0), g_min = -5, the printed bounds;
- §5.1.2 eq. (17): the state after a segment is affine in the entering state, S = M S0 + S~.
DeltaNet (the recurrence with no decay) is the g = 0 special case named at the top of §2.1.1.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import c_oracle, chunkwise, kda_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np_fwd(q, k, v, g, beta, S0=None, cu=None):
    return kda_oracle.kda_forward(q, k, v, g, beta, S0, cu)


def _c_fwd(q, k, v, g, beta, S0=None, cu=None):
    return c_oracle.kda_forward(q, k, v, g, beta, S0, cu)


FORWARDS = {"numpy": _np_fwd, "c": _c_fwd}


def _rand_inputs(B=1, T=24, H=2, dk=6, dv=5, seed=0, g_scale=1.0, beta_one=False,
                 S0_std=0.3, cu=None):
    """float32-stored inputs (every value exact in float64)."""
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, H, dk, generator=gen)
    q = q / q.norm(dim=-1, keepdim=True)
    k = torch.randn(B, T, H, dk, generator=gen)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(B, T, H, dv, generator=gen)
    g = (-5.0 * torch.sigmoid(torch.randn(B, T, H, dk, generator=gen))) * g_scale
    beta = torch.ones(B, T, H) if beta_one else torch.sigmoid(torch.randn(B, T, H, generator=gen))
    N = B if cu is None else len(cu) - 1
    S0 = torch.randn(N, H, dk, dv, generator=gen) * S0_std
    return q.float(), k.float(), v.float(), g.float(), beta.float(), S0.float()


def _f64(t):
    return t.double().numpy()


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------------------- pin functions

def pin_beta_zero(fwd):
    """beta = 0: pure per-channel decay.  S_T = Diag(exp(sum g)) S0 and
    o_t = S0^T (exp(G_t) * q_t) with G_t the running sum of g (eq. (1) with the write off)."""
    q, k, v, g, beta, S0 = _rand_inputs(T=20, dk=6, dv=4)
    beta = torch.zeros_like(beta)
    o, ST = fwd(q, k, v, g, beta, S0)
    G = np.cumsum(_f64(g)[0], axis=0)                       # [T, H, dk]
    o_exp = np.einsum("hcd,thc->thd", _f64(S0)[0], np.exp(G) * _f64(q)[0])
    ST_exp = np.exp(G[-1])[:, :, None] * _f64(S0)[0]
    return max(_rel(o[0], o_exp), _rel(ST[0], ST_exp))


def pin_single_token_dense(fwd):
    """One token, eq. (1) evaluated literally with dense matrices:
    S_1 = (I - beta k k^T) Diag(alpha) S0 + beta k v^T,  o = S_1^T q."""
    q, k, v, g, beta, S0 = _rand_inputs(T=1, H=3, dk=5, dv=7, seed=3)
    o, ST = fwd(q, k, v, g, beta, S0)
    err = 0.0
    for h in range(3):
        qq, kk, vv = _f64(q)[0, 0, h], _f64(k)[0, 0, h], _f64(v)[0, 0, h]
        a = np.exp(_f64(g)[0, 0, h])
        b = float(beta[0, 0, h])
        S1 = (np.eye(5) - b * np.outer(kk, kk)) @ np.diag(a) @ _f64(S0)[0, h] + b * np.outer(kk, vv)
        err = max(err, _rel(ST[0, h], S1), _rel(o[0, 0, h], S1.T @ qq))
    return err


def pin_orthonormal_overwrite(fwd):
    """g = 0 (DeltaNet), beta = 1, k_t = e_{j(t)}: each token overwrites row j(t) of the state
    with v_t exactly, so S_T[j] = v at the last t with j(t) = j (else S0[j]) and
    o_t = S_t^T q_t."""
    T, dk, dv = 12, 4, 3
    gen = torch.Generator().manual_seed(5)
    js = [int(x) for x in torch.randint(0, dk - 1, (T,), generator=gen)]   # row dk-1 untouched
    k = torch.zeros(1, T, 1, dk)
    for t, j in enumerate(js):
        k[0, t, 0, j] = 1.0
    q = torch.randn(1, T, 1, dk, generator=gen)
    v = torch.randn(1, T, 1, dv, generator=gen)
    g = torch.zeros(1, T, 1, dk)
    beta = torch.ones(1, T, 1)
    S0 = torch.randn(1, 1, dk, dv, generator=gen)
    o, ST = fwd(q, k, v, g, beta, S0)
    S = _f64(S0)[0, 0].copy()
    err = 0.0
    for t, j in enumerate(js):
        S[j] = _f64(v)[0, t, 0]
        err = max(err, float(np.abs(o[0, t, 0] - S.T @ _f64(q)[0, t, 0]).max()))
    return max(err, float(np.abs(ST[0, 0] - S).max()))


def pin_read_after_write(fwd):
    """beta = 1 and |k| = 1: after token t the state maps k_t to v_t exactly (the delta rule
    writes the residual so that S_t^T k_t = v_t).  Checked through o_t with q_t = k_t."""
    q, k, v, g, beta, S0 = _rand_inputs(T=16, dk=8, dv=5, seed=7, beta_one=True)
    k = k.double()
    k = (k / k.norm(dim=-1, keepdim=True)).float()
    o, _ = fwd(k, k, v, g, beta, S0)
    kn = np.linalg.norm(_f64(k), axis=-1)                     # float32 rounding of |k| ~ 1e-7
    assert np.abs(kn - 1).max() < 1e-6
    return float(np.abs(o - _f64(v)).max())


def pin_brute_force_rational(fwd):
    """Exact rational arithmetic on a tiny case: the dense products of eq. (1) over 5 tokens with
    dk = 2, dv = 3, all inputs dyadic (exact in float32) and alpha = exp(g) taken as the exact
    rational value of the float64 exp.  Returns the relative error of the oracle."""
    T, dk, dv = 5, 2, 3
    gen = torch.Generator().manual_seed(11)

    def dy(shape, den=64):
        return (torch.randint(-den, den + 1, shape, generator=gen).float() / den)

    q, k, v = dy((1, T, 1, dk)), dy((1, T, 1, dk)), dy((1, T, 1, dv))
    g = -(torch.randint(1, 64, (1, T, 1, dk), generator=gen).float() / 16)
    beta = torch.randint(1, 16, (1, T, 1), generator=gen).float() / 16
    S0 = dy((1, 1, dk, dv))
    o, ST = fwd(q, k, v, g, beta, S0)

    F = Fraction
    S = [[F(float(S0[0, 0, i, j])) for j in range(dv)] for i in range(dk)]
    o_exact = []
    for t in range(T):
        kk = [F(float(k[0, t, 0, i])) for i in range(dk)]
        qq = [F(float(q[0, t, 0, i])) for i in range(dk)]
        vv = [F(float(v[0, t, 0, j])) for j in range(dv)]
        al = [F(math.exp(float(g[0, t, 0, i]))) for i in range(dk)]
        b = F(float(beta[0, t, 0]))
        M = [[(1 if i == r else 0) - b * kk[i] * kk[r] for r in range(dk)] for i in range(dk)]
        DS = [[al[r] * S[r][j] for j in range(dv)] for r in range(dk)]
        S = [[sum(M[i][r] * DS[r][j] for r in range(dk)) + b * kk[i] * vv[j] for j in range(dv)]
             for i in range(dk)]
        o_exact.append([sum(S[i][j] * qq[i] for i in range(dk)) for j in range(dv)])
    oe = np.array([[float(x) for x in row] for row in o_exact])
    Se = np.array([[float(x) for x in row] for row in S])
    return max(_rel(o[0, :, 0], oe), _rel(ST[0, 0], Se))


def pin_chunkwise(fwd, chunks=(1, 2, 3, 4, 8, 16, 32, 64, 96)):
    """The chunkwise form (eqs. (3)-(4), with the UT transform written out) is exact algebra, so
    the independent chunkwise algorithm must reproduce the token loop for every chunk size."""
    q, k, v, g, beta, S0 = _rand_inputs(T=96, H=2, dk=16, dv=8, seed=13)
    o, ST = fwd(q, k, v, g, beta, S0)
    err = 0.0
    for C in chunks:
        oc, STc = chunkwise.kda_forward_chunkwise(_f64(q)[0], _f64(k)[0], _f64(v)[0], _f64(g)[0],
                                                  _f64(beta)[0], _f64(S0)[0], chunk=C)
        err = max(err, _rel(o[0], oc), _rel(ST[0], STc))
    return err


def pin_affine_transition(fwd):
    """eq. (17): the state after a segment is S = M S0 + S~, where S~ is the state reached from
    S0 = 0 and M (dk x dk) is the product of the per-token transitions, obtained by running the
    same recurrence on V = 0 with S0 = I.  Also linear in (V, S0) jointly."""
    q, k, v, g, beta, S0 = _rand_inputs(T=30, H=2, dk=6, dv=4, seed=17)
    _, ST = fwd(q, k, v, g, beta, S0)
    _, S_tilde = fwd(q, k, v, g, beta, torch.zeros_like(S0))
    eye = torch.eye(6).expand(1, 2, 6, 6).contiguous()
    _, M = fwd(q, k, torch.zeros(1, 30, 2, 6), g, beta, eye)
    pred = np.einsum("nhij,nhjd->nhid", M, _f64(S0)) + S_tilde
    err = _rel(ST, pred)
    # joint linearity in (V, S0); dyadic values keep v + 2 v2 and S0 + 2 S02 exact in float32
    def dyadic(t):
        return torch.round(t * 256) / 256
    v, S0 = dyadic(v), dyadic(S0)
    v2 = dyadic(torch.randn(v.shape, generator=torch.Generator().manual_seed(1)))
    S02 = dyadic(torch.randn(S0.shape, generator=torch.Generator().manual_seed(2)))
    o1, ST1 = fwd(q, k, v, g, beta, S0)
    o2, ST2 = fwd(q, k, v2, g, beta, S02)
    o3, ST3 = fwd(q, k, v + 2 * v2, g, beta, S0 + 2 * S02)
    return max(err, _rel(o3, o1 + 2 * o2), _rel(ST3, ST1 + 2 * ST2))


def pin_resume(fwd):
    """Running a sequence in two pieces, the second entered with the first's final state, gives
    the same outputs and final state (eq. (17) with two segments)."""
    q, k, v, g, beta, S0 = _rand_inputs(T=40, H=2, dk=5, dv=6, seed=19)
    o, ST = fwd(q, k, v, g, beta, S0)
    t = 17
    oa, Sa = fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0)
    ob, Sb = fwd(q[:, t:], k[:, t:], v[:, t:], g[:, t:], beta[:, t:], torch.from_numpy(Sa).float())
    # Sa is rounded to float32 when re-entered; allow that rounding.
    return max(_rel(o, np.concatenate([oa, ob], axis=1)), _rel(ST, Sb)) * 1e-2


def pin_varlen_independence(fwd):
    """Packed sequences are independent: the packed call equals separate calls."""
    lens = [5, 0, 13, 1, 9]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    q, k, v, g, beta, S0 = _rand_inputs(B=1, T=cu[-1], H=2, dk=4, dv=3, seed=23, cu=cu)
    o, ST = fwd(q, k, v, g, beta, S0, cu)
    err = 0.0
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, STn = fwd(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e], S0[n:n + 1])
        d_o = np.abs(o[:, s:e] - on)
        err = max(err, float(d_o.max()) if d_o.size else 0.0, float(np.abs(ST[n] - STn[0]).max()))
    return err


def pin_column_independence(fwd, col_sets=([5, 1, 3, 0, 4, 2], [4, 0])):
    """Value columns evolve independently: column j of S, v and o forms its own recurrence with the
    shared keys, decays and betas (eq. (1) acts on S from the left only).  A run with the columns
    of V and S0 permuted gives the same permutation of the full run's columns, and a run on a
    subset gives exactly those columns; this is what allows the state to be split over dv.  The
    permuted run keeps dk = dv, where a transposed state would still be well-formed."""
    q, k, v, g, beta, S0 = _rand_inputs(T=24, H=2, dk=6, dv=6, seed=29)
    o, ST = fwd(q, k, v, g, beta, S0)
    err = 0.0
    for cols in col_sets:
        oc, STc = fwd(q, k, v[..., cols].contiguous(), g, beta, S0[..., cols].contiguous())
        err = max(err, _rel(oc, o[..., cols]), _rel(STc, ST[..., cols]))
    return err


PINS = {
    "beta_zero": (pin_beta_zero, 1e-13),
    "single_token_dense": (pin_single_token_dense, 1e-13),
    "orthonormal_overwrite": (pin_orthonormal_overwrite, 1e-13),
    "read_after_write": (pin_read_after_write, 1e-5),
    "brute_force_rational": (pin_brute_force_rational, 1e-13),
    "chunkwise": (pin_chunkwise, 1e-11),
    "affine_transition": (pin_affine_transition, 1e-12),
    "resume": (pin_resume, 1e-8),
    "varlen_independence": (pin_varlen_independence, 0.0),
    "column_independence": (pin_column_independence, 1e-13),
}


@pytest.mark.parametrize("impl", sorted(FORWARDS))
@pytest.mark.parametrize("pin", sorted(PINS))
def test_pin(impl, pin):
    fn, tol = PINS[pin]
    err = fn(FORWARDS[impl])
    assert err <= tol, f"{impl} oracle fails pin {pin}: error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(step):
    def fwd(q, k, v, g, beta, S0=None, cu=None):
        orig = kda_oracle.kda_token_step
        kda_oracle.kda_token_step = step
        try:
            return kda_oracle.kda_forward(q, k, v, g, beta, S0, cu)
        finally:
            kda_oracle.kda_token_step = orig
    return fwd


def _read_before_update(S, q, k, v, g, beta, scale=1.0):
    S = np.exp(g)[:, None] * S
    o = S.T @ q
    S = S + np.outer(k, beta * (v - S.T @ k))
    return o, S


def _decay_after_delta(S, q, k, v, g, beta, scale=1.0):
    S = S + np.outer(k, beta * (v - S.T @ k))
    S = np.exp(g)[:, None] * S
    return S.T @ q, S


def _decay_on_columns(S, q, k, v, g, beta, scale=1.0):
    a = np.exp(g)
    S = S * np.resize(a, S.shape[1])[None, :]
    S = S + np.outer(k, beta * (v - S.T @ k))
    return S.T @ q, S


def _sign_flip(S, q, k, v, g, beta, scale=1.0):
    S = np.exp(g)[:, None] * S
    S = S + np.outer(k, beta * (v + S.T @ k))
    return S.T @ q, S


def _residual_on_old_state(S, q, k, v, g, beta, scale=1.0):
    u = beta * (v - S.T @ k)
    S = np.exp(g)[:, None] * S + np.outer(k, u)
    return S.T @ q, S


def _beta_dropped(S, q, k, v, g, beta, scale=1.0):
    S = np.exp(g)[:, None] * S
    S = S + np.outer(k, (v - S.T @ k))
    return S.T @ q, S


def _base2_decay(S, q, k, v, g, beta, scale=1.0):
    S = np.exp2(g)[:, None] * S
    S = S + np.outer(k, beta * (v - S.T @ k))
    return S.T @ q, S


def _transposed_state(S, q, k, v, g, beta, scale=1.0):
    S = np.exp(g)[:, None] * S
    S = S + np.outer(k, beta * (v - S @ k))   # S k in place of S^T k (well-formed when dk = dv)
    return S.T @ q, S


MUTANTS = {
    "read_before_update": _read_before_update,
    "transposed_state": _transposed_state,
    "decay_after_delta": _decay_after_delta,
    "decay_on_columns": _decay_on_columns,
    "sign_flip": _sign_flip,
    "residual_on_old_state": _residual_on_old_state,
    "beta_dropped": _beta_dropped,
    "base2_decay": _base2_decay,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    fwd = _mutant(MUTANTS[name])
    failed = []
    for pin, (fn, tol) in PINS.items():
        if pin in ("chunkwise",):
            continue  # the chunkwise algorithm is independent; compare via closed forms only
        try:
            if fn(fwd) > max(tol, 1e-9):
                failed.append(pin)
        except (AssertionError, ValueError):   # ValueError: a shape the mistake cannot take
            failed.append(pin)
    assert failed, f"planted mistake {name} passes every pin"


def test_column_pin_catches_a_transposed_state_numerically():
    """With dk = dv the transposed-state mistake is well-formed; the permuted-column run alone
    rejects it by value, not by shape."""
    assert pin_column_independence(_mutant(_transposed_state), col_sets=([5, 1, 3, 0, 4, 2],)) > 1e-3


def test_chunkwise_catches_planted_mistakes():
    """The chunkwise cross-check alone also rejects each planted mistake."""
    for name, step in MUTANTS.items():
        try:
            err = pin_chunkwise(_mutant(step), chunks=(16,))
        except ValueError:   # the mistake cannot take this shape (dk != dv): rejected as well
            continue
        assert err > 1e-6, name


# ----------------------------------------------------------------------------- page constants

def test_page_decay_bounds():
    """The numbers printed after eq. (5): exp(-5) ~ 6.7e-3, 16-token log-decay > -80, and
    exp(80) inside the BF16 range; the synthetic gate respects them."""
    d = json.load(open(os.path.join(GOLDEN, "decay_bounds.json")))
    assert abs(math.exp(d["g_min"]) - d["alpha_lower_bound_printed"]) < 0.05e-3
    assert d["tile_tokens"] * d["g_min"] == d["tile_log_decay_lower_bound"]
    assert math.exp(d["reciprocal_bound_log"]) < d["bf16_max"]
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    assert bf16_max == d["bf16_max"]
    from linear_attention_chunkwise_amd import inputs
    x = inputs.make_prefill_inputs(1, 256, 4, 32, 8, seed=3, near_gmin_frac=0.1)
    g = x["g"].double()
    assert float(g.max()) < 0 and float(g.min()) > d["g_min"]
    win = g.unfold(1, 16, 1).sum(-1)
    assert float(win.min()) > d["tile_log_decay_lower_bound"]


def test_c_matches_numpy_on_bf16():
    """The two token loops agree on bf16-stored inputs with packed sequences."""
    from linear_attention_chunkwise_amd import inputs
    cu = inputs.cu_from_lengths([7, 33, 1, 20])
    x = inputs.make_prefill_inputs(1, int(cu[-1]), 3, 16, 12, seed=4, cu_seqlens=cu)
    a = kda_oracle.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], cu)
    b = c_oracle.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], cu)
    assert _rel(b[0], a[0]) < 1e-13 and _rel(b[1], a[1]) < 1e-13


def test_decode_step_is_one_token():
    from linear_attention_chunkwise_amd import inputs
    x = inputs.make_decode_inputs(3, 2, 8, 6, seed=2)
    o, S = kda_oracle.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S"])
    o2, S2 = kda_oracle.kda_forward(x["q"][:, None], x["k"][:, None], x["v"][:, None],
                                    x["g"][:, None], x["beta"][:, None], x["S"])
    assert np.array_equal(o, o2[:, 0]) and np.array_equal(S, S2)


# ----------------------------------------------------------------------------- decay map, eq. (5)

def _gate_pins(gate):
    """Errors of a gate map g(z, A_log) against what eq. (5) and the text after it fix."""
    import scipy.special
    rng = np.random.default_rng(5)
    H, dk = 3, 8
    A = np.array([0.0, 0.7, -1.3])
    z = rng.standard_normal((2, 4, H, dk)) * 3
    errs = {}
    # Sigmoid(0) = 1/2: g = g_min / 2 for every head, whatever A_h is
    errs["zero_logit"] = float(np.abs(gate(np.zeros((1, H, dk)), A) - (-2.5)).max())
    # A_h = 0 (the initialisation the text gives): g_min times the logistic function (scipy)
    g0 = gate(z, np.zeros(H))
    errs["logistic_at_A0"] = float(np.abs(g0 - (-5.0) * scipy.special.expit(z)).max())
    # Sigmoid(x) + Sigmoid(-x) = 1: g(z) + g(-z) = g_min
    errs["reflection"] = float(np.abs(gate(z, A) + gate(-z, A) - (-5.0)).max())
    # exp(A_h) scales the logit of head h only: head h with A_h equals A = 0 on exp(A_h) z
    ga = gate(z, A)
    errs["head_scale"] = max(float(np.abs(ga[..., h, :] - (-5.0) * scipy.special.expit(
        math.exp(A[h]) * z[..., h, :])).max()) for h in range(H))
    # range (g_min, 0) and its limits at saturated logits, without NaN
    zs = np.array([[[-1e4] * dk, [1e4] * dk, [0.0] * dk]]).reshape(1, 3, dk)
    gs = gate(zs, np.zeros(3))
    errs["limits"] = float(abs(gs[0, 0]).max() + abs(gs[0, 1] + 5.0).max())
    errs["range"] = 0.0 if (np.all(ga <= 0) and np.all(ga >= -5.0)) else 1.0
    # monotone: a larger logit never gives a weaker decay
    zz = np.sort(z.reshape(-1))
    gg = gate(zz.reshape(-1, 1, 1) * np.ones((1, 1, 1)), np.array([0.4]))[:, 0, 0]
    errs["monotone"] = 0.0 if np.all(np.diff(gg) <= 0) else 1.0
    return errs


def test_gate_pins():
    for name, err in _gate_pins(kda_oracle.kda_gate).items():
        assert err <= 1e-14, f"gate pin {name}: {err:.3e}"


def test_gate_respects_page_bounds():
    """α = exp(g) > exp(-5) ≈ 6.7e-3 and a 16-token window sums to more than -80 (the numbers
    printed after eq. (5)), on the decay-heavy synthetic recipe (10% of channels at z = +3)."""
    from linear_attention_chunkwise_amd import inputs
    d = json.load(open(os.path.join(GOLDEN, "decay_bounds.json")))
    x = inputs.make_prefill_inputs(1, 256, 4, 32, 8, seed=6, near_gmin_frac=0.1, with_logits=True)
    g = kda_oracle.kda_gate(x["z"], x["A_log"])
    assert np.exp(g).min() > math.exp(d["g_min"]) and g.max() < 0
    win = np.lib.stride_tricks.sliding_window_view(g, 16, axis=1).sum(-1)
    assert win.min() > d["tile_log_decay_lower_bound"]


GATE_MUTANTS = {
    # the unbounded map eq. (5) replaces (negative Softplus, scaled by exp(A_h))
    "softplus_map": lambda z, A: -np.exp(_np(A))[:, None] * np.log1p(np.exp(_np(z))),
    # A_h used as the scale itself instead of exp(A_h)
    "no_exp_on_A": lambda z, A: -5.0 / (1.0 + np.exp(-_np(A)[:, None] * _np(z))),
    # the logistic function mirrored
    "mirrored_sigmoid": lambda z, A: -5.0 / (1.0 + np.exp(np.exp(_np(A))[:, None] * _np(z))),
    # the per-head scale applied along the key channels
    "scale_on_channels": lambda z, A: -5.0 / (1.0 + np.exp(-np.resize(np.exp(_np(A)),
                                                                       _np(z).shape[-1]) * _np(z))),
}


def _np(x):
    return np.asarray(x, np.float64)


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_pins_catch_planted_mistake(name):
    try:
        errs = _gate_pins(GATE_MUTANTS[name])
    except (ValueError, IndexError):
        return  # a shape mistake that cannot even broadcast is caught too
    assert max(errs.values()) > 1e-6, f"planted gate mistake {name} passes every pin"


def test_c_oracle_takes_float64_decay():
    """The C token loop reads float64 g (the eq. (5) map evaluated in double) like float32 g."""
    from linear_attention_chunkwise_amd import inputs
    x = inputs.make_prefill_inputs(2, 19, 2, 16, 8, seed=7, with_logits=True)
    g = kda_oracle.kda_gate(x["z"], x["A_log"])
    a = kda_oracle.kda_forward(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    b = c_oracle.kda_forward(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    assert _rel(b[0], a[0]) < 1e-13 and _rel(b[1], a[1]) < 1e-13


# ----------------------------------------------------------------------------- fused decode steps

def _fused_pins(l2norm, sigmoid, gated_rmsnorm):
    import scipy.special
    import sklearn.preprocessing
    rng = np.random.default_rng(9)
    errs = {}
    x = rng.standard_normal((5, 3, 16)) * 2.0
    # L2Norm against scikit-learn's row normalisation; unit norm; invariant to positive scale;
    # a zero vector stays zero (the floor), never NaN
    ref = sklearn.preprocessing.normalize(x.reshape(-1, 16)).reshape(x.shape)
    errs["l2_sklearn"] = float(np.abs(l2norm(x) - ref).max())
    errs["l2_scale"] = float(np.abs(l2norm(3.7 * x) - l2norm(x)).max())
    zv = l2norm(np.zeros((2, 16)))
    errs["l2_zero"] = 0.0 if np.all(zv == 0) else 1.0
    # Sigmoid against scipy
    errs["sigmoid"] = float(np.abs(sigmoid(x) - scipy.special.expit(x)).max())
    # Sigmoid(G) * RMSNorm(o) * w against torch's rms_norm (float64)
    o = rng.standard_normal((4, 2, 32))
    G = rng.standard_normal((4, 2, 32))
    w = rng.standard_normal(32)
    t = torch.nn.functional.rms_norm(torch.from_numpy(o), (32,), torch.from_numpy(w), 1e-6).numpy()
    errs["rms_torch"] = float(np.abs(gated_rmsnorm(o, G, w, 1e-6) - scipy.special.expit(G) * t).max())
    # closed form: a constant vector c with G = 0 and no weight gives 0.5 c / sqrt(c^2 + eps)
    c = np.full((1, 8), -2.5)
    errs["rms_const"] = float(np.abs(gated_rmsnorm(c, np.zeros((1, 8)), None, 1e-6)
                                     - 0.5 * (-2.5) / math.sqrt(6.25 + 1e-6)).max())
    return errs


def test_fused_decode_pins():
    errs = _fused_pins(kda_oracle.l2norm, kda_oracle.sigmoid, kda_oracle.gated_rmsnorm)
    for name, err in errs.items():
        assert err <= 1e-12, f"fused pin {name}: {err:.3e}"


FUSED_MUTANTS = {
    "l2_no_floor": (lambda x: _np(x) / np.sqrt((_np(x) ** 2).sum(-1, keepdims=True)), None, None),
    "rms_mean_removed": (None, None, lambda o, G, w=None, eps=1e-6: kda_oracle.sigmoid(G) * (
        (_np(o) - _np(o).mean(-1, keepdims=True)) / np.sqrt(_np(o).var(-1, keepdims=True) + eps)
        * (1.0 if w is None else _np(w)))),
    "weight_inside": (None, None, lambda o, G, w=None, eps=1e-6: kda_oracle.gated_rmsnorm(
        _np(o) * (1.0 if w is None else _np(w)), G, None, eps)),
    "gate_mirrored": (None, lambda x: 1.0 / (1.0 + np.exp(_np(x))), None),
}


@pytest.mark.parametrize("name", sorted(FUSED_MUTANTS))
def test_fused_pins_catch_planted_mistake(name):
    import warnings
    l2, sg, rms = FUSED_MUTANTS[name]
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        errs = _fused_pins(l2 or kda_oracle.l2norm, sg or kda_oracle.sigmoid,
                           rms or kda_oracle.gated_rmsnorm)
    assert any(not (e <= 1e-6) for e in errs.values()), f"planted mistake {name} passes every pin"


def test_fused_decode_invariants():
    """Positive rescaling of the raw q and k changes nothing (they are L2-normalised); n_commit = 0
    leaves the state; K tokens at once equal K single-token calls."""
    from linear_attention_chunkwise_amd import inputs
    x = inputs.make_prefill_inputs(2, 3, 2, 16, 8, dtype=torch.float32, seed=12, with_logits=True)
    rng = np.random.default_rng(4)
    b = rng.standard_normal((2, 3, 2))
    G = rng.standard_normal((2, 3, 2, 8))
    w = rng.standard_normal(8)
    args = (x["v"], x["z"], x["A_log"], b, x["S0"], G, w)
    y1, s1 = kda_oracle.kda_fused_decode(x["q"], x["k"], *args)
    y2, s2 = kda_oracle.kda_fused_decode(_np(x["q"]) * 2.5, _np(x["k"]) * 0.3, *args)
    assert np.abs(y1 - y2).max() < 1e-12 and np.abs(s1 - s2).max() < 1e-12
    _, s0 = kda_oracle.kda_fused_decode(x["q"], x["k"], *args, n_commit=[0, 0])
    assert np.array_equal(s0, _np(x["S0"]))
    S = _np(x["S0"])
    for t in range(3):
        sl = lambda a: _np(a)[:, t:t + 1]
        yt, S = kda_oracle.kda_fused_decode(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["z"]),
                                            x["A_log"], b[:, t:t + 1], S, G[:, t:t + 1], w)
        assert np.abs(yt[:, 0] - y1[:, t]).max() < 1e-12
    assert np.abs(S - s1).max() < 1e-12


# ------------------------------------------------------------------ short convolution (eq. (2))

def _conv_pins(conv, sw):
    """Errors of a short-convolution / Swish pair against library routines and closed forms."""
    import scipy.signal
    rng = np.random.default_rng(21)
    errs = {}
    N, K, H, C, W = 2, 7, 3, 5, 4
    x = rng.standard_normal((N, K, H, C))
    w = rng.standard_normal((H, C, W))
    st = rng.standard_normal((N, H, C, W - 1))
    y, xx = conv(x, w, st)
    ref_np = np.zeros_like(y)
    ref_lf = np.zeros_like(y)
    for n in range(N):
        for h in range(H):
            for c in range(C):
                series = np.concatenate([st[n, h, c], x[n, :, h, c]])
                # numpy.convolve flips its second argument: reversed taps give sum_j w_j xx_{t+j}
                ref_np[n, :, h, c] = np.convolve(series, w[h, c][::-1], mode="valid")
                # an FIR filter y[m] = sum_k b_k s[m - k] with b = reversed taps, from m = W - 1 on
                ref_lf[n, :, h, c] = scipy.signal.lfilter(w[h, c][::-1], [1.0], series)[W - 1:]
    errs["conv_numpy"] = float(np.abs(y - ref_np).max())
    errs["conv_lfilter"] = float(np.abs(y - ref_lf).max())
    # the returned history: state, then the inputs
    errs["history"] = float(np.abs(xx[..., W - 1:] - np.transpose(x, (0, 2, 3, 1))).max()
                            + np.abs(xx[..., :W - 1] - st).max())
    # a one-tap filter scales each input; a delta tap at position 0 returns the input W-1 back
    y1, _ = conv(x, w[..., -1:], None)
    errs["one_tap"] = float(np.abs(y1 - x * w[None, None, :, :, -1]).max())
    d = np.zeros((H, C, W))
    d[..., 0] = 1.0
    yd, _ = conv(x, d, st)
    errs["delta_back"] = float(np.abs(yd[:, W - 1:] - x[:, :K - W + 1]).max()
                               + np.abs(yd[:, 0] - np.transpose(st[..., 0], (0, 1, 2))).max())
    # resume: the first m tokens, then the rest entered with the window after m
    m = 3
    ya, xa = conv(x[:, :m], w, st)
    yb, _ = conv(x[:, m:], w, xa[..., m:m + W - 1])
    errs["resume"] = float(np.abs(np.concatenate([ya, yb], 1) - y).max())
    # Swish against torch's silu and the definition with scipy's logistic
    import scipy.special
    z = rng.standard_normal(50) * 4
    errs["swish_torch"] = float(np.abs(sw(z) - torch.nn.functional.silu(torch.from_numpy(z)).numpy()).max())
    errs["swish_expit"] = float(np.abs(sw(z) - z * scipy.special.expit(z)).max())
    return errs


def test_short_conv_pins():
    errs = _conv_pins(kda_oracle.short_conv, kda_oracle.swish)
    for name, err in errs.items():
        assert err <= 1e-12, f"short-conv pin {name}: {err:.3e}"


def _conv_off_by_one(x, w, state=None):
    y, xx = kda_oracle.short_conv(x, w, state)
    W = _np(w).shape[-1]
    yy = np.zeros_like(y)
    for t in range(y.shape[1]):          # window one token late: drops the current input
        lo = max(0, t - 1)
        yy[:, t] = (xx[..., lo:lo + W] * _np(w)[None]).sum(-1)
    return yy, xx


def _conv_taps_unreversed(x, w, state=None):
    return kda_oracle.short_conv(x, _np(w)[..., ::-1], state)


CONV_MUTANTS = {
    "window_off_by_one": (_conv_off_by_one, None),
    "taps_reversed": (_conv_taps_unreversed, None),
    "swish_is_sigmoid": (None, kda_oracle.sigmoid),
}


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_pins_catch_planted_mistake(name):
    conv, sw = CONV_MUTANTS[name]
    errs = _conv_pins(conv or kda_oracle.short_conv, sw or kda_oracle.swish)
    assert any(not (e <= 1e-6) for e in errs.values()), f"planted mistake {name} passes every pin"


def test_fused_decode_with_conv_composes():
    """The fused decode with the short convolution equals the fused decode without it on the
    convolved, Swish-activated projections; the window it returns is the inputs around the
    committed prefix; K tokens at once equal token-by-token calls that carry state and window."""
    rng = np.random.default_rng(31)
    N, K, H, dk, dv, W = 2, 4, 2, 8, 6, 4
    C = 2 * dk + dv
    pq, pk = rng.standard_normal((N, K, H, dk)), rng.standard_normal((N, K, H, dk))
    pv = rng.standard_normal((N, K, H, dv))
    z = rng.standard_normal((N, K, H, dk))
    A = rng.standard_normal(H) * 0.5
    b = rng.standard_normal((N, K, H))
    G = rng.standard_normal((N, K, H, dv))
    S = rng.standard_normal((N, H, dk, dv)) * 0.1
    cw = rng.standard_normal((H, C, W)) * 0.5
    cs = rng.standard_normal((N, H, C, W - 1))
    nc = [2, 4]
    y, s1, win = kda_oracle.kda_fused_decode(pq, pk, pv, z, A, b, S, G, None, 1e-6, 1.0, nc, cw, cs)
    cq, _ = kda_oracle.short_conv(pq, cw[:, :dk], cs[:, :, :dk])
    ck, _ = kda_oracle.short_conv(pk, cw[:, dk:2 * dk], cs[:, :, dk:2 * dk])
    cv, _ = kda_oracle.short_conv(pv, cw[:, 2 * dk:], cs[:, :, 2 * dk:])
    y2, s2 = kda_oracle.kda_fused_decode(kda_oracle.swish(cq), kda_oracle.swish(ck), kda_oracle.swish(cv),
                                         z, A, b, S, G, None, 1e-6, 1.0, nc)
    assert np.abs(y - y2).max() < 1e-12 and np.abs(s1 - s2).max() < 1e-12
    for n, c in enumerate(nc):
        series = np.concatenate([cs[n], np.concatenate([np.transpose(a[n], (1, 2, 0)) for a in (pq, pk, pv)], 1)], -1)
        assert np.array_equal(win[n], series[..., c:c + W - 1])
    Sc, Wc = S, cs
    for t in range(K):
        sl = lambda a: a[:, t:t + 1]
        yt, Sc, Wc = kda_oracle.kda_fused_decode(sl(pq), sl(pk), sl(pv), sl(z), A, sl(b), Sc, sl(G),
                                                 None, 1e-6, 1.0, None, cw, Wc)
        assert np.abs(yt[:, 0] - y[:, t]).max() < 1e-12
    _, s_all, w_all = kda_oracle.kda_fused_decode(pq, pk, pv, z, A, b, S, G, None, 1e-6, 1.0, None, cw, cs)
    assert np.abs(Sc - s_all).max() < 1e-12 and np.abs(Wc - w_all).max() < 1e-12
