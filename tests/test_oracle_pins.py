"""Pins of the float64 CPU oracle against facts that do not come from the oracle.

Each check is written against an independent statement: a hand-derived worked
example, an algebraic identity of the delta rule, a special case that reduces
to a textbook method (DeltaNet, a one-dimensional exponential moving average,
cumulative linear attention), exact rational brute force, or an invariance of
the method.  ``test_mutants_are_caught`` plants plausible mistakes in copies of
the oracle's step and checks that the same pins reject every one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.kda_oracle import gate_rmsnorm, kda_chunked, kda_decode_step, kda_recurrent
from oracle.kda_rational import rational_kda

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def rand_inputs(rng, B, T, H, dk, dv, g_std=1.0, s0_std=None, unit=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 / (1.0 + np.exp(-g_std * rng.standard_normal((B, T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = None if s0_std is None else s0_std * rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, s0


def fwd_from_step(step):
    """Sequence forward built from any single-token step (used for mutants)."""
    def fwd(q, k, v, g, beta, s0=None, scale=1.0):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
        o = np.zeros((B, T, H, dv))
        for t in range(T):
            o[:, t], S = step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S, scale)
        return o, S
    return fwd


# ----------------------------------------------------------------------------- checks
# Each check takes a sequence forward ``fwd`` and raises AssertionError on failure.

def check_worked_example(fwd):
    """Two tokens worked by hand (tests/golden/worked_example_2x2.json)."""
    with open(os.path.join(GOLDEN, "worked_example_2x2.json")) as f:
        ex = json.load(f)
    sh = lambda x: np.array(x, dtype=np.float64)[None, :, None, :]  # noqa: E731
    g = np.log(np.array(ex["alpha"]))[None, :, None, :]
    beta = np.array(ex["beta"])[None, :, None]
    s0 = np.array(ex["s0"])[None, None]
    o, S = fwd(sh(ex["q"]), sh(ex["k"]), sh(ex["v"]), g, beta, s0)
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["expected_o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], np.array(ex["expected_state"]), rtol=0, atol=1e-12)


def check_exact_overwrite(fwd):
    """P1: beta=1 and a unit key make the state return exactly v for that key:
    k^T (I - k k^T) = 0, so S_t^T k_t = v_t whatever alpha and S_{t-1}."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, s0 = rand_inputs(rng, 1, 9, 2, 8, 6, s0_std=0.5)
    t = 6
    beta[:, t] = 1.0
    q[:, t] = k[:, t]
    o, _ = fwd(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o[:, t], v[:, t], rtol=0, atol=1e-12)
    # the state after token t, read back with k_t, is v_t
    _, S = fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1], beta[:, :t + 1], s0)
    np.testing.assert_allclose(np.einsum("bhkv,bhk->bhv", S, k[:, t]), v[:, t], atol=1e-12)


def check_deltanet(fwd):
    """P2: g = 0 (alpha = 1) is plain DeltaNet.  The textbook form keeps the
    transposed state M in R^{dv x dk}: M_t = M_{t-1}(I - b k k^T) + b v k^T,
    o_t = M_t q_t."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, s0 = rand_inputs(rng, 2, 11, 2, 5, 7, s0_std=0.3)
    g[:] = 0.0
    o, S = fwd(q, k, v, g, beta, s0)
    B, T, H, dk = q.shape
    for b in range(B):
        for h in range(H):
            M = s0[b, h].T.copy()
            for t in range(T):
                kk = k[b, t, h]
                M = M @ (np.eye(dk) - beta[b, t, h] * np.outer(kk, kk)) + \
                    beta[b, t, h] * np.outer(v[b, t, h], kk)
                np.testing.assert_allclose(o[b, t, h], M @ q[b, t, h], atol=1e-12)
            np.testing.assert_allclose(S[b, h], M.T, atol=1e-12)


def check_one_hot_keys_ema(fwd):
    """P3: with one-hot keys the key channels decouple.  Row i of the state is
    a 1-D exponential moving average: it decays by alpha_{t,i} every token and,
    when key i is written, becomes (1 - beta) * alpha * row + beta * v.  This
    fixes which axis the per-channel decay scales (rows = key channels)."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 1, 12, 1, 4, 3
    q, _, v, g, beta, s0 = rand_inputs(rng, B, T, H, dk, dv, s0_std=1.0)
    which = rng.integers(0, dk, size=T)
    k = np.zeros((B, T, H, dk))
    k[0, np.arange(T), 0, which] = 1.0
    o, S = fwd(q, k, v, g, beta, s0)
    rows = s0[0, 0].copy()
    for t in range(T):
        a = np.exp(g[0, t, 0])
        for i in range(dk):
            if i == which[t]:
                rows[i] = (1 - beta[0, t, 0]) * a[i] * rows[i] + beta[0, t, 0] * v[0, t, 0]
            else:
                rows[i] = a[i] * rows[i]
        np.testing.assert_allclose(o[0, t, 0], rows.T @ q[0, t, 0], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], rows, atol=1e-12)


def check_beta_zero_closed_form(fwd):
    """P4a: beta = 0 removes every write, so S_t = Diag(exp(sum_{s<=t} g_s)) S_0."""
    rng = np.random.default_rng(14)
    q, k, v, g, beta, s0 = rand_inputs(rng, 1, 10, 3, 6, 5, s0_std=1.0)
    beta[:] = 0.0
    o, S = fwd(q, k, v, g, beta, s0)
    G = np.cumsum(g, axis=1)                                        # [B,T,H,dk]
    St = np.exp(G)[..., None] * s0[:, None]                         # [B,T,H,dk,dv]
    np.testing.assert_allclose(o, np.einsum("bthkv,bthk->bthv", St, q), atol=1e-12)
    np.testing.assert_allclose(S, St[:, -1], atol=1e-12)


def check_orthogonal_keys_linear_attention(fwd):
    """P4b: with mutually orthogonal unit keys, alpha = 1 and a zero start state
    the erase never touches earlier writes, so the output is cumulative linear
    attention o_t = sum_{s<=t} beta_s (q_t . k_s) v_s."""
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 1, 6, 1, 8, 5
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis.T[:T][None, :, None, :]
    q = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = np.zeros((B, T, H, dk))
    beta = rng.uniform(0.1, 0.9, size=(B, T, H))
    o, _ = fwd(q, k, v, g, beta, None)
    for t in range(T):
        expect = sum(beta[0, s, 0] * (q[0, t, 0] @ k[0, s, 0]) * v[0, s, 0] for s in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], expect, atol=1e-12)


def check_rational_brute_force(fwd):
    """P11: exact rational arithmetic on a tiny case (dk = dv = 4, T = 6) with
    rational unit keys, rational alpha and beta, and dense transition-matrix
    products; the float64 forward must agree to 1e-13 relative."""
    F = Fraction
    keys = [(F(1, 3), F(2, 3), F(2, 3), F(0)), (F(0), F(3, 5), F(4, 5), F(0)),
            (F(2, 7), F(3, 7), F(0), F(6, 7)), (F(1, 2), F(1, 2), F(1, 2), F(1, 2)),
            (F(4, 9), F(0), F(4, 9), F(7, 9)), (F(0), F(0), F(1), F(0))]
    T, dk, dv = len(keys), 4, 4
    rng = np.random.default_rng(16)
    rint = lambda lo, hi: F(int(rng.integers(lo, hi)), 8)  # noqa: E731
    q = [[rint(-8, 9) for _ in range(dk)] for _ in range(T)]
    v = [[rint(-8, 9) for _ in range(dv)] for _ in range(T)]
    alpha = [[F(int(rng.integers(1, 9)), 8) for _ in range(dk)] for _ in range(T)]
    beta = [F(int(rng.integers(1, 8)), 8) for _ in range(T)]
    s0 = [[rint(-8, 9) for _ in range(dv)] for _ in range(dk)]
    o_ex, S_ex = rational_kda(q, keys, v, alpha, beta, s0)
    fl = lambda x: np.array([[float(e) for e in r] for r in x])  # noqa: E731
    o, S = fwd(fl(q)[None, :, None], fl(keys)[None, :, None], fl(v)[None, :, None],
               np.log(fl(alpha))[None, :, None], np.array([float(b) for b in beta])[None, :, None],
               fl(s0)[None, None])
    o_ex, S_ex = fl(o_ex), fl(S_ex)
    np.testing.assert_allclose(o[0, :, 0], o_ex, rtol=1e-13, atol=1e-13 * np.abs(o_ex).max())
    np.testing.assert_allclose(S[0, 0], S_ex, rtol=1e-13, atol=1e-13 * np.abs(S_ex).max())


CHECKS = [check_worked_example, check_exact_overwrite, check_deltanet, check_one_hot_keys_ema,
          check_beta_zero_closed_form, check_orthogonal_keys_linear_attention,
          check_rational_brute_force]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(kda_recurrent)


# ----------------------------------------------------------------------------- chunked form
@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16, 53])
def test_chunked_matches_recurrent(chunk):
    """P5: the chunkwise rewrite equals the token recurrence for every chunk
    size (the result must not depend on the tile), here with a ragged tail."""
    rng = np.random.default_rng(17)
    q, k, v, g, beta, s0 = rand_inputs(rng, 2, 53, 2, 8, 6, s0_std=0.2)
    o_r, S_r = kda_recurrent(q, k, v, g, beta, s0, scale=0.7)
    o_c, S_c = kda_chunked(q, k, v, g, beta, s0, scale=0.7, chunk=chunk)
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-12)


def test_chunked_decay_floor_tile():
    """Whole key channels at g = -4.999 for a full 16-token tile (cumulative
    log-decay near -80): the chunked rewrite still agrees with the recurrence."""
    rng = np.random.default_rng(18)
    q, k, v, g, beta, s0 = rand_inputs(rng, 1, 48, 1, 16, 8, s0_std=0.1)
    g[..., ::5] = -4.999
    o_r, S_r = kda_recurrent(q, k, v, g, beta, s0)
    o_c, S_c = kda_chunked(q, k, v, g, beta, s0, chunk=16)
    scale = np.sqrt(np.mean(o_r ** 2))
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_r, rtol=0, atol=1e-10 * scale)
    np.testing.assert_allclose(S_c, S_r, rtol=0, atol=1e-10)


# ----------------------------------------------------------------------------- invariances
def test_continuation():
    """P6: running [0, T1) then [T1, T) from the carried state equals one run
    (the initial/final state is what a prefix cache stores)."""
    rng = np.random.default_rng(19)
    q, k, v, g, beta, s0 = rand_inputs(rng, 1, 40, 3, 8, 8, s0_std=0.2)
    o, S = kda_recurrent(q, k, v, g, beta, s0)
    o1, S1 = kda_recurrent(q[:, :17], k[:, :17], v[:, :17], g[:, :17], beta[:, :17], s0)
    o2, S2 = kda_recurrent(q[:, 17:], k[:, 17:], v[:, 17:], g[:, 17:], beta[:, 17:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-13)
    np.testing.assert_allclose(S2, S, atol=1e-13)


def test_identity_tokens():
    """P8: a token with g = 0 and beta = 0 leaves the state exactly unchanged
    whatever its key (the padding a partial last tile relies on)."""
    rng = np.random.default_rng(20)
    q, k, v, g, beta, s0 = rand_inputs(rng, 1, 5, 2, 6, 4, s0_std=1.0)
    g[:] = 0.0
    beta[:] = 0.0
    _, S = kda_recurrent(q, k, v, g, beta, s0)
    assert np.array_equal(S, s0)


def test_linearity_and_permutation():
    """P12: for fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear, and
    permuting heads permutes the outputs."""
    rng = np.random.default_rng(21)
    q, k, v1, g, beta, s1 = rand_inputs(rng, 1, 12, 3, 6, 5, s0_std=0.5)
    v2 = rng.standard_normal(v1.shape)
    s2 = rng.standard_normal(s1.shape)
    a, b = 0.7, -1.3
    o1, S1 = kda_recurrent(q, k, v1, g, beta, s1)
    o2, S2 = kda_recurrent(q, k, v2, g, beta, s2)
    o, S = kda_recurrent(q, k, a * v1 + b * v2, g, beta, a * s1 + b * s2)
    np.testing.assert_allclose(o, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(S, a * S1 + b * S2, atol=1e-12)
    perm = [2, 0, 1]
    op, Sp = kda_recurrent(q[:, :, perm], k[:, :, perm], v1[:, :, perm], g[:, :, perm],
                           beta[:, :, perm], s1[:, perm])
    np.testing.assert_allclose(op, o1[:, :, perm], atol=1e-14)
    np.testing.assert_allclose(Sp, S1[:, perm], atol=1e-14)


def test_decode_step_is_one_token():
    """A decode step on a resident state equals a one-token sequence."""
    rng = np.random.default_rng(22)
    q, k, v, g, beta, s0 = rand_inputs(rng, 3, 1, 2, 8, 8, s0_std=0.5)
    o, S = kda_decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], s0)
    o_r, S_r = kda_recurrent(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o, o_r[:, 0], atol=0)
    np.testing.assert_allclose(S, S_r, atol=0)


# ----------------------------------------------------------------------------- epilogue
def test_gate_rmsnorm_closed_forms():
    """P10: norm first, then the sigmoid gate ("after head-wise RMSNorm").
    A worked row: x = (3, 4), eps = 0: rms = sqrt(12.5); gate 0 halves it;
    a very large gate leaves x / rms; the normalised row has RMS
    rms / sqrt(rms^2 + eps)."""
    x = np.array([[3.0, 4.0]])
    r = math.sqrt(12.5)
    np.testing.assert_allclose(gate_rmsnorm(x, np.zeros((1, 2)), eps=0.0),
                               [[0.5 * 3 / r, 0.5 * 4 / r]], rtol=1e-15)
    np.testing.assert_allclose(gate_rmsnorm(x, np.full((1, 2), 60.0), eps=0.0),
                               [[3 / r, 4 / r]], rtol=1e-15)
    np.testing.assert_allclose(gate_rmsnorm(x, np.full((1, 2), 60.0), weight=[2.0, -1.0], eps=0.0),
                               [[6 / r, -4 / r]], rtol=1e-15)
    rng = np.random.default_rng(23)
    x = 1e-3 * rng.standard_normal((4, 16))
    eps = 1e-6
    y = gate_rmsnorm(x, np.full_like(x, 60.0), eps=eps)
    ms = np.mean(x ** 2, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y ** 2, axis=-1)), np.sqrt(ms / (ms + eps)),
                               rtol=1e-14)


# ----------------------------------------------------------------------------- mutation test
def _mut_erase_before_decay(q, k, v, g, beta, S, scale=1.0):
    pred = np.einsum("...kv,...k->...v", S, k)
    S = S + k[..., :, None] * (beta[..., None] * (v - pred))[..., None, :]
    S = np.exp(g)[..., :, None] * S
    return scale * np.einsum("...kv,...k->...v", S, q), S


def _mut_decay_on_columns(q, k, v, g, beta, S, scale=1.0):
    S = np.exp(g)[..., None, :] * S if S.shape[-1] == S.shape[-2] else S
    pred = np.einsum("...kv,...k->...v", S, k)
    S = S + k[..., :, None] * (beta[..., None] * (v - pred))[..., None, :]
    return scale * np.einsum("...kv,...k->...v", S, q), S


def _mut_no_beta(q, k, v, g, beta, S, scale=1.0):
    return kda_decode_step(q, k, v, g, np.ones_like(beta), S, scale)


def _mut_output_before_write(q, k, v, g, beta, S, scale=1.0):
    Sd = np.exp(g)[..., :, None] * S
    o = scale * np.einsum("...kv,...k->...v", Sd, q)
    _, S_new = kda_decode_step(q, k, v, g, beta, S, scale)
    return o, S_new


def _mut_sign_flip(q, k, v, g, beta, S, scale=1.0):
    S = np.exp(g)[..., :, None] * S
    pred = np.einsum("...kv,...k->...v", S, k)
    S = S + k[..., :, None] * (beta[..., None] * (v + pred))[..., None, :]
    return scale * np.einsum("...kv,...k->...v", S, q), S


def _mut_predict_undecayed(q, k, v, g, beta, S, scale=1.0):
    pred = np.einsum("...kv,...k->...v", S, k)
    S = np.exp(g)[..., :, None] * S
    S = S + k[..., :, None] * (beta[..., None] * (v - pred))[..., None, :]
    return scale * np.einsum("...kv,...k->...v", S, q), S


def _mut_inverse_decay(q, k, v, g, beta, S, scale=1.0):
    return kda_decode_step(q, k, v, -g, beta, S, scale)


def _mut_output_with_query_as_key(q, k, v, g, beta, S, scale=1.0):
    o, S_new = kda_decode_step(q, k, v, g, beta, S, scale)
    return scale * np.einsum("...kv,...k->...v", S_new, k), S_new


MUTANTS = [_mut_erase_before_decay, _mut_decay_on_columns, _mut_no_beta,
           _mut_output_before_write, _mut_sign_flip, _mut_predict_undecayed,
           _mut_inverse_decay, _mut_output_with_query_as_key]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutants_are_caught(mutant):
    """A plausible mistake planted in a copy of the oracle's step must fail at
    least one pin; otherwise the pins would not be pinning anything."""
    fwd = fwd_from_step(mutant)
    failures = 0
    for check in CHECKS:
        try:
            check(fwd)
        except AssertionError:
            failures += 1
    assert failures > 0, f"{mutant.__name__} passed every pin"


def test_decay_gates_closed_forms():
    """g = -5 sigmoid(a), beta = sigmoid(b): values at 0 and the limits, the
    bound g in (-5, 0), monotonicity, and sigmoid(x) + sigmoid(-x) = 1."""
    from oracle.kda_oracle import decay_gates
    g, beta = decay_gates(np.array([0.0, 40.0, -40.0]), np.array([0.0, 40.0, -40.0]))
    assert g[0] == -2.5 and beta[0] == 0.5
    assert abs(g[1] + 5.0) < 1e-15 and abs(g[2]) < 1e-16
    assert abs(beta[1] - 1.0) < 1e-15 and beta[2] < 1e-17
    x = np.linspace(-30, 30, 601)
    g, beta = decay_gates(x, x)
    assert np.all(g > -5.0) and np.all(g < 0.0) and np.all(np.diff(g) < 0)
    gm, bm = decay_gates(-x, -x)
    assert np.allclose(beta + bm, 1.0, atol=1e-15)
    assert np.allclose(g + gm, -5.0, atol=1e-14)
    # ln 3 maps to sigmoid = 3/4 exactly (up to rounding): g = -3.75
    g, beta = decay_gates(np.log(3.0), np.log(3.0))
    assert abs(g + 3.75) < 1e-15 and abs(beta - 0.75) < 1e-16


def test_l2_normalize_pins():
    """Unit norm, direction kept, a zero vector stays zero, scale invariance,
    and the 3-4-5 triangle exactly."""
    from oracle.kda_oracle import l2_normalize
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 7, 16))
    y = l2_normalize(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-15)
    assert np.allclose(np.sum(y * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    assert np.allclose(l2_normalize(3.7 * x), y, atol=1e-15)
    assert np.all(l2_normalize(np.zeros((2, 4))) == 0.0)
    assert np.array_equal(l2_normalize(np.array([3.0, 4.0])), np.array([0.6, 0.8]))


# ----------------------------------------------------------------------------- gradient oracle
def _vjp_case(seed, B=1, T=3, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    x = {"q": rng.normal(size=(B, T, H, dk)), "k": rng.normal(size=(B, T, H, dk)) / 2,
         "v": rng.normal(size=(B, T, H, dv)), "g": -5.0 / (1 + np.exp(-rng.normal(size=(B, T, H, dk)))),
         "beta": 1.0 / (1 + np.exp(-rng.normal(size=(B, T, H)))),
         "s0": 0.5 * rng.normal(size=(B, H, dk, dv))}
    do = rng.normal(size=(B, T, H, dv))
    dsf = rng.normal(size=(B, H, dk, dv))
    return x, do, dsf


def test_vjp_central_differences():
    """Every gradient element of kda_recurrent_vjp (autograd through a torch
    loop) against a central difference of the NumPy forward kda_recurrent
    (independent code), for L = sum(o * do) + sum(S_T * dS_T) and scale 0.7."""
    from oracle.kda_oracle_grad import kda_recurrent_vjp
    x, do, dsf = _vjp_case(11)
    scale = 0.7

    def loss(xx):
        o, S = kda_recurrent(xx["q"], xx["k"], xx["v"], xx["g"], xx["beta"], xx["s0"], scale)
        return float(np.sum(o * do) + np.sum(S * dsf))

    got = kda_recurrent_vjp(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], do, dsf, scale)
    h = 1e-5
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("s0", "ds0")]:
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert got[key].shape == x[name].shape
        np.testing.assert_allclose(got[key], fd, rtol=1e-6, atol=1e-8, err_msg=key)


def test_vjp_single_token_closed_form():
    """One token: S_1 = M S_0 + beta k v^T with M = (I - beta k k^T) Diag(a),
    o = scale S_1^T q.  From S_0 = 0: dv = scale beta (k.q) do,
    dq = scale beta (v.do) k, dk = scale beta (v.do) q, dbeta = scale (k.q)(v.do),
    dg = 0 (the decay multiplies a zero state), and for any S_0
    dS_0 = M^T (scale q do^T) = Diag(a) (I - beta k k^T) scale q do^T."""
    from oracle.kda_oracle_grad import kda_recurrent_vjp
    rng = np.random.default_rng(5)
    dk, dv, scale = 4, 3, 1.3
    q, k, v = rng.normal(size=dk), rng.normal(size=dk), rng.normal(size=dv)
    g, beta, do = -rng.uniform(0.1, 5.0, size=dk), 0.6, rng.normal(size=dv)
    r = lambda a: a.reshape(1, 1, 1, -1)  # noqa: E731
    got = kda_recurrent_vjp(r(q), r(k), r(v), r(g), np.full((1, 1, 1), beta), None, r(do),
                            None, scale)
    kq, vd = k @ q, v @ do
    np.testing.assert_allclose(got["dv"].ravel(), scale * beta * kq * do, rtol=1e-12)
    np.testing.assert_allclose(got["dq"].ravel(), scale * beta * vd * k, rtol=1e-12)
    np.testing.assert_allclose(got["dk"].ravel(), scale * beta * vd * q, rtol=1e-12)
    np.testing.assert_allclose(got["dbeta"].ravel(), [scale * kq * vd], rtol=1e-12)
    np.testing.assert_array_equal(got["dg"], np.zeros((1, 1, 1, dk)))
    M = (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(g))
    np.testing.assert_allclose(got["ds0"][0, 0], M.T @ (scale * np.outer(q, do)), rtol=1e-12,
                               atol=1e-15)
