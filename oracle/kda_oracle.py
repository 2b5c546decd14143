"""CPU oracle for the Kimi Delta Attention (KDA) layer core.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
link this module; only the test suite, the smoke check and the CPU-baseline leg
of the benchmark use it.  It is deliberately plain and slow: float64 NumPy,
one token at a time, no blocking, no fusion, no reordering.

What is computed
----------------
The pages describe KDA in prose only:

* "Kimi K3 from Moonshot AI: 2.8 Trillion Parameters Unveiled", section
  "Kimi Delta Attention (KDA)": a delta rule built on the generalized
  Householder transformation, derived from Gated DeltaNet, with a chunkwise
  ("piecewise parallel") reformulation.
* "Kimi K3 Architecture Explained: KDA, Attention Residuals and LatentMoE",
  section "Token mixing: what KDA is and why 3:1": a fixed-size recurrent
  state, an error-correcting write that replaces what the state predicts for a
  key, a forget gate that acts per channel, log-decay bounded below by a scaled
  sigmoid, and an output gate applied after a head-wise RMSNorm.
* "Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
  "Dimension 1: Sequence Length via Hybrid KDA-Gated MLA": channel-wise
  forget gate, g_min = -5 so every retention factor exceeds e^-5.

Written out, with a state S in R^{dk x dv} whose rows are key channels,
alpha_t = exp(g_t) in R^dk and beta_t a scalar per token and head:

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t

Readings taken where the pages are silent (each one is listed in the design
notes of the repository as well):

* decay acts first, then the Householder erase/write (the erase sees the
  decayed state);
* the state's rows are key channels, so Diag(alpha) scales rows and
  o = S^T q has dv entries;
* ``scale`` multiplies the output; the pages print no 1/sqrt(dk) factor, so
  the parity workloads use scale = 1;
* the epilogue is RMSNorm over one head's dv vector (eps added to the mean
  square, inside the square root), times a weight, times sigmoid(gate).

Layouts (all contiguous, row-major):
    q, k  [B, T, H, dk]     v [B, T, H, dv]     g [B, T, H, dk]
    beta  [B, T, H]         s0 / state [B, H, dk, dv]
    o     [B, T, H, dv]     gate [B, T, H, dv]

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, special cases that reduce to textbook methods (DeltaNet, a 1-D
exponential moving average, cumulative linear attention), exact rational brute
force and a hand-derived worked example.  None is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kda_decode_step",
    "kda_recurrent",
    "gate_rmsnorm",
    "kda_chunked",
    "decay_gates",
    "l2_normalize",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def kda_decode_step(q, k, v, g, beta, state, scale=1.0):
    """One token of the recurrence for every (batch, head) at once.

    The single-token update of the fixed-size state (constant per-token cost,
    "Kimi K3 Architecture Explained ...", section "Token mixing").

    q, k: [..., dk]; v: [..., dv]; g: [..., dk]; beta: [...];
    state: [..., dk, dv].  Returns (o [..., dv], new_state [..., dk, dv]) in
    float64; the input state is not modified.
    """
    q, k, v, g, beta, S = map(_f64, (q, k, v, g, beta, state))
    alpha = np.exp(g)                                    # per key channel
    S = alpha[..., :, None] * S                          # Diag(alpha_t) S_{t-1}
    predicted = np.einsum("...kv,...k->...v", S, k)      # what S predicts for k_t
    correction = beta[..., None] * (v - predicted)       # beta_t (v_t - prediction)
    S = S + k[..., :, None] * correction[..., None, :]   # rank-one write along k_t
    o = scale * np.einsum("...kv,...k->...v", S, q)      # o_t = S_t^T q_t
    return o, S


def kda_recurrent(q, k, v, g, beta, s0=None, scale=1.0):
    """Token-by-token forward over a whole sequence.

    Returns (o [B,T,H,dv], s_final [B,H,dk,dv]) in float64.  ``s0`` None means
    a zero initial state.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        o[:, t], S = kda_decode_step(q[:, t], k[:, t], v[:, t], g[:, t],
                                     beta[:, t], S, scale)
    return o, S


def gate_rmsnorm(x, gate, weight=None, eps=1e-6):
    """Head-wise RMSNorm followed by a sigmoid output gate.

    "Kimi K3 Architecture Explained ...", section "Token mixing": the output
    gate is applied after a head-wise RMSNorm.  The norm runs over the last
    axis (one head's dv vector):  y = x / sqrt(mean(x^2) + eps) * w * sigmoid(gate).
    ``weight`` None means a unit weight.
    """
    x, gate = _f64(x), _f64(gate)
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / rms
    if weight is not None:
        y = y * _f64(weight)
    return y / (1.0 + np.exp(-gate))


def kda_chunked(q, k, v, g, beta, s0=None, scale=1.0, chunk=16):
    """Chunkwise ("piecewise parallel") form of the same recurrence, float64.

    "Kimi K3 from Moonshot AI ...", section "Kimi Delta Attention (KDA)",
    says KDA can be rewritten chunkwise; "Kimi K3: Engineering ...", section
    "Dimension 1", fixes 16-token tiles with dense products on every causal
    tile.  The pages print no chunked equations; this is the plainest exact
    rewrite (the WY/UT form of the delta rule with a per-channel decay).
    Within a chunk, with start state S0 and Gamma_r = sum_{s<=r} g_s:

      delta_r = beta_r (v_r - S_{r-1}^T (alpha_r * k_r))          (write term)
      S_r     = Diag(e^{Gamma_r}) S0 + sum_{s<=r} Diag(e^{Gamma_r-Gamma_s}) k_s delta_s^T
      (I + A) Delta = Diag(beta) (V - Khat S0),
          A[r,s] = beta_r * sum_c khat[r,c] kchk[s,c]  for s < r, else 0,
          khat = k * e^{Gamma},  kchk = k * e^{-Gamma}
      O   = Qhat S0 + tril(Qhat Kchk^T) Delta,  qhat = q * e^{Gamma}
      S_n = Diag(e^{Gamma_n}) S0 + (k * e^{Gamma_n - Gamma})^T Delta

    The triangular system is solved with numpy.linalg.solve (a library step).
    It exists to pin the algebra a chunked kernel relies on: it must agree with
    ``kda_recurrent`` to float64 rounding for every chunk size.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S_all = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            S = S_all[b, h]
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                n = c1 - c0
                Q, K, V = q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h]
                G, bt = g[b, c0:c1, h], beta[b, c0:c1, h]
                Gam = np.cumsum(G, axis=0)                     # [n, dk]
                Khat = K * np.exp(Gam)
                Kchk = K * np.exp(-Gam)
                Qhat = Q * np.exp(Gam)
                Kbar = K * np.exp(Gam[-1][None, :] - Gam)
                A = np.tril(bt[:, None] * (Khat @ Kchk.T), k=-1)
                rhs = bt[:, None] * (V - Khat @ S)
                Delta = np.linalg.solve(np.eye(n) + A, rhs)
                Aqk = np.tril(Qhat @ Kchk.T)
                o[b, c0:c1, h] = scale * (Qhat @ S + Aqk @ Delta)
                S = np.exp(Gam[-1])[:, None] * S + Kbar.T @ Delta
            S_all[b, h] = S
    return o, S_all


def decay_gates(a, b):
    """Log-decay and write strength from their logits.

    "Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
    "Dimension 1", and "Kimi K3 Architecture Explained ...", section "Token
    mixing": the log-decay is bounded below by -5 through a scaled sigmoid,
    g = -5 * sigmoid(a), so every retention factor exp(g) lies in (e^-5, 1).
    The write strength is read as beta = sigmoid(b) (the workloads draw beta
    that way).  a: [..., dk] logits per key channel; b: [...] one per token and
    head.  Returns (g, beta) in float64.
    """
    a, b = _f64(a), _f64(b)
    return -5.0 / (1.0 + np.exp(-a)), 1.0 / (1.0 + np.exp(-b))


def l2_normalize(x, eps=1e-12):
    """x / max(||x||, eps) over the last axis (one head's dk vector).

    The method's keys (and queries) are unit vectors per head: the erase
    replaces what the state predicts for a unit key ("Kimi K3 Architecture
    Explained ...", section "Token mixing"), and the workloads normalise q and
    k this way.  eps only keeps a zero vector at zero.
    """
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)
