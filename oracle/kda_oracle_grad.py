"""CPU oracle for the gradients of the KDA token recurrence.

TEST INFRASTRUCTURE ONLY, like ``kda_oracle``: nothing in the product package
may import it.  It defines the backward of the layer core as the plain
derivative of the forward recurrence, computed by reverse-mode automatic
differentiation (torch.autograd, float64, CPU) through a token-by-token loop.
No blocking, no chunking, no reordering.

The forward is the recurrence of "Kimi K3 Architecture Explained: KDA,
Attention Residuals and LatentMoE", section "Token mixing: what KDA is and why
3:1" (decay per key channel, then the Householder erase and write), with the
readings of ``kda_oracle``:

    S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t

The pages print no backward pass; training needs the gradients of a scalar
loss L with respect to q, k, v, g, beta and the initial state, given dL/do_t
for every token and dL/dS_T for the final state.  Those gradients are what
this module returns.

Pins (``tests/test_oracle_pins.py``): central differences of the float64
NumPy forward ``kda_oracle.kda_recurrent`` (an implementation that shares no
code with this one), and the closed form of a single token from a zero state.
"""
from __future__ import annotations

import numpy as np

__all__ = ["kda_recurrent_vjp"]


def kda_recurrent_vjp(q, k, v, g, beta, s0, do, ds_final=None, scale=1.0):
    """Gradients of L = sum(o * do) + sum(S_T * ds_final).

    Shapes as ``kda_oracle.kda_recurrent``: q, k, g [B,T,H,dk], v and do
    [B,T,H,dv], beta [B,T,H], s0 and ds_final [B,H,dk,dv] (s0 None: zero
    initial state, ds_final None: no final-state term).  Returns a dict of
    float64 arrays dq, dk, dv, dg, dbeta, ds0 with the shapes of the inputs.
    """
    import torch

    def leaf(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)

    q, k, v, g, beta = map(leaf, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = leaf(np.zeros((B, H, dk, dv)) if s0 is None else s0)
    do_t = torch.tensor(np.asarray(do, dtype=np.float64))

    S = S0
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        a = torch.exp(g[:, t])                            # [B,H,dk] retention per key channel
        Sd = a[..., None] * S                             # decay first
        kt, bt = k[:, t], beta[:, t]
        p = (Sd * kt[..., None]).sum(dim=-2)              # what the decayed state predicts for k
        u = bt[..., None] * (v[:, t] - p)                 # error-correcting write
        S = Sd + kt[..., None] * u[..., None, :]
        o = scale * (S * q[:, t][..., None]).sum(dim=-2)  # o_t = scale S_t^T q_t
        loss = loss + (o * do_t[:, t]).sum()
    if ds_final is not None:
        loss = loss + (S * torch.tensor(np.asarray(ds_final, dtype=np.float64))).sum()

    grads = torch.autograd.grad(loss, [q, k, v, g, beta, S0], allow_unused=True)
    names = ["dq", "dk", "dv", "dg", "dbeta", "ds0"]
    like = [q, k, v, g, beta, S0]
    return {n: (np.zeros(tuple(x.shape)) if d is None else d.numpy())
            for n, d, x in zip(names, grads, like)}
