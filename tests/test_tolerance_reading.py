"""Why io-dtype outputs are compared with their final rounding allowed.

The parity bound is max|x - ref| <= 2e-2 * RMS(ref) for bfloat16 inputs with
float32 accumulation.  On the workloads' own distributions the layer output has
max|o| / RMS(o) of 12-15, so even the exact float64 answer, merely rounded to
bfloat16 (half an ulp, 2^-9 relative), already misses that bound.  The bound
can therefore only be meant for the computation: the tests subtract the
half-ulp of the stored value's final rounding and apply 2e-2 to what remains.
This test shows both facts on the oracle alone.
"""
import numpy as np
import torch

from oracle.kda_oracle import kda_recurrent
from tests.gpu_helpers import rel_max_err


def test_exact_answer_rounded_to_bf16_needs_the_allowance():
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 1, 1024, 8, 128, 128
    q = rng.standard_normal((B, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 / (1.0 + np.exp(-2.0 * rng.standard_normal((B, T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.02 * rng.standard_normal((B, H, dk, dv))
    o, _ = kda_recurrent(q, k, v, g, beta, s0)
    o_bf16 = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    assert np.abs(o).max() / np.sqrt(np.mean(o ** 2)) > 10.0
    assert rel_max_err(o_bf16, o) > 2e-2                       # raw bound fails
    assert rel_max_err(o_bf16, o, torch.bfloat16) < 1e-6       # only rounding is present
    perturbed = o_bf16 + 1e-2 * np.sqrt(np.mean(o ** 2))       # a real error still counts
    assert rel_max_err(perturbed, o, torch.bfloat16) > 9e-3


def test_host_normalised_keys_are_a_different_problem():
    """Why the prologue entry points are not compared with the plain ones fed
    host-normalised inputs.  Normalising raw q and k on the host and rounding
    the unit vectors to bfloat16 changes the problem: on the oracle alone, in
    float64, the final state of the two problems differs by 2-4e-2 RMS over
    these seeds (96 tokens, 4 heads, raw k of norm ~ 23), almost all of it from
    the rounding of the normalised keys; so each entry point is checked
    against the oracle run on its own inputs instead."""
    from oracle.kda_oracle import decay_gates, l2_normalize
    errs = []
    for seed in range(3):
        gen = torch.Generator().manual_seed(2180 + seed)
        r = lambda *s: torch.randn(*s, generator=gen)  # noqa: E731
        B, T, H = 1, 96, 4
        q = (0.3 * r(B, T, H, 128)).bfloat16()
        k = (2.0 * r(B, T, H, 128)).bfloat16()
        v = r(B, T, H, 128).bfloat16()
        a, b, s0 = r(B, T, H, 128).bfloat16(), r(B, T, H), 0.05 * r(B, H, 128, 128)
        f = lambda t: t.double().numpy()  # noqa: E731
        g, beta = decay_gates(f(a), f(b))
        _, S_raw = kda_recurrent(l2_normalize(f(q)), l2_normalize(f(k)), f(v), g, beta, f(s0))
        kn = torch.nn.functional.normalize(k.float(), dim=-1).bfloat16()
        _, S_host = kda_recurrent(l2_normalize(f(q)), f(kn), f(v), g, beta, f(s0))
        errs.append(rel_max_err(S_host, S_raw))
    assert max(errs) > 2e-2 and min(errs) > 1e-2
