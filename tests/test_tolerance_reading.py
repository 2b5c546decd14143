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
