"""Magnitude range of the matrix-core prefill (bfloat16 io, dk = dv = 128).

The state, the values and the delta enter that path's products as float16.
For fixed q, k, g and beta the method is linear in (v, s0) (pin P12: the
recurrence S_t = (I - beta k k^T) Diag(e^g) S_{t-1} + beta k v^T is linear in
(S_0, v), and o_t = S_t^T q_t), so scaling v and s0 by 2^p must scale o and
the final state by 2^p.  These tests run every power of two from 2^-24 to
2^24 (bfloat16 values from about 1e-7 to 1e8, float32 states alike) through
both workgroup layouts, the gated epilogue and the entry point that
normalises raw projections, and compare each case element by element with
the float64 oracle on the same inputs at the bfloat16 bar (2e-2 RMS, half an
ulp of the output's final rounding not counted).  The prologue entry point
also takes raw q and k whose norms span 2^-4 .. 2^7, the range its header
states.  Head permutation (the other half of P12) must permute the results
bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle.kda_oracle import decay_gates, l2_normalize
from oracle.kda_oracle import gate_rmsnorm as o_gate_rmsnorm
from oracle.kda_oracle import kda_recurrent as o_recurrent
from tests.gpu_helpers import assert_close, dev, f64

pytestmark = pytest.mark.gpu

TOL = 2e-2
BF = torch.bfloat16
POWERS = [-24, -16, -12, -8, -4, 4, 8, 12, 16, 24]


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_112_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def gen(B, T, H, seed, gate=False):
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    q = r(B, T, H, 128)
    k = r(B, T, H, 128)
    q = (q / q.norm(dim=-1, keepdim=True)).to(BF)
    k = (k / k.norm(dim=-1, keepdim=True)).to(BF)
    v = r(B, T, H, 128)  # float32; scaled, then rounded to bfloat16
    g = -5.0 * torch.sigmoid(r(B, T, H, 128))
    beta = torch.sigmoid(r(B, T, H))
    s0 = 0.1 * r(B, H, 128, 128)
    gt = r(B, T, H, 128).to(BF) if gate else None
    return q, k, v, g, beta, s0, gt


def oracle(q, k, v, g, beta, s0, gate=None):
    o, S = o_recurrent(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(s0))
    if gate is not None:
        o = o_gate_rmsnorm(o, f64(gate), None, 1e-6)
    return o, S


@pytest.mark.parametrize("split", ["1", "2"])
@pytest.mark.parametrize("p", POWERS)
def test_values_and_state_scaled(kda, monkeypatch, split, p):
    """v and s0 times 2^p: every output and the final state against the oracle,
    and against 2^p times the unscaled call."""
    monkeypatch.setenv("KDA_CHUNK_SPLIT", split)
    q, k, v, g, beta, s0, _ = gen(1, 100, 3, 3000 + p)
    f = 2.0 ** p
    vs, s0s = (v * f).to(BF), s0 * f
    o, S = kda.chunk_fwd(q, k, vs, g, beta, s0s)
    o1, S1 = kda.chunk_fwd(q, k, v.to(BF), g, beta, s0)
    o_ref, S_ref = oracle(q, k, vs, g, beta, s0s)
    torch.cuda.synchronize()
    assert_close(f64(o), o_ref, TOL, f"o, 2^{p}", BF)
    assert_close(f64(S), S_ref, TOL, f"state, 2^{p}")
    # linearity of the kernel itself: the scaled call against 2^p times the
    # plain one (both rounded to bfloat16 at the output)
    assert_close(f64(o), f64(o1) * f, TOL, f"o linear, 2^{p}", BF)
    assert_close(f64(S), f64(S1) * f, TOL, f"state linear, 2^{p}")


@pytest.mark.parametrize("p", [-24, -12, 12, 24])
def test_scaled_gated_and_segments(kda, monkeypatch, p):
    """The gated epilogue (one workgroup per head) over segments of one pair,
    v and s0 times 2^p, growing magnitudes along the sequence included."""
    monkeypatch.setenv("KDA_SEG_PAIRS", "1")
    q, k, v, g, beta, s0, gt = gen(2, 130, 2, 3100 + p, gate=True)
    f = 2.0 ** p
    ramp = torch.logspace(-3, 3, 130, base=2.0, device=dev()).view(1, 130, 1, 1)
    vs, s0s = (v * f * ramp).to(BF), s0 * f
    y, S = kda.chunk_fwd(q, k, vs, g, beta, s0s, gate=gt)
    y_ref, S_ref = oracle(q, k, vs, g, beta, s0s, gt)
    torch.cuda.synchronize()
    assert_close(f64(y), y_ref, TOL, f"y, 2^{p}", BF)
    assert_close(f64(S), S_ref, TOL, f"state, 2^{p}")


@pytest.mark.parametrize("p", [-24, -8, 8, 24])
@pytest.mark.parametrize("qk_norm", [2.0 ** -4, 1.0, 2.0 ** 7])
def test_prologue_scaled(kda, p, qk_norm):
    """Raw projections: q and k with norms near qk_norm (normalised in the
    kernels), logits a and b, v and s0 times 2^p."""
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(3200 + p)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    B, T, H = 1, 100, 2
    q = (qk_norm / 128 ** 0.5 * r(B, T, H, 128)).to(BF)
    k = (qk_norm / 128 ** 0.5 * r(B, T, H, 128)).to(BF)
    a = r(B, T, H, 128).to(BF)
    b = r(B, T, H)
    f = 2.0 ** p
    v = (f * r(B, T, H, 128)).to(BF)
    s0 = 0.1 * f * r(B, H, 128, 128)
    y, S = kda.chunk_fwd(q, k, v, a, b, s0, prologue=True)
    gg, bb = decay_gates(f64(a), f64(b))
    o_ref, S_ref = o_recurrent(l2_normalize(f64(q)), l2_normalize(f64(k)), f64(v), gg, bb,
                               f64(s0))
    torch.cuda.synchronize()
    assert_close(f64(y), o_ref, TOL, f"o, |q|,|k| ~ {qk_norm}, 2^{p}", BF)
    assert_close(f64(S), S_ref, TOL, f"state, |q|,|k| ~ {qk_norm}, 2^{p}")


@pytest.mark.parametrize("split", ["1", "2"])
def test_head_permutation(kda, monkeypatch, split):
    """Permuting the heads of every input permutes the outputs and the final
    states exactly."""
    monkeypatch.setenv("KDA_CHUNK_SPLIT", split)
    q, k, v, g, beta, s0, _ = gen(2, 77, 5, 3300)
    v = v.to(BF)
    perm = torch.tensor([3, 0, 4, 2, 1], device=dev())
    o, S = kda.chunk_fwd(q, k, v, g, beta, s0)
    ph = lambda x: x[:, :, perm].contiguous()  # noqa: E731
    op, Sp = kda.chunk_fwd(ph(q), ph(k), ph(v), ph(g), beta[:, :, perm].contiguous(),
                           s0[:, perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(op, o[:, :, perm]) and torch.equal(Sp, S[:, perm])


def test_decode_scaled(kda):
    """The decode step (float32 arithmetic) under the same scaling, 2^-24 and
    2^24, against the oracle's step."""
    from oracle.kda_oracle import kda_decode_step as o_decode
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(3400)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    B, H = 3, 4
    q = r(B, H, 128)
    k = r(B, H, 128)
    q = (q / q.norm(dim=-1, keepdim=True)).to(BF)
    k = (k / k.norm(dim=-1, keepdim=True)).to(BF)
    g = -5.0 * torch.sigmoid(r(B, H, 128))
    beta = torch.sigmoid(r(B, H))
    for p in (-24, 24):
        f = 2.0 ** p
        v = (f * r(B, H, 128)).to(BF)
        st = 0.1 * f * r(B, H, 128, 128)
        S0 = st.clone()
        o = kda.decode_step(q, k, v, g, beta, st)
        o_ref, S_ref = o_decode(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(S0))
        torch.cuda.synchronize()
        assert_close(f64(o), o_ref, TOL, f"decode o, 2^{p}", BF)
        assert_close(f64(st), S_ref, TOL, f"decode state, 2^{p}")


@pytest.mark.parametrize("dtype", [BF, torch.float32])
def test_prologue_zero_rows(kda, dtype):
    """Raw projections with all-zero key or query rows at some tokens (the
    normalisation maps them to zero: such a key writes nothing, such a query
    reads nothing), on the matrix-core (bfloat16) and vector (float32) paths."""
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(3500)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    B, T, H = 1, 90, 2
    q, k = r(B, T, H, 128), r(B, T, H, 128)
    k[:, 3] = 0.0
    k[:, 40:43, 1] = 0.0
    q[:, 7] = 0.0
    q, k = q.to(dtype), k.to(dtype)
    a, b = r(B, T, H, 128).to(dtype), r(B, T, H)
    v = r(B, T, H, 128).to(dtype)
    s0 = 0.1 * r(B, H, 128, 128)
    y, S = kda.chunk_fwd(q, k, v, a, b, s0, prologue=True)
    gg, bb = decay_gates(f64(a), f64(b))
    o_ref, S_ref = o_recurrent(l2_normalize(f64(q)), l2_normalize(f64(k)), f64(v), gg, bb,
                               f64(s0))
    torch.cuda.synchronize()
    tol = TOL if dtype == BF else 1e-4
    assert_close(f64(y), o_ref, tol, "o, zero rows", dtype)
    assert_close(f64(S), S_ref, tol, "state, zero rows")
