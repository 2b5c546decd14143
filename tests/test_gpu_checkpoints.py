"""GPU parity of the state checkpoints (kda_chunk_fwd_checkpoints), through the C ABI.

Checkpoint i of (b, h) must be the state after the first (i + 1) * every tokens:
the oracle computes it by running the float64 token recurrence piece by piece,
each piece starting from the state the previous one ended in.  Tolerance per
checkpoint tensor: 1e-4 x RMS for float32 io (vector path), 2e-2 x RMS for
bfloat16 io (matrix-core path); the outputs and final state must match the
plain kda_chunk_fwd call bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle.kda_oracle import kda_recurrent as o_recurrent
from tests.gpu_helpers import assert_close, dev, f64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_112_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def gen(B, T, H, dk, dv, dtype, seed, s0_std=0.05, gate=False):
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    q = r(B, T, H, dk)
    k = r(B, T, H, dk)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = r(B, T, H, dv).to(dtype)
    g = -5.0 * torch.sigmoid(r(B, T, H, dk))
    beta = torch.sigmoid(r(B, T, H))
    s0 = s0_std * r(B, H, dk, dv)
    gt = r(B, T, H, dv).to(dtype) if gate else None
    return q, k, v, g, beta, s0, gt


def oracle_checkpoints(q, k, v, g, beta, s0, every, run=o_recurrent):
    """[B, T // every, H, dk, dv]: the state after each whole interval."""
    x = [f64(t) for t in (q, k, v, g, beta)]
    S = s0 if isinstance(s0, np.ndarray) else f64(s0)
    T = x[0].shape[1]
    out = []
    for i in range(T // every):
        _, S = run(*(t[:, i * every:(i + 1) * every] for t in x), S)
        out.append(S)
    return np.stack(out, axis=1)


CASES = [  # (dk, dv, dtype, T, every)
    (128, 128, torch.bfloat16, 100, 32),
    (128, 128, torch.bfloat16, 160, 64),
    (128, 128, torch.bfloat16, 64, 64),
    (64, 32, torch.float32, 100, 32),
    (128, 128, torch.float32, 96, 32),
]


@pytest.mark.parametrize("dk,dv,dtype,T,every", CASES)
@pytest.mark.parametrize("gated", [False, True])
def test_checkpoints_match_oracle(kda, dk, dv, dtype, T, every, gated):
    q, k, v, g, beta, s0, gate = gen(2, T, 3, dk, dv, dtype, 900 + T + every + dk, gate=gated)
    y, S, ck = kda.chunk_fwd_checkpoints(q, k, v, g, beta, s0, every=every, gate=gate)
    y2, S2 = kda.chunk_fwd(q, k, v, g, beta, s0, gate=gate)
    ref = oracle_checkpoints(q, k, v, g, beta, s0, every)
    torch.cuda.synchronize()
    assert tuple(ck.shape) == (2, T // every, 3, dk, dv)
    for i in range(T // every):
        assert_close(f64(ck[:, i]), ref[:, i], TOL[dtype], f"checkpoint {i}")
    assert torch.equal(y, y2) and torch.equal(S, S2), "checkpoints must not change the results"


@pytest.mark.parametrize("split", ["1", "2"])
@pytest.mark.parametrize("seg", ["1", "3", "0"])
def test_checkpoints_segments(kda, monkeypatch, split, seg):
    """Matrix-core path: checkpoints that fall on segment boundaries, inside
    segments, with one or two state workgroups per head."""
    monkeypatch.setenv("KDA_CHUNK_SPLIT", split)
    if seg != "0":
        monkeypatch.setenv("KDA_SEG_PAIRS", seg)
    q, k, v, g, beta, s0, _ = gen(2, 230, 2, 128, 128, torch.bfloat16, 950 + int(seg))
    _, S, ck = kda.chunk_fwd_checkpoints(q, k, v, g, beta, s0, every=64)
    _, S_ref = o_recurrent(*(f64(t) for t in (q, k, v, g, beta)), f64(s0))
    ref = oracle_checkpoints(q, k, v, g, beta, s0, 64)
    torch.cuda.synchronize()
    assert_close(f64(ck), ref, TOL[torch.bfloat16], "checkpoints")
    assert_close(f64(S), S_ref, TOL[torch.bfloat16], "final state")


def test_checkpoints_short_sequence(kda):
    """T shorter than the interval: no checkpoint, same results."""
    q, k, v, g, beta, s0, _ = gen(1, 40, 2, 128, 128, torch.bfloat16, 970)
    y, S, ck = kda.chunk_fwd_checkpoints(q, k, v, g, beta, s0, every=64)
    y2, S2 = kda.chunk_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    assert ck.shape[1] == 0
    assert torch.equal(y, y2) and torch.equal(S, S2)


def test_checkpoints_full_width_sampled(kda):
    """B=1, H=96, T=32768 with the gated epilogue (the benchmark's workload and
    launch) and a checkpoint every 2048 tokens: all 16 checkpoints of 3 sampled
    heads against the oracle's token-by-token recurrence."""
    from gated_delta_rule_112_amd.inputs import WORKLOADS, make_prefill_inputs
    w = WORKLOADS["full_width_prefill"]
    x = make_prefill_inputs(w, device=dev())
    _, S, ck = kda.chunk_fwd_checkpoints(x["q"], x["k"], x["v"], x["g"], x["beta"], None,
                                         every=2048, gate=x["gate"])
    torch.cuda.synchronize()
    for h in [0, 47, 95]:
        sl = [x[key][:, :, h:h + 1] for key in ["q", "k", "v", "g", "beta"]]
        ref = oracle_checkpoints(*sl, np.zeros((1, 1, 128, 128)), 2048)
        assert_close(f64(ck[:, :, h:h + 1]), ref, TOL[torch.bfloat16], f"checkpoints head {h}")
        assert_close(f64(ck[0, -1, h]), f64(S[0, h]), 1e-6, f"last checkpoint == state, {h}")
