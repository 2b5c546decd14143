"""GPU parity of packed variable-length prefill (kda_chunk_fwd_varlen), through the C ABI.

Every sequence of the packed batch must equal the float64 token recurrence of
the oracle run on that sequence alone, from its own initial state: outputs,
final state and checkpoints.  Tolerances as for the uniform prefill: 1e-4 x RMS
for float32 io (vector path), 2e-2 x RMS for bfloat16 io (matrix-core path; half
an ulp of the bfloat16 output's rounding not counted).
"""
import numpy as np
import pytest
import torch

from oracle.kda_oracle import gate_rmsnorm as o_gate_rmsnorm
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


def gen(lens, H, dk, dv, dtype, seed, gate=False):
    total = int(sum(lens))
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    q = r(total, H, dk)
    k = r(total, H, dk)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = r(total, H, dv).to(dtype)
    g = -5.0 * torch.sigmoid(r(total, H, dk))
    beta = torch.sigmoid(r(total, H))
    s0 = 0.05 * r(len(lens), H, dk, dv)
    gt = r(total, H, dv).to(dtype) if gate else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev())
    return q, k, v, g, beta, s0, gt, cu


def check(kda, lens, H, dk, dv, dtype, seed, gate=False, every=0, heads=None):
    q, k, v, g, beta, s0, gt, cu = gen(lens, H, dk, dv, dtype, seed, gate)
    max_len = max(max(lens), 1)
    y, S, ck = kda.chunk_fwd_varlen(q, k, v, g, beta, cu, max_len, s0, gate=gt, every=every)
    torch.cuda.synchronize()
    cuh = cu.cpu().numpy()
    for b, n in enumerate(lens):
        a = int(cuh[b])
        if n == 0:
            assert torch.equal(S[b], s0[b]), "an empty sequence keeps its initial state"
            continue
        x = [f64(t[a:a + n])[None] for t in (q, k, v, g, beta)]
        o_ref, S_ref = o_recurrent(*x, f64(s0[b:b + 1]))
        if gt is not None:
            o_ref = o_gate_rmsnorm(o_ref, f64(gt[a:a + n])[None], None, 1e-6)
        assert_close(f64(y[a:a + n]), o_ref[0], TOL[dtype], f"y seq {b} (len {n})", dtype)
        assert_close(f64(S[b]), S_ref[0], TOL[dtype], f"state seq {b}")
        for i in range(n // every if every else 0):
            _, Si = o_recurrent(*(t[:, :(i + 1) * every] for t in x), f64(s0[b:b + 1]))
            assert_close(f64(ck[b, i]), Si[0], TOL[dtype], f"checkpoint {i} seq {b}")
    return y, S


LENS = [1, 37, 0, 100, 64, 33]


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (64, 32, torch.float32),
                                         (128, 128, torch.float32)])
@pytest.mark.parametrize("gated", [False, True])
def test_varlen_matches_oracle(kda, dk, dv, dtype, gated):
    check(kda, LENS, 3, dk, dv, dtype, 1700 + dk + dv, gate=gated, every=32)


@pytest.mark.parametrize("split", ["1", "2"])
@pytest.mark.parametrize("seg", ["1", "3"])
def test_varlen_segments(kda, monkeypatch, split, seg):
    """Matrix-core path with segments of one and three pairs, one or two state
    workgroups per head: sequences end inside, at, and before segments."""
    monkeypatch.setenv("KDA_CHUNK_SPLIT", split)
    monkeypatch.setenv("KDA_SEG_PAIRS", seg)
    check(kda, [130, 5, 64, 96, 31], 2, 128, 128, torch.bfloat16, 1750 + int(seg), every=64)


def test_varlen_equal_lengths_equal_uniform(kda):
    """Equal lengths: the packed call computes what the [B, T] call does, bit for bit."""
    B, T, H = 3, 80, 4
    q, k, v, g, beta, s0, gt, cu = gen([T] * B, H, 128, 128, torch.bfloat16, 1780, gate=True)
    y, S, _ = kda.chunk_fwd_varlen(q, k, v, g, beta, cu, T, s0, gate=gt)
    rs = lambda t: t.view(B, T, *t.shape[1:])  # noqa: E731
    y2, S2 = kda.chunk_fwd(rs(q), rs(k), rs(v), rs(g), rs(beta), s0, gate=rs(gt))
    torch.cuda.synchronize()
    assert torch.equal(rs(y), y2) and torch.equal(S, S2)


def test_varlen_serving_batch(kda):
    """64 sequences of 1 to 700 tokens, 8 heads, the gated epilogue: a serving
    batch on the matrix-core path, every sequence against the oracle."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 701, 64)]
    check(kda, lens, 8, 128, 128, torch.bfloat16, 1790, gate=True)


def check_prologue(kda, lens, H, dk, dv, dtype, seed, gated=False, every=0, output=True,
                   final_state=True):
    """kda_chunk_fwd_varlen_prologue: raw q and k (norms far from 1), decay and
    write-strength logits; per sequence the oracle normalises q and k
    (l2_normalize), forms g and beta (decay_gates) and runs the token
    recurrence from the sequence's own initial state; checkpoints too."""
    from oracle.kda_oracle import decay_gates, l2_normalize
    total = sum(lens)
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    q = (0.3 * r(total, H, dk)).to(dtype)
    k = (2.0 * r(total, H, dk)).to(dtype)
    v = r(total, H, dv).to(dtype)
    a = (2.0 * r(total, H, dk)).to(dtype)
    b = r(total, H)
    s0 = 0.05 * r(len(lens), H, dk, dv)
    gt = r(total, H, dv).to(dtype) if gated else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev())
    y, S, ck = kda.chunk_fwd_varlen(q, k, v, a, b, cu, max(lens), s0, gate=gt, every=every,
                                    output=output, final_state=final_state, prologue=True)
    torch.cuda.synchronize()
    g, beta = decay_gates(f64(a), f64(b))
    x_all = [l2_normalize(f64(q)), l2_normalize(f64(k)), f64(v), g, beta]
    for i, n in enumerate(lens):
        st = int(sum(lens[:i]))
        if n == 0:
            if final_state:
                assert torch.equal(S[i], s0[i]), "an empty sequence keeps its initial state"
            continue
        x = [t[st:st + n][None] for t in x_all]
        o_ref, S_ref = o_recurrent(*x, f64(s0[i:i + 1]))
        if gt is not None:
            o_ref = o_gate_rmsnorm(o_ref, f64(gt[st:st + n])[None], None, 1e-6)
        if output:
            assert_close(f64(y[st:st + n]), o_ref[0], TOL[dtype], f"y seq {i} (len {n})", dtype)
        if final_state:
            assert_close(f64(S[i]), S_ref[0], TOL[dtype], f"state seq {i}")
        for j in range(n // every if every else 0):
            _, Sj = o_recurrent(*(t[:, :(j + 1) * every] for t in x), f64(s0[i:i + 1]))
            assert_close(f64(ck[i, j]), Sj[0], TOL[dtype], f"checkpoint {j} seq {i}")


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (64, 32, torch.float32)])
@pytest.mark.parametrize("gated", [False, True])
def test_varlen_prologue_matches_oracle(kda, dk, dv, dtype, gated):
    check_prologue(kda, [1, 37, 0, 100, 64, 33], 3, dk, dv, dtype, 1800 + dk + dv + gated,
                   gated=gated, every=32)


@pytest.mark.parametrize("split", ["1", "2"])
@pytest.mark.parametrize("seg", ["1", "3"])
@pytest.mark.parametrize("what", ["output", "state"])
def test_varlen_prologue_segments(kda, monkeypatch, split, seg, what):
    """Matrix-core path from raw projections: segments of one and three pairs,
    one or two state workgroups per head, output-only and state-only calls."""
    monkeypatch.setenv("KDA_CHUNK_SPLIT", split)
    monkeypatch.setenv("KDA_SEG_PAIRS", seg)
    check_prologue(kda, [70, 0, 130, 5], 2, 128, 128, torch.bfloat16, 1850 + int(seg),
                   output=what == "output", final_state=what == "state")


@pytest.mark.parametrize("group", ["1", "2", "4"])
def test_varlen_launch_groups(kda, monkeypatch, group):
    """Sequences split into launch groups of 1, 2 or 4 (6 sequences: 6, 3 or 2
    groups, the last one short), records and carried state handed from group
    to group inside one pipeline; gated, with checkpoints."""
    monkeypatch.setenv("KDA_GROUP_SEQS", group)
    check(kda, LENS, 3, 128, 128, torch.bfloat16, 1900 + int(group), gate=True, every=32)
