"""Seeded input generators: determinism, shapes and the stated distributions."""
import os

import torch

from gated_delta_rule_112_amd.inputs import (WORKLOADS, Workload, make_decode_state,
                                             make_decode_step_inputs, make_prefill_inputs)


def test_prefill_inputs_deterministic_and_shaped():
    w = Workload("t", B=2, H=3, T=37, dk=16, dv=32, io="bf16", g_std=2.0, s0_std=0.02, gate=True,
                 seed=5)
    a = make_prefill_inputs(w)
    b = make_prefill_inputs(w)
    for key in ["q", "k", "v", "g", "beta", "s0", "gate"]:
        assert torch.equal(a[key], b[key]), key
    assert a["q"].shape == (2, 37, 3, 16) and a["q"].dtype == torch.bfloat16
    assert a["v"].shape == (2, 37, 3, 32)
    assert a["g"].dtype == torch.float32 and a["beta"].shape == (2, 37, 3)
    assert a["s0"].shape == (2, 3, 16, 32)
    assert float(a["g"].max()) < 0 and float(a["g"].min()) > -5.0
    assert float(a["beta"].min()) > 0 and float(a["beta"].max()) < 1
    norms = a["k"].float().norm(dim=-1)
    assert torch.allclose(norms, torch.ones_like(norms), atol=1e-2)
    c = make_prefill_inputs(w, seed=6)
    assert not torch.equal(a["q"], c["q"])


def test_forced_decay_channels():
    w = WORKLOADS["million_token_prefill"]
    small = Workload("m", B=1, H=w.H, T=4, dk=w.dk, dv=w.dv, io="bf16",
                     force_every=w.force_every, forced_g=w.forced_g, seed=w.seed)
    x = make_prefill_inputs(small)
    g = x["g"].view(-1, w.H * w.dk)
    forced = (g == torch.tensor(w.forced_g)).all(dim=0)
    idx = torch.nonzero(forced).flatten().tolist()
    assert idx == [j for j in range(w.H * w.dk) if j % 1000 == 0]
    assert len(idx) == 13


def test_decode_inputs():
    w = Workload("d", B=4, H=2, T=1, dk=32, dv=16, io="bf16", s0_std=0.02, steps=3, seed=9)
    s = make_decode_state(w)
    assert s.shape == (4, 2, 32, 16) and abs(float(s.std()) - 0.02) < 0.01
    x0 = make_decode_step_inputs(w, 0)
    x1 = make_decode_step_inputs(w, 1)
    assert x0["q"].shape == (4, 2, 32) and x0["beta"].shape == (4, 2)
    assert not torch.equal(x0["k"], x1["k"])
    assert torch.equal(x0["k"], make_decode_step_inputs(w, 0)["k"])


def test_bench_byte_accounting():
    """The benchmark's algorithmic bytes, against the per-element sizes written
    out: prefill 1,796 B per token-head with the gate at bf16 and 128/128 (q, k,
    v, o, gate 2 B each; g 4 B per channel; beta 4 B), decode 132,612 B per
    (b, h) and step, and the multi-token verify / commit split."""
    import bench
    total, per = bench.prefill_bytes(1, 32768, 96, 128, 128, 2, with_o=True, with_gate=True)
    assert per == 2 * 128 * 2 + 128 * 2 + 128 * 4 + 4 + 128 * 2 + 128 * 2 == 1796
    assert total == 32768 * 96 * 1796 + 96 * 128 * 128 * 4        # plus the final state
    _, per_d = bench.decode_bytes(256, 96, 128, 128, 2)
    assert per_d == 8 * 128 * 128 + 3 * 128 * 2 + 4 * 128 + 4 + 128 * 2 == 132612
    v, c = bench.verify_bytes(2, 3, 4, 128, 128, 2, [0, 3])
    tok_in = 3 * 128 * 2 + 4 * 128 + 4
    assert v == 2 * 3 * (4 * 128 * 128 + 4 * (tok_in + 2 * 128 * 2))
    assert c == 4 + (3 * (8 * 128 * 128 + 3 * tok_in) + 4)          # nothing read for 0 accepted
    assert bench.prefill_flops(1, 1, 1, 128, 128) == 6 * 16 * 128 + 4 * 16 * 128 + 6 * 128 * 128


def test_bench_refuses_several_gpus():
    """The benchmark measures one GPU: --gpus above 1 exits with status 2 and a
    message, before any GPU work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
