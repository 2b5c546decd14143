"""GPU parity of the backward pass (kda_recurrent_bwd), through the C ABI.

Every gradient (dq, dk, dv, dg, dbeta, ds0) against the float64 gradient
oracle (kda_oracle_grad.kda_recurrent_vjp, pinned by central differences of
the forward oracle) on the same inputs.  Tolerance per tensor: 1e-4 x RMS for
float32 io; for bfloat16 io 2e-2 x RMS on dq, dk, dv (half an ulp of their
bfloat16 rounding not counted) and 2e-3 x RMS on the float32 dg, dbeta, ds0.
Lengths span several 64-token pieces with a ragged last piece.
"""
import pytest
import torch

from oracle.kda_oracle_grad import kda_recurrent_vjp
from tests.gpu_helpers import assert_close, dev, f64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_112_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def gen(B, T, H, dtype, seed, with_s0, with_dsf):
    gen_ = torch.Generator(device=dev())
    gen_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen_, device=dev())  # noqa: E731
    D = 128
    q = r(B, T, H, D)
    k = r(B, T, H, D)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = r(B, T, H, D).to(dtype)
    g = -5.0 * torch.sigmoid(r(B, T, H, D))
    beta = torch.sigmoid(r(B, T, H))
    do = r(B, T, H, D).to(dtype)
    s0 = 0.05 * r(B, H, D, D) if with_s0 else None
    dsf = r(B, H, D, D) if with_dsf else None
    return q, k, v, g, beta, do, s0, dsf


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,H,with_s0,with_dsf", [(2, 70, 2, True, True), (1, 130, 3, False, True),
                                                    (1, 64, 1, True, False), (2, 5, 1, False, False)])
def test_backward_matches_oracle(kda, dtype, B, T, H, with_s0, with_dsf):
    q, k, v, g, beta, do, s0, dsf = gen(B, T, H, dtype, 4000 + T + B, with_s0, with_dsf)
    print(f"backward case B={B} T={T} H={H} {dtype}", flush=True)
    got = kda.recurrent_bwd(q, k, v, g, beta, do, s0, dsf, scale=0.7)
    torch.cuda.synchronize()
    ref = kda_recurrent_vjp(f64(q), f64(k), f64(v), f64(g), f64(beta),
                            None if s0 is None else f64(s0), f64(do),
                            None if dsf is None else f64(dsf), 0.7)
    for name, x in zip(["dq", "dk", "dv", "dg", "dbeta", "ds0"], got):
        io_out = name in ("dq", "dk", "dv")   # stored in the io dtype: its rounding not counted
        tol = TOL[dtype] if io_out else TOL[dtype] / (10 if dtype == torch.bfloat16 else 1)
        assert_close(f64(x), ref[name], tol, f"{name} B={B} T={T}", dtype if io_out else None)
