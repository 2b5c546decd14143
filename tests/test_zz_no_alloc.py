"""kda_chunk_fwd_noalloc (the prefill on the library's fixed device scratch,
for callers that cannot allocate), through the C ABI: two calls in a row, the
second with a smaller input, each against kda_chunk_fwd with its own
workspace at the bfloat16 bar (2e-2 RMS, half an ulp of the output's final
rounding not counted; float32 inputs at 1e-4), and a shape whose records
cannot fit the scratch, rejected on the host with KDA_ERR_WORKSPACE.
"""
import pytest
import torch

from tests.gpu_helpers import assert_close, dev, f64

pytestmark = pytest.mark.gpu

WORKSPACE = 9


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_112_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def gen(B, T, H, dtype, seed, gate=False):
    g_ = torch.Generator(device=dev())
    g_.manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g_, device=dev())  # noqa: E731
    q, k = r(B, T, H, 128), r(B, T, H, 128)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = r(B, T, H, 128).to(dtype)
    g = -5.0 * torch.sigmoid(r(B, T, H, 128))
    beta = torch.sigmoid(r(B, T, H))
    s0 = 0.02 * r(B, H, 128, 128)
    gt = r(B, T, H, 128).to(dtype) if gate else None
    return q, k, v, g, beta, s0, gt


def test_noalloc_two_calls_match_workspace_entry_point(kda):
    assert kda.load_library().kda_chunk_fwd_noalloc_scratch_bytes() == 64 << 20
    cases = [(1, 4096, 96, True, 5000),    # the full-width head count, gated: 128 pairs,
                                           # segments cut to fit the scratch
             (2, 300, 5, False, 5001)]     # then a smaller input on the same scratch
    for B, T, H, gated, seed in cases:
        q, k, v, g, beta, s0, gt = gen(B, T, H, torch.bfloat16, seed, gate=gated)
        y0, S0 = kda.chunk_fwd(q, k, v, g, beta, s0, gate=gt)
        y = torch.empty_like(y0)
        S = torch.empty_like(S0)
        kda.chunk_fwd_noalloc(q, k, v, g, beta, s0, gate=gt, out=y, s_out=S)
        torch.cuda.synchronize()
        assert_close(f64(y), f64(y0), 2e-2, f"y B={B} T={T} H={H}", torch.bfloat16)
        assert_close(f64(S), f64(S0), 2e-2, f"state B={B} T={T} H={H}")


def test_noalloc_vector_path(kda):
    q, k, v, g, beta, s0, _ = gen(1, 50, 3, torch.float32, 5002)
    o0, S0 = kda.chunk_fwd(q, k, v, g, beta, s0)
    o, S = kda.chunk_fwd_noalloc(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(S, S0)


def test_noalloc_rejects_what_cannot_fit(kda):
    """600 heads of one sequence: one pair of records per head and the carried
    state exceed the 64 MiB scratch; rejected before any launch."""
    lib = kda.load_library()
    import ctypes
    p = ctypes.c_void_p(1 << 40)  # never dereferenced: the call fails validation
    st = lib.kda_chunk_fwd_noalloc(p, ctypes.c_void_p((1 << 40) + (1 << 34)),
                                   ctypes.c_void_p((1 << 40) + (2 << 34)),
                                   ctypes.c_void_p((1 << 40) + (3 << 34)),
                                   ctypes.c_void_p((1 << 40) + (4 << 34)), None,
                                   ctypes.c_void_p((1 << 40) + (5 << 34)), None, None, None,
                                   1e-6, 1, 64, 600, 128, 128, 1.0, 1, None)
    assert st == WORKSPACE
