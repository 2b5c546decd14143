"""HIP graph capture of the hot path, through the C ABI.

A prefill, decode or verify call enqueues only kernel launches on the
caller's stream (no memset, allocation or synchronisation), so it can be
captured once (torch.cuda.CUDAGraph) and replayed with new input contents.
Every replay, with eager work and synchronisations between replays, must give
what the eager call gives on the same inputs, bit for bit: the kernels have no
atomics and a fixed reduction order.
"""
import pytest
import torch

from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_112_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def fill(tensors, seed):
    """New contents for the captured input tensors (unit q, k; g < 0; beta in (0, 1))."""
    gen = torch.Generator(device=dev())
    gen.manual_seed(seed)
    for name, t in tensors.items():
        x = torch.randn(t.shape, generator=gen, device=dev())
        if name in ("q", "k"):
            x = x / x.norm(dim=-1, keepdim=True)
        elif name == "g":
            x = -5.0 * torch.sigmoid(x)
        elif name == "beta":
            x = torch.sigmoid(x)
        elif name == "state":
            x = 0.3 * x
        t.copy_(x.to(t.dtype))


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("B,T,H,gated", [(2, 200, 4, True), (1, 1000, 2, False)])
def test_prefill_graph_replays(kda, monkeypatch, B, T, H, gated):
    """Matrix-core prefill (several launches per call: segments of 3 pairs)."""
    dk = dv = 128
    bf = torch.bfloat16
    x = {"q": torch.empty(B, T, H, dk, dtype=bf, device=dev()),
         "k": torch.empty(B, T, H, dk, dtype=bf, device=dev()),
         "v": torch.empty(B, T, H, dv, dtype=bf, device=dev()),
         "g": torch.empty(B, T, H, dk, device=dev()),
         "beta": torch.empty(B, T, H, device=dev()),
         "s0": torch.empty(B, H, dk, dv, device=dev())}
    if gated:
        x["gate"] = torch.empty(B, T, H, dv, dtype=bf, device=dev())
    out = torch.empty(B, T, H, dv, dtype=bf, device=dev())
    s_out = torch.empty(B, H, dk, dv, device=dev())
    nws = kda.chunk_workspace_size(B, T, H, dk, dv, bf)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev())
    fill(x, 3000)

    def run(o, s, w):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gate=x.get("gate"),
                      out=o, s_out=s, workspace=w)

    monkeypatch.setenv("KDA_SEG_PAIRS", "3")
    graph = capture(lambda: run(out, s_out, ws))
    ws_e = torch.empty_like(ws)
    for i in range(REPLAYS):
        fill(x, 3001 + i)
        y_e, S_e = torch.empty_like(out), torch.empty_like(s_out)
        run(y_e, S_e, ws_e)                      # eager, on the same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_e), f"replay {i}: outputs differ from the eager call"
        assert torch.equal(s_out, S_e), f"replay {i}: final state differs"


def test_decode_graph_replays(kda):
    """Decode step and a 4-token verify call, captured together; the state
    is updated in place by the captured decode step."""
    B, H, dk, dv, K = 8, 4, 128, 128, 4
    bf = torch.bfloat16
    x = {"q": torch.empty(B, H, dk, dtype=bf, device=dev()),
         "k": torch.empty(B, H, dk, dtype=bf, device=dev()),
         "v": torch.empty(B, H, dv, dtype=bf, device=dev()),
         "g": torch.empty(B, H, dk, device=dev()),
         "beta": torch.empty(B, H, device=dev()),
         "gate": torch.empty(B, H, dv, dtype=bf, device=dev())}
    m = {"q": torch.empty(B, K, H, dk, dtype=bf, device=dev()),
         "k": torch.empty(B, K, H, dk, dtype=bf, device=dev()),
         "v": torch.empty(B, K, H, dv, dtype=bf, device=dev()),
         "g": torch.empty(B, K, H, dk, device=dev()),
         "beta": torch.empty(B, K, H, device=dev()),
         "gate": torch.empty(B, K, H, dv, dtype=bf, device=dev())}
    st = {"state": torch.empty(B, H, dk, dv, device=dev())}
    zero = torch.zeros(B, dtype=torch.int32, device=dev())
    o1 = torch.empty(B, H, dv, dtype=bf, device=dev())
    ov = torch.empty(B, K, H, dv, dtype=bf, device=dev())
    fill(x, 3100)
    fill(m, 3101)
    fill(st, 3102)

    def run(state, a, b):
        kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, gate=x["gate"], out=a)
        kda.decode_multi(m["q"], m["k"], m["v"], m["g"], m["beta"], state, zero,
                         gate=m["gate"], out=b)

    graph = capture(lambda: run(st["state"], o1, ov))
    for i in range(REPLAYS):
        fill(x, 3110 + i)
        fill(m, 3120 + i)
        fill(st, 3130 + i)
        S_e = st["state"].clone()
        a_e, b_e = torch.empty_like(o1), torch.empty_like(ov)
        run(S_e, a_e, b_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, a_e), f"replay {i}: decode output differs"
        assert torch.equal(ov, b_e), f"replay {i}: verify output differs"
        assert torch.equal(st["state"], S_e), f"replay {i}: state differs"


def test_backward_graph_replays(kda):
    """The chunkwise backward captured whole (five launches); every replay
    equals the eager call bit for bit."""
    B, T, H, D = 1, 200, 2, 128
    bf = torch.bfloat16
    x = {"q": torch.empty(B, T, H, D, dtype=bf, device=dev()),
         "k": torch.empty(B, T, H, D, dtype=bf, device=dev()),
         "v": torch.empty(B, T, H, D, dtype=bf, device=dev()),
         "dout": torch.empty(B, T, H, D, dtype=bf, device=dev()),
         "g": torch.empty(B, T, H, D, device=dev()),
         "beta": torch.empty(B, T, H, device=dev()),
         "state": torch.empty(B, H, D, D, device=dev()),
         "dsf": torch.empty(B, H, D, D, device=dev())}
    nws = kda.load_library().kda_recurrent_bwd_workspace_size(B, T, H, D, D)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev())
    ws_e = torch.empty(nws, dtype=torch.uint8, device=dev())
    fill(x, 3200)
    held = {}

    def run(w):
        return kda.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["dout"],
                                 x["state"], x["dsf"], scale=0.7, workspace=w)

    def captured():
        held["out"] = run(ws)

    graph = capture(captured)
    for i in range(REPLAYS):
        fill(x, 3210 + i)
        eager = run(ws_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(["dq", "dk", "dv", "dg", "dbeta", "ds0"], held["out"], eager):
            assert torch.equal(a, b), f"replay {i}: {name} differs"
