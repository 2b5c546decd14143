"""Seeded synthetic inputs for the KDA workloads.

This module only draws random tensors with the shapes and distributions of the
workloads below; it holds none of the layer's arithmetic.  Both the HIP path
and the CPU oracle are fed from it (the oracle receives host copies of exactly
the tensors the device consumed, promoted to float64).

Distributions (N(mu, s) means mean mu and standard deviation s):
  q, k  ~ N(0, 1) per element, then L2-normalised over dk per (b, t, h),
        then cast to the io dtype (round to nearest even);
  v     ~ N(0, 1) in the io dtype;
  beta  = sigmoid(N(0, 1)) in float32, one per (b, t, h);
  g     = -5 * sigmoid(N(0, g_std)) in float32, one per (b, t, h, dk): the
        log-decay bounded below by -5 (pages: "Kimi K3: Engineering a 2.8
        Trillion Parameter Frontier", section "Dimension 1", and "Kimi K3
        Architecture Explained ...", section "Token mixing");
  s0    ~ N(0, s0_std) in float32, or no initial state;
  gate  ~ N(0, 1) in the io dtype, for the output-gate epilogue.
Optionally every key channel j = h*dk + i with j % force_every == 0 gets
g = forced_g at every token (stress of the decay floor).
The multi-token decode workload draws T draft tokens per sequence with the
same distributions, and an accepted count per sequence uniform in [0, T].
The packed workload draws B sequence lengths uniform in [T/4, 7T/4) (mean T)
and packs the sequences along the token axis.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_prefill_inputs", "make_decode_state",
           "make_decode_step_inputs", "make_verify_inputs", "make_packed_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    io: str                 # "f32" or "bf16"
    g_std: float = 1.0
    s0_std: Optional[float] = None   # None: zero / absent initial state
    gate: bool = False
    force_every: int = 0    # 0: no forced channels
    forced_g: float = -4.999
    steps: int = 0          # decode workloads: number of single-token steps
    seed: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, T=64, dk=16, dv=16, io="f32", seed=1001),
    "small_prefill": Workload("small_prefill", B=2, H=32, T=4096, dk=128, dv=128, io="bf16",
                              g_std=2.0, s0_std=0.02, seed=1002),
    "full_width_prefill": Workload("full_width_prefill", B=1, H=96, T=32768, dk=128, dv=128,
                                   io="bf16", gate=True, seed=1003),
    "million_token_prefill": Workload("million_token_prefill", B=1, H=96, T=1 << 20, dk=128,
                                      dv=128, io="bf16", force_every=1000, seed=1004),
    "batched_decode": Workload("batched_decode", B=256, H=96, T=1, dk=128, dv=128, io="bf16",
                               s0_std=0.02, steps=64, seed=1005),
    # a serving batch: 16 sequences of 512 .. 3583 tokens packed along the token axis
    "packed_prefill": Workload("packed_prefill", B=16, H=96, T=2048, dk=128, dv=128,
                               io="bf16", gate=True, seed=1007),
    # speculative decoding: T = 4 draft tokens per sequence against the resident state
    "batched_verify": Workload("batched_verify", B=256, H=96, T=4, dk=128, dv=128, io="bf16",
                               s0_std=0.02, gate=True, seed=1006),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def _unit_rows(shape, gen, device, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    return x.to(dtype)


def _decay(shape, g_std, gen, device):
    return -5.0 * torch.sigmoid(g_std * torch.randn(shape, generator=gen, device=device,
                                                    dtype=torch.float32))


def _force_channels(g, H, dk, every, value):
    if every <= 0:
        return g
    j = torch.arange(H * dk, device=g.device).view(H, dk)
    mask = (j % every) == 0
    g[..., mask] = value
    return g


def make_prefill_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                        T: Optional[int] = None, t_offset_slab: int = 0):
    """Draw one prefill batch.  Returns a dict of tensors on ``device``.

    ``T`` overrides the workload's length (for sub-sequence slabs); slab
    ``t_offset_slab`` uses its own seed so a long sequence can be produced in
    pieces without holding float32 temporaries for all of it.
    """
    T = w.T if T is None else T
    seed = (w.seed if seed is None else seed) + 7919 * t_offset_slab
    gen = _gen(seed, device)
    dt = _DT[w.io]
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    out = {
        "q": _unit_rows((B, T, H, dk), gen, device, dt),
        "k": _unit_rows((B, T, H, dk), gen, device, dt),
        "v": torch.randn((B, T, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt),
        "beta": torch.sigmoid(torch.randn((B, T, H), generator=gen, device=device,
                                          dtype=torch.float32)),
    }
    g = _decay((B, T, H, dk), w.g_std, gen, device)
    out["g"] = _force_channels(g, H, dk, w.force_every, w.forced_g)
    if w.s0_std is not None and t_offset_slab == 0:
        out["s0"] = w.s0_std * torch.randn((B, H, dk, dv), generator=gen, device=device,
                                           dtype=torch.float32)
    else:
        out["s0"] = None
    if w.gate:
        out["gate"] = torch.randn((B, T, H, dv), generator=gen, device=device,
                                  dtype=torch.float32).to(dt)
    else:
        out["gate"] = None
    return out


def make_decode_state(w: Workload, device="cpu", seed: Optional[int] = None):
    """Resident float32 state [B, H, dk, dv] ~ N(0, s0_std)."""
    gen = _gen(w.seed if seed is None else seed, device)
    std = 0.0 if w.s0_std is None else w.s0_std
    return std * torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=device,
                             dtype=torch.float32)


def make_decode_step_inputs(w: Workload, step: int, device="cpu"):
    """Fresh single-token inputs for decode step ``step`` (seed 2000 + step)."""
    gen = _gen(2000 + step, device)
    dt = _DT[w.io]
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    out = {
        "q": _unit_rows((B, H, dk), gen, device, dt),
        "k": _unit_rows((B, H, dk), gen, device, dt),
        "v": torch.randn((B, H, dv), generator=gen, device=device, dtype=torch.float32).to(dt),
        "beta": torch.sigmoid(torch.randn((B, H), generator=gen, device=device,
                                          dtype=torch.float32)),
        "g": _decay((B, H, dk), w.g_std, gen, device),
    }
    out["gate"] = (torch.randn((B, H, dv), generator=gen, device=device,
                               dtype=torch.float32).to(dt) if w.gate else None)
    return out


def make_verify_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """T draft tokens per sequence ([B, T, H, *] tensors, seed w.seed + 1), the
    gate when the workload has one, and ``n_commit``: an accepted count per
    sequence, int32 uniform in [0, T]."""
    x = make_prefill_inputs(w, device=device, seed=(w.seed if seed is None else seed) + 1)
    gen = _gen((w.seed if seed is None else seed) + 2, device)
    x["n_commit"] = torch.randint(0, w.T + 1, (w.B,), generator=gen, device=device,
                                  dtype=torch.int32)
    del x["s0"]
    return x


def make_packed_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """B sequences of lengths uniform in [T/4, 7T/4) packed along the token axis:
    q, k, g [total, H, dk], v, gate [total, H, dv], beta [total, H], the int32
    offsets ``cu_seqlens`` [B + 1] and the host list ``lens``."""
    seed = w.seed if seed is None else seed
    lens = torch.randint(w.T // 4, 7 * w.T // 4, (w.B,), generator=_gen(seed + 3, "cpu"))
    total = int(lens.sum())
    flat = dataclasses.replace(w, B=1, T=total)
    x = make_prefill_inputs(flat, device=device, seed=seed)
    out = {key: (t[0] if t is not None and key != "s0" else t) for key, t in x.items()}
    del out["s0"]
    cu = torch.zeros(w.B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0)
    out["cu_seqlens"] = cu.to(device)
    out["lens"] = [int(n) for n in lens]
    return out
