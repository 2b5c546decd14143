"""Throughput of the KDA layer core on one MI355X, with roofline and CPU-oracle context.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one ``kda_chunk_fwd`` call (the whole chunkwise prefill: tile load,
cumulative log-decay, rescaled operands, intra-tile products, UT solve, WY
factors, delta correction, outputs, state pass, final state and the fused
RMSNorm x sigmoid(gate) epilogue) over one batch of seeded synthetic inputs
already resident in HBM.  The default workload is the full-width layer prefill
(B=1, H=96, T=32768, dk=dv=128, bf16 q/k/v/gate, fp32 g/beta/state, epilogue
on).  A second leg times the batched decode workload (B=256, H=96, 64
successive single-token steps against a 1.6 GB fp32 state) and reports its
HBM rate in the ``decode`` object of the same JSON line; a third times the
multi-token decode step of speculative decoding (B=256, H=96, 4 draft tokens:
one verify call and one commit call) in the ``verify`` object, and the prefill
with a state checkpoint every 2048 tokens in the ``checkpoints`` object, and a
packed serving batch (16 sequences of 512-3583 tokens, H=96, gated) in the
``packed`` object; the same layer from the raw projections (q, k normalised
and the decay and write strength formed from logits in the kernels) in the
``prologue`` object.

Output: ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=96,dk=dv=128) + decode GB/s, % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3        # MI355X fp32, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    # path name reported by the library -> source files of its kernels
    "kda_chunk_mfma": ["gated_delta_rule_112_amd/csrc/kda_chunk_tile.h",
                       "gated_delta_rule_112_amd/csrc/kda_chunk_state.hip",
                       "gated_delta_rule_112_amd/csrc/kda_chunk_rec.h"],
    "kda_chunk_valu": ["gated_delta_rule_112_amd/csrc/kda_chunk_valu.hip"],
    "kda_decode": ["gated_delta_rule_112_amd/csrc/kda_decode.hip"],
    "kda_bwd_chunk": ["gated_delta_rule_112_amd/csrc/kda_bwd_chunk.hip",
                      "gated_delta_rule_112_amd/csrc/kda_chunk_tile.h",
                      "gated_delta_rule_112_amd/csrc/kda_chunk_state.hip",
                      "gated_delta_rule_112_amd/csrc/kda_chunk_rec.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic units
def prefill_bytes(B, T, H, dk, dv, es, with_o=True, with_gate=False, with_s0=False, with_sout=True):
    """Bytes a prefill must move at least: every input read once, every output
    written once.  Per token-head: q, k (dk each) and v (dv) in the io dtype,
    g (dk fp32), beta (fp32), o (dv io) and gate (dv io) when present; per
    (b, h): the fp32 state in and/or out."""
    per_tok = (2 * dk + dv) * es + 4 * dk + 4
    if with_o:
        per_tok += dv * es
    if with_gate:
        per_tok += dv * es
    per_bh = 4 * dk * dv * (int(with_s0) + int(with_sout))
    return B * T * H * per_tok + B * H * per_bh, per_tok


def prefill_flops(B, T, H, dk, dv, C=16):
    """Flops of the chunked method per token-head: 6*C*dk + 4*C*dv + 6*dk*dv
    (intra-tile products, WY factors, delta correction, outputs, state pass)."""
    return B * T * H * (6 * C * dk + 4 * C * dv + 6 * dk * dv)


def decode_bytes(B, H, dk, dv, es, with_gate=False):
    """Per (b, h) per step: the fp32 state read and written once, q, k, v, o in
    the io dtype, g fp32, beta fp32 (gate when present)."""
    per = 8 * dk * dv + (2 * dk + dv) * es + 4 * dk + 4 + dv * es
    if with_gate:
        per += dv * es
    return B * H * per, per


def verify_bytes(B, H, K, dk, dv, es, n_commit, with_gate=True):
    """Multi-token decode (speculative decoding), per (b, h).  Verify (outputs
    of all K draft tokens, nothing committed): the fp32 state read once and K
    tokens of q, k, v (io), g, beta (fp32), gate and o (io).  Commit (accepted
    n_b tokens of sequence b, no outputs): the state read and written once when
    n_b > 0, n_b tokens of q, k, v, g, beta, and the int32 count."""
    tok_in = (2 * dk + dv) * es + 4 * dk + 4
    tok_verify = tok_in + dv * es * (2 if with_gate else 1)
    verify = B * H * (4 * dk * dv + K * tok_verify)
    commit = sum(H * ((8 * dk * dv if n > 0 else 0) + n * tok_in) + 4 for n in n_commit)
    return verify, commit


# ----------------------------------------------------------------------------- HBM traffic record
def source_digest(kernel):
    path = KERNEL_SOURCES.get(kernel)
    if path is None:
        return None
    h = hashlib.sha256()
    for p in [*path, "gated_delta_rule_112_amd/csrc/kda_device.h"]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per step (one kda_chunk_fwd or kda_decode_step call, summed
    over its launches) from the committed rocprofv3 counter record, or None
    when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(kernel, {}).get(workload)
    if not e or e.get("source_sha256") != source_digest(kernel):
        return None
    return e.get("bytes_per_step")


# ----------------------------------------------------------------------------- CPU oracle leg
def _oracle_worker(args):
    """Run the float64 oracle on a few heads of a workload-shaped sample."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    name, heads, T, seed = args
    import torch  # CPU only in this process
    torch.set_num_threads(1)
    from gated_delta_rule_112_amd.inputs import WORKLOADS, make_prefill_inputs
    from oracle.kda_oracle import gate_rmsnorm, kda_recurrent
    import dataclasses
    w = dataclasses.replace(WORKLOADS[name], B=1, H=heads, T=T)
    x = make_prefill_inputs(w, device="cpu", seed=seed)
    f = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    t0 = time.perf_counter()
    done = 0
    for h in range(heads):
        sl = lambda t: None if t is None else t[:, :, h:h + 1]  # noqa: E731
        o, _ = kda_recurrent(f(sl(x["q"])), f(sl(x["k"])), f(sl(x["v"])), f(sl(x["g"])),
                             f(sl(x["beta"])), None if x["s0"] is None else f(x["s0"][:, h:h + 1]))
        if x["gate"] is not None:
            gate_rmsnorm(o, f(sl(x["gate"])), None, 1e-6)
        done += T
    return done, time.perf_counter() - t0


def _decode_oracle_worker(args):
    """The float64 oracle's decode step over a sample of (b, h) states of the
    batched decode workload, for every one of its steps."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    n_bh, steps, seed = args
    import numpy as np
    rng = np.random.default_rng(seed)
    from oracle.kda_oracle import gate_rmsnorm, kda_decode_step
    dk = dv = 128
    S = 0.02 * rng.standard_normal((n_bh, dk, dv))
    t0 = time.perf_counter()
    for _ in range(steps):
        q = rng.standard_normal((n_bh, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((n_bh, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((n_bh, dv))
        g = -5.0 / (1.0 + np.exp(-rng.standard_normal((n_bh, dk))))
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(n_bh)))
        o, S = kda_decode_step(q, k, v, g, beta, S)
        gate_rmsnorm(o, rng.standard_normal((n_bh, dv)), None, 1e-6)
    return n_bh * steps, time.perf_counter() - t0


def cpu_decode_baseline(H, workers, bh_per_worker, steps):
    """Oracle decode steps on the host cores: (b, h)-steps/s, as sequence
    tokens/s (each token carries H heads) and as the state bytes it streams."""
    import concurrent.futures as cf
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    jobs = [(bh_per_worker, steps, 60_000 + i) for i in range(workers)]
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        res = list(ex.map(_decode_oracle_worker, jobs))
    bh_steps = sum(r[0] for r in res)
    busy = max(r[1] for r in res)
    return {
        "value": bh_steps / busy / H,
        "unit": "tokens/s",
        "state_gb_per_s": round(bh_steps / busy * 8 * 128 * 128 / 1e9, 2),
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{workers} processes x {bh_per_worker} (b, h) states x {steps} steps of the "
                   f"batched_decode distributions (float64 decode step + epilogue); "
                   f"rate = (b, h)-steps/s / H={H}; slowest worker {busy:.1f} s"),
    }


def cpu_baseline(workload, H, workers, heads_per_worker, T):
    """Oracle token-heads/s on the host cores, converted to tokens/s of the
    workload (each token carries H heads)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    jobs = [(workload, heads_per_worker, T, 50_000 + i) for i in range(workers)]
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_worker, jobs))
    wall = time.perf_counter() - t0
    token_heads = sum(r[0] for r in res)
    busy = max(r[1] for r in res)
    return {
        "value": token_heads / busy / H,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"{workers} processes x {heads_per_worker} heads x {T} tokens of the "
                   f"{workload} distributions (float64 token-by-token recurrence"
                   f"{' + epilogue' if workload == 'full_width_prefill' else ''}); "
                   f"rate = token-heads/s / H={H}; slowest worker {busy:.1f} s, wall {wall:.1f} s"),
    }


# ----------------------------------------------------------------------------- GPU legs
def bench_prefill(kda, torch, w, steps, warmup):
    from gated_delta_rule_112_amd.inputs import make_prefill_inputs
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name} inputs on the device")
    x = make_prefill_inputs(w, device=dev)
    io = x["q"].dtype
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=io, device=dev)
    s_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    nws = kda.chunk_workspace_size(w.B, w.T, w.H, w.dk, w.dv, io)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    log(f"[bench] workspace {nws / 2**20:.1f} MiB")
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gate=x["gate"],
                      out=out, s_out=s_out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({warmup}); timing {steps} prefill steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del x, out, s_out, ws
    return ms, io


def bench_prefill_median(kda, torch, w, reps, evict_bytes=0, output=True):
    """Median over ``reps`` single prefill calls of workload ``w``, each timed by
    HIP events on the launch stream.  With ``evict_bytes``, a buffer that size
    is overwritten between calls (outside the timed region) so that no input
    is left in the 256 MB memory-side cache; with ``output`` False only the
    final state is computed (o = NULL).  Returns (median ms, all ms)."""
    from gated_delta_rule_112_amd.inputs import make_prefill_inputs
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name} inputs on the device")
    x = make_prefill_inputs(w, device=dev)
    io = x["q"].dtype
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=io, device=dev) if output else None
    s_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    nws = kda.chunk_workspace_size(w.B, w.T, w.H, w.dk, w.dv, io)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    evict = torch.empty(evict_bytes // 4, dtype=torch.float32, device=dev) if evict_bytes else None
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], gate=x["gate"],
                      out=out, s_out=s_out, output=output, workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    times = []
    for i in range(reps):
        if evict is not None:
            evict.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del x, out, s_out, ws, evict
    torch.cuda.empty_cache()
    st = sorted(times)
    return st[len(st) // 2], times


def prefill_leg(kda, torch, w, reps, evict_bytes=0, output=True):
    """One prefill workload as a bench sub-object: tokens/s and its HBM
    roofline fraction (algorithmic bytes of the call / median time)."""
    ms, _ = bench_prefill_median(kda, torch, w, reps, evict_bytes, output)
    es = 2 if w.io == "bf16" else 4
    nbytes, per_tok = prefill_bytes(w.B, w.T, w.H, w.dk, w.dv, es, with_o=output,
                                    with_gate=w.gate, with_s0=w.s0_std is not None)
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = prefill_flops(w.B, w.T, w.H, w.dk, w.dv)
    leg = {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "output": output,
           "reps": reps, "evict_bytes_between_reps": evict_bytes,
           "ms_median": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes": nbytes, "bytes_per_token_head": per_tok,
                        "matrix_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    log(f"[bench] {w.name} (o {'written' if output else 'NULL'}): {ms:.3f} ms, "
        f"{w.B * w.T / (ms * 1e-3) / 1e6:.2f} M tok/s, {gbs:.0f} GB/s")
    return leg


def bench_checkpoints(kda, torch, w, every, steps):
    """The prefill of ``bench_prefill`` with a state checkpoint every ``every``
    tokens (prefix caching); returns ms per step."""
    from gated_delta_rule_112_amd.inputs import make_prefill_inputs
    dev = torch.device("cuda:0")
    x = make_prefill_inputs(w, device=dev)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    s_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ck = torch.empty((w.B, w.T // every, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    nws = kda.chunk_workspace_size(w.B, w.T, w.H, w.dk, w.dv, x["q"].dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd_checkpoints(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"],
                                  every=every, gate=x["gate"], out=out, s_out=s_out, ckpt=ck,
                                  workspace=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prologue(kda, torch, w, steps):
    """The prefill of ``bench_prefill`` from the raw projections: q and k
    unnormalised (normalised in the kernels), the decay and write strength as
    logits (a in the io dtype in place of float32 g, b in place of beta);
    returns ms per step."""
    from gated_delta_rule_112_amd.inputs import make_prefill_inputs
    dev = torch.device("cuda:0")
    x = make_prefill_inputs(w, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 11)
    a = torch.randn(x["g"].shape, generator=gen, device=dev).to(x["q"].dtype)
    b = torch.randn(x["beta"].shape, generator=gen, device=dev)
    del x["g"], x["beta"]
    x["q"] = (3.0 * x["q"].float()).to(x["v"].dtype)  # raw projections: not unit vectors
    x["k"] = (0.5 * x["k"].float()).to(x["v"].dtype)
    out = torch.empty((w.B, w.T, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    s_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    nws = kda.chunk_workspace_size(w.B, w.T, w.H, w.dk, w.dv, x["q"].dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], a, b, x["s0"], gate=x["gate"], out=out,
                      s_out=s_out, workspace=ws, prologue=True, stream=stream)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_packed(kda, torch, w, steps, prologue=False):
    """Prefill of a packed serving batch (kda_chunk_fwd_varlen; with
    ``prologue``, from the raw projections as in ``bench_prologue``:
    kda_chunk_fwd_varlen_prologue); returns (ms per step, total tokens, longest
    length)."""
    from gated_delta_rule_112_amd.inputs import make_packed_inputs
    dev = torch.device("cuda:0")
    x = make_packed_inputs(w, device=dev)
    if prologue:
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 11)
        x["g"] = torch.randn(x["g"].shape, generator=gen, device=dev).to(x["q"].dtype)
        x["beta"] = torch.randn(x["beta"].shape, generator=gen, device=dev)
        x["q"] = (3.0 * x["q"].float()).to(x["v"].dtype)
        x["k"] = (0.5 * x["k"].float()).to(x["v"].dtype)
    max_len = max(x["lens"])
    total = x["q"].shape[0]
    out = torch.empty((total, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    s_out = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    nws = kda.chunk_workspace_size(w.B, max_len, w.H, w.dk, w.dv, x["q"].dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                             max_len, gate=x["gate"], out=out, s_out=s_out, workspace=ws,
                             stream=stream, prologue=prologue)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, total, max_len


def bench_backward(kda, torch, w, steps):
    """The backward pass (kda_recurrent_bwd) over a prefill workload's inputs,
    with dO drawn like v and a final-state gradient; returns ms per call, and ms
    per call of kda_recurrent_bwd_ckpt given the forward's states every 64 tokens
    (kept by one kda_chunk_fwd_checkpoints call beforehand, outside the timing)."""
    from gated_delta_rule_112_amd.inputs import make_prefill_inputs
    dev = torch.device("cuda:0")
    x = make_prefill_inputs(w, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 21)
    dout = torch.randn(x["v"].shape, generator=gen, device=dev).to(x["v"].dtype)
    dsf = torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=dev)
    nws = kda.load_library().kda_recurrent_bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    scale = w.dk ** -0.5
    _, _, ck = kda.chunk_fwd_checkpoints(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"],
                                         every=64, scale=scale, output=False, stream=stream)

    def timed(ckpt):
        def step():
            kda.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dout, x["s0"], dsf,
                              scale=scale, workspace=ws, stream=stream, ckpt=ckpt)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    return timed(None), timed(ck)


def bench_decode(kda, torch, w, repeats=1):
    from gated_delta_rule_112_amd.inputs import make_decode_state, make_decode_step_inputs
    dev = torch.device("cuda:0")
    log(f"[bench] decode: state {w.B}x{w.H}x{w.dk}x{w.dv} fp32, {w.steps} steps")
    state = make_decode_state(w, device=dev)
    xs = [make_decode_step_inputs(w, s, device=dev) for s in range(w.steps)]
    io = xs[0]["q"].dtype
    outs = [torch.empty((w.B, w.H, w.dv), dtype=io, device=dev) for _ in range(w.steps)]
    stream = torch.cuda.current_stream(dev)

    def run(n):
        for s in range(n):
            x = xs[s]
            kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, gate=x["gate"],
                            out=outs[s], stream=stream)

    run(1)  # warm-up step
    torch.cuda.synchronize()
    best = None
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(w.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / w.steps
        best = ms if best is None else min(best, ms)
    return best, io


def bench_verify(kda, torch, w, repeats=20):
    """Time the verify call (K draft tokens, outputs, state untouched) and the
    commit call (accepted counts, no outputs) of the multi-token decode step."""
    from gated_delta_rule_112_amd.inputs import make_decode_state, make_verify_inputs
    dev = torch.device("cuda:0")
    log(f"[bench] verify: state {w.B}x{w.H}x{w.dk}x{w.dv} fp32, {w.T} draft tokens")
    state = make_decode_state(w, device=dev)
    x = make_verify_inputs(w, device=dev)
    stream = torch.cuda.current_stream(dev)
    zeros = torch.zeros(w.B, dtype=torch.int32, device=dev)
    y = torch.empty((w.B, w.T, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    ins = [x[key] for key in ["q", "k", "v", "g", "beta"]]

    def verify():
        kda.decode_multi(*ins, state, zeros, gate=x["gate"], out=y, stream=stream)

    def commit():
        kda.decode_multi(*ins, state, x["n_commit"], output=False, stream=stream)

    res = {}
    for name, fn in [("verify", verify), ("commit", commit)]:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(repeats):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / repeats
    return res, x["n_commit"].cpu().tolist(), x["q"].dtype


def stream_ceiling(torch, nbytes, reps=20):
    """The streaming ceiling the decode step is held to: an in-place
    read-modify-write of a float32 buffer of the decode state's size (torch's
    vectorised elementwise kernel, x *= c) and a copy between two such buffers;
    GB/s counting every byte read and every byte written."""
    dev = torch.device("cuda:0")
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn in [("rmw", lambda: x.mul_(1.0000001)), ("copy", lambda: y.copy_(x))]:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"{name}_gbs"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    del x, y
    return res


def copy_probe(torch, nbytes=1 << 30):
    """A plain device copy of known size, run once so that a counter pass over
    this process can scale FETCH_SIZE / WRITE_SIZE against it."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: {nbytes} bytes read, {nbytes} bytes written")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full_width_prefill",
                    choices=["small_prefill", "full_width_prefill", "million_token_prefill"])
    ap.add_argument("--decode-repeats", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-checkpoints", action="store_true")
    ap.add_argument("--no-packed", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-small", action="store_true", help="skip the small-prefill leg")
    ap.add_argument("--no-million", action="store_true", help="skip the million-token leg")
    ap.add_argument("--cpu-heads-per-worker", type=int, default=4)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (for counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA layer core here is a single-GPU "
              "library (heads and batch shard across GPUs without communication), so "
              "--gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    from gated_delta_rule_112_amd.inputs import WORKLOADS
    w = WORKLOADS[a.workload]

    # The oracle leg runs first, in spawned CPU-only processes, before this
    # process touches the GPU.
    cpu = cpu_dec = None
    if not a.no_cpu_baseline:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"[bench] cpu oracle leg: {workers} workers")
        cpu = cpu_baseline(a.workload, w.H, workers, a.cpu_heads_per_worker,
                           min(a.cpu_tokens, w.T))
        log(f"[bench] cpu oracle: {cpu['value']:.1f} tokens/s")
        cpu_dec = None
        if not a.no_decode:
            cpu_dec = cpu_decode_baseline(96, workers, 384, 64)
            log(f"[bench] cpu oracle decode: {cpu_dec['value']:.1f} tokens/s")

    import torch
    import gated_delta_rule_112_amd as kda
    kda.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (HIP device); none is visible", file=sys.stderr)
        sys.exit(3)

    if a.copy_probe:
        copy_probe(torch)

    ms, io = bench_prefill(kda, torch, w, a.steps, a.warmup)
    es = 2 if io == torch.bfloat16 else 4
    nbytes, per_tok = prefill_bytes(w.B, w.T, w.H, w.dk, w.dv, es, with_o=True,
                                    with_gate=w.gate, with_s0=w.s0_std is not None)
    flops = prefill_flops(w.B, w.T, w.H, w.dk, w.dv)
    kernel = kda.chunk_kernel_name(w.dk, w.dv, io)
    achieved = nbytes / (ms * 1e-3) / 1e9
    tokens_per_s = w.B * w.T / (ms * 1e-3)
    mfma = kernel == "kda_chunk_mfma"
    roofline = {
        "bound": "hbm",
        "kernel": kernel,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(kernel, w.name),
        "algorithmic_bytes_per_step": nbytes,
        "launches_per_step": kda.chunk_launches(w.B, w.T, w.H, w.dk, w.dv, io),
        "bytes_per_token_head": per_tok,
        "matrix_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "matrix_frac": round(flops / (ms * 1e-3) / 1e12 /
                             (BF16_PEAK_TFLOPS if mfma else F32_PEAK_TFLOPS), 4),
    }
    log(f"[bench] prefill {ms:.3f} ms/step, {tokens_per_s / 1e6:.2f} M tok/s, "
        f"{achieved:.0f} GB/s ({kernel})")

    checkpoints = None
    if not a.no_checkpoints:
        every = 2048
        cms = bench_checkpoints(kda, torch, w, every, a.steps)
        ck_bytes = w.B * (w.T // every) * w.H * w.dk * w.dv * 4
        checkpoints = {"every_tokens": every, "ms_per_step": round(cms, 4),
                       "checkpoint_bytes": ck_bytes,
                       "overhead_vs_prefill": round(cms / ms - 1.0, 4)}
        log(f"[bench] prefill with a checkpoint every {every} tokens: {cms:.3f} ms/step")

    small = None
    if not a.no_small:  # 0.41 GB per call: a 512 MB write between calls evicts the inputs
        small = prefill_leg(kda, torch, WORKLOADS["small_prefill"], 20, evict_bytes=512 << 20)

    million = None
    if not a.no_million:
        wm = WORKLOADS["million_token_prefill"]
        million = {"with_o": prefill_leg(kda, torch, wm, 5),
                   "state_only": prefill_leg(kda, torch, wm, 5, output=False)}

    prologue = None
    if not a.no_prologue:
        gms = bench_prologue(kda, torch, w, a.steps)
        gbytes = nbytes - w.B * w.T * w.H * w.dk * (4 - es)  # a in the io dtype, not fp32 g
        ggbs = gbytes / (gms * 1e-3) / 1e9
        prologue = {"ms_per_step": round(gms, 4), "tokens_per_s": round(w.B * w.T / (gms * 1e-3), 1),
                 "algorithmic_bytes_per_step": gbytes, "achieved": round(ggbs, 1),
                 "unit": "GB/s", "peak": HBM_PEAK_GBS, "frac": round(ggbs / HBM_PEAK_GBS, 4)}
        log(f"[bench] prefill from raw q, k and gate logits: {gms:.3f} ms/step, "
            f"{w.B * w.T / (gms * 1e-3) / 1e6:.2f} M tok/s")

    packed = None
    if not a.no_packed:
        wp = WORKLOADS["packed_prefill"]
        pms, ptot, pmax = bench_packed(kda, torch, wp, a.steps)
        pbytes, _ = prefill_bytes(1, ptot, wp.H, wp.dk, wp.dv, 2, with_o=True,
                                  with_gate=wp.gate, with_s0=False)
        pbytes += (wp.B - 1) * wp.H * 4 * wp.dk * wp.dv  # one final state per sequence
        pgbs = pbytes / (pms * 1e-3) / 1e9
        packed = {"workload": wp.name, "sequences": wp.B, "H": wp.H, "total_tokens": ptot,
                  "longest": pmax, "ms_per_step": round(pms, 4),
                  "tokens_per_s": round(ptot / (pms * 1e-3), 1),
                  "achieved": round(pgbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
                  "frac": round(pgbs / HBM_PEAK_GBS, 4)}
        log(f"[bench] packed batch: {wp.B} sequences, {ptot} tokens (longest {pmax}): "
            f"{pms:.3f} ms, {ptot / (pms * 1e-3) / 1e6:.2f} M tok/s")
        if not a.no_prologue:  # the same batch from the raw projections
            rms, _, _ = bench_packed(kda, torch, wp, a.steps, prologue=True)
            packed["prologue_ms"] = round(rms, 4)
            packed["prologue_tokens_per_s"] = round(ptot / (rms * 1e-3), 1)
            log(f"[bench] packed batch from raw projections: {rms:.3f} ms, "
                f"{ptot / (rms * 1e-3) / 1e6:.2f} M tok/s")

    backward = None
    if not a.no_backward:
        wb = WORKLOADS["small_prefill"]
        bms, bcms = bench_backward(kda, torch, wb, 3)
        ntok = wb.B * wb.T
        # per token and head: q, k, v, dO read and dq, dk, dv written (io dtype),
        # g read and dg written (float32), beta and dbeta; plus s0, dS_T, ds0 per head
        es = 2 if wb.io == "bf16" else 4
        per = 7 * wb.dk * es + 2 * wb.dk * 4 + 8
        bbytes = ntok * wb.H * per + 3 * wb.B * wb.H * wb.dk * wb.dv * 4
        bgbs = bbytes / (bms * 1e-3) / 1e9
        backward = {"workload": wb.name, "B": wb.B, "H": wb.H, "T": wb.T,
                    "ms": round(bms, 4), "tokens_per_s": round(ntok / (bms * 1e-3), 1),
                    "algorithmic_bytes": bbytes, "achieved": round(bgbs, 1), "unit": "GB/s",
                    "peak": HBM_PEAK_GBS, "frac": round(bgbs / HBM_PEAK_GBS, 4),
                    "kernel": "kda_bwd_chunk",
                    "traffic": measured_traffic("kda_bwd_chunk", wb.name),
                    "with_forward_checkpoints_ms": round(bcms, 4)}
        log(f"[bench] backward ({wb.name}): {bms:.3f} ms, "
            f"{ntok / (bms * 1e-3) / 1e6:.3f} M tok/s; given the forward's checkpoints "
            f"{bcms:.3f} ms")

    decode = None
    if not a.no_decode:
        wd = WORKLOADS["batched_decode"]
        dms, dio = bench_decode(kda, torch, wd, a.decode_repeats)
        des = 2 if dio == torch.bfloat16 else 4
        dbytes, dper = decode_bytes(wd.B, wd.H, wd.dk, wd.dv, des, wd.gate)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        decode = {
            "workload": wd.name, "B": wd.B, "H": wd.H, "dk": wd.dk, "dv": wd.dv,
            "steps": wd.steps, "ms_per_step": round(dms, 4),
            "tokens_per_s": round(wd.B / (dms * 1e-3), 1),
            "roofline": {"bound": "hbm", "kernel": "kda_decode", "achieved": round(dgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("kda_decode", wd.name),
                         "algorithmic_bytes_per_step": dbytes,
                         "bytes_per_bh": dper},
            "cpu_baseline": cpu_dec,
        }
        log(f"[bench] decode {dms:.4f} ms/step, {dgbs:.0f} GB/s")
        ceil = stream_ceiling(torch, wd.B * wd.H * wd.dk * wd.dv * 4)
        ceil["decode_frac_of_rmw"] = round(dgbs / ceil["rmw_gbs"], 4)
        decode["streaming_ceiling"] = ceil
        log(f"[bench] streaming ceiling over the state's size: in-place read-modify-write "
            f"{ceil['rmw_gbs']:.0f} GB/s, copy {ceil['copy_gbs']:.0f} GB/s")

    verify = None
    if not a.no_verify:
        wv = WORKLOADS["batched_verify"]
        vms, n_commit, vio = bench_verify(kda, torch, wv)
        ves = 2 if vio == torch.bfloat16 else 4
        vb, cb = verify_bytes(wv.B, wv.H, wv.T, wv.dk, wv.dv, ves, n_commit, wv.gate)
        verify = {"workload": wv.name, "B": wv.B, "H": wv.H, "draft_tokens": wv.T,
                  "dk": wv.dk, "dv": wv.dv, "accepted_tokens": int(sum(n_commit))}
        for name, nb in [("verify", vb), ("commit", cb)]:
            gbs = nb / (vms[name] * 1e-3) / 1e9
            verify[name] = {"ms": round(vms[name], 4), "algorithmic_bytes": nb,
                            "achieved": round(gbs, 1), "unit": "GB/s", "peak": HBM_PEAK_GBS,
                            "frac": round(gbs / HBM_PEAK_GBS, 4)}
            log(f"[bench] {name} {vms[name]:.4f} ms, {gbs:.0f} GB/s")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mfma else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "chunk": 16, "io": w.io, "epilogue": w.gate,
                   "initial_state": w.s0_std is not None},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "small_prefill": small,
        "million_token_prefill": million,
        "checkpoints": checkpoints,
        "packed": packed,
        "prologue": prologue,
        "decode": decode,
        "verify": verify,
        "backward": backward,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
