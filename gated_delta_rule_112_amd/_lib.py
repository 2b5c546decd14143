"""ctypes binding over libkda.so (the C ABI declared in include/kda.h).

Argument marshalling only: this module allocates output tensors with torch,
checks that tensors are contiguous CUDA tensors of the right dtype, and passes
raw device pointers and the current stream to the library.  Every step of the
computation runs in the library's HIP kernels.  If the library is missing,
every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
_IO = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}

_lib = None


class KDAError(RuntimeError):
    """A non-OK kda_status returned by the library."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkda.so once (in-tree build).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m gated_delta_rule_112_amd.build` "
            "(hipcc, gfx950). The KDA ops have no fallback.")
    lib = ctypes.CDLL(p)
    vp, f32, i64, ci = ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                  i64, i64, i64, ci, ci, f32, ci, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_fwd.restype = ci
    lib.kda_chunk_fwd_checkpoints.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                              i64, i64, i64, ci, ci, f32, ci, vp,
                                              ctypes.c_size_t, vp, i64, vp]
    lib.kda_chunk_fwd_checkpoints.restype = ci
    lib.kda_chunk_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp,
                                         vp, f32, i64, ci, ci, f32, ci, vp, ctypes.c_size_t,
                                         vp, i64, vp]
    lib.kda_chunk_fwd_varlen.restype = ci
    lib.kda_recurrent_bwd.argtypes = [vp] * 14 + [i64, i64, i64, ci, ci, f32, ci, vp,
                                                 ctypes.c_size_t, vp]
    lib.kda_recurrent_bwd.restype = ci
    lib.kda_recurrent_bwd_ckpt.argtypes = [vp] * 15 + [i64, i64, i64, ci, ci, f32, ci, vp,
                                                      ctypes.c_size_t, vp]
    lib.kda_recurrent_bwd_ckpt.restype = ci
    lib.kda_recurrent_bwd_workspace_size.argtypes = [i64, i64, i64, ci, ci]
    lib.kda_recurrent_bwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_varlen_prologue.argtypes = lib.kda_chunk_fwd_varlen.argtypes
    lib.kda_chunk_fwd_varlen_prologue.restype = ci
    lib.kda_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, ci, ci, ci]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_launches.argtypes = [i64, i64, i64, ci, ci, ci]
    lib.kda_chunk_fwd_launches.restype = i64
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                    i64, i64, ci, ci, f32, ci, vp]
    lib.kda_decode_step.restype = ci
    lib.kda_chunk_fwd_prologue.argtypes = lib.kda_chunk_fwd.argtypes
    lib.kda_chunk_fwd_prologue.restype = ci
    lib.kda_decode_step_prologue.argtypes = lib.kda_decode_step.argtypes
    lib.kda_decode_step_prologue.restype = ci
    lib.kda_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                     i64, i64, i64, ci, ci, f32, ci, vp]
    lib.kda_decode_multi.restype = ci
    lib.kda_decode_multi_prologue.argtypes = lib.kda_decode_multi.argtypes
    lib.kda_decode_multi_prologue.restype = ci
    lib.kda_gate_rmsnorm.argtypes = [vp, vp, vp, vp, i64, ci, f32, ci, vp]
    lib.kda_gate_rmsnorm.restype = ci
    lib.kda_status_string.argtypes = [ci]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_kernel.argtypes = [ci, ci, ci]
    lib.kda_chunk_fwd_kernel.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ci
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                          i64, i64, i64, ci, ci, f32, ci, vp]
    lib.kda_chunk_fwd_noalloc.restype = ci
    lib.kda_chunk_fwd_noalloc_scratch_bytes.argtypes = []
    lib.kda_chunk_fwd_noalloc_scratch_bytes.restype = ctypes.c_size_t
    if path is None:
        _lib = lib
    return lib


def _check(lib, fn: str, status: int):
    if status != 0:
        raise KDAError(fn, status, lib.kda_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def chunk_fwd(q, k, v, g, beta, s0=None, *, scale: float = 1.0, gate=None, norm_w=None,
              eps: float = 1e-6, output: bool = True, final_state: bool = True,
              out=None, s_out=None, workspace=None, prologue: bool = False,
              stream=None) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Prefill over [B, T, H, *] tensors; returns (o or y, final state).

    ``output=False`` computes the final state only; ``s_out`` may be ``s0``
    for an in-place state update.  ``workspace`` (a uint8 CUDA tensor of at
    least ``chunk_workspace_size(...)`` bytes) is allocated per call if absent.
    ``prologue=True``: q and k are the raw projections (normalised in the
    kernels), ``g`` holds the log-decay logits a (io dtype) and ``beta`` the
    write-strength logits b; the kernels form g = -5 sigmoid(a) and
    beta = sigmoid(b).
    """
    o, s, _ = _chunk_fwd(q, k, v, g, beta, s0, scale, gate, norm_w, eps, output, final_state,
                         out, s_out, workspace, 0, None, stream, prologue)
    return o, s


def chunk_fwd_noalloc(q, k, v, g, beta, s0=None, *, scale: float = 1.0, gate=None,
                      norm_w=None, eps: float = 1e-6, output: bool = True,
                      final_state: bool = True, out=None, s_out=None,
                      stream=None) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """``chunk_fwd`` through kda_chunk_fwd_noalloc: no workspace, the library's
    fixed device scratch instead (for callers that cannot allocate; pass ``out``
    and ``s_out`` to allocate nothing here either)."""
    o, s, _ = _chunk_fwd(q, k, v, g, beta, s0, scale, gate, norm_w, eps, output, final_state,
                         out, s_out, None, 0, None, stream, noalloc=True)
    return o, s


def chunk_fwd_checkpoints(q, k, v, g, beta, s0=None, *, every: int, scale: float = 1.0,
                          gate=None, norm_w=None, eps: float = 1e-6, output: bool = True,
                          final_state: bool = True, out=None, s_out=None, ckpt=None,
                          workspace=None, stream=None):
    """``chunk_fwd`` that also returns the state after every ``every`` tokens
    (a multiple of 32): (o or y, final state, checkpoints [B, T // every, H, dk, dv])."""
    if every <= 0 or every % 32:
        raise ValueError(f"checkpoint interval {every} is not a positive multiple of 32")
    return _chunk_fwd(q, k, v, g, beta, s0, scale, gate, norm_w, eps, output, final_state,
                      out, s_out, workspace, every, ckpt, stream)


def chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, max_len: int, s0=None, *,
                     scale: float = 1.0, gate=None, norm_w=None, eps: float = 1e-6,
                     output: bool = True, final_state: bool = True, out=None, s_out=None,
                     every: int = 0, ckpt=None, workspace=None, stream=None,
                     prologue: bool = False):
    """Prefill over N sequences packed along the token axis: q, k, g [total, H, dk],
    v [total, H, dv], beta [total, H]; ``cu_seqlens`` int32 [N + 1] on the device
    (sequence b is rows cu[b] .. cu[b+1]-1), ``max_len`` >= the longest.  Returns
    (o or y [total, H, dv], final states [N, H, dk, dv], checkpoints
    [N, max_len // every, H, dk, dv] or None when ``every`` is 0).  With
    ``prologue``, q and k are raw, g holds the decay logits a (io dtype) and beta
    the write-strength logits b (kda_chunk_fwd_varlen_prologue)."""
    lib = load_library()
    if q.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev = q.device
    total, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    io = q.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    if N < 1 or max_len < 1:
        raise ValueError("need at least one sequence and max_len >= 1")
    if every and (every < 0 or every % 32):
        raise ValueError(f"checkpoint interval {every} is not a positive multiple of 32")
    _need(q, "q", io, (total, H, dk), dev)
    _need(k, "k", io, (total, H, dk), dev)
    _need(v, "v", io, (total, H, dv), dev)
    _need(g, "a" if prologue else "g", io if prologue else torch.float32, (total, H, dk), dev)
    _need(beta, "beta", torch.float32, (total, H), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if s0 is not None:
        _need(s0, "s0", torch.float32, (N, H, dk, dv), dev)
    if gate is not None:
        _need(gate, "gate", io, (total, H, dv), dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32, (dv,), dev)
    if not output:
        out = None
    elif out is None:
        out = torch.empty((total, H, dv), dtype=io, device=dev)
    else:
        _need(out, "out", io, (total, H, dv), dev)
    if not final_state:
        s_out = None
    elif s_out is None:
        s_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _need(s_out, "s_out", torch.float32, (N, H, dk, dv), dev)
    nck = max_len // every if every else 0
    if every:
        if ckpt is None:
            ckpt = torch.empty((N, nck, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _need(ckpt, "ckpt", torch.float32, (N, nck, H, dk, dv), dev)
    ws_bytes = lib.kda_chunk_fwd_workspace_size(N, max_len, H, dk, dv, _IO[io])
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    fn = "kda_chunk_fwd_varlen_prologue" if prologue else "kda_chunk_fwd_varlen"
    st = getattr(lib, fn)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, total,
        int(max_len), _ptr(s0), _ptr(out), _ptr(s_out), _ptr(gate), _ptr(norm_w), float(eps), H,
        dk, dv, float(scale), _IO[io], _ptr(workspace),
        0 if workspace is None else workspace.numel(), _ptr(ckpt) if nck else None,
        int(every), _stream(dev, stream))
    _check(lib, fn, st)
    return out, s_out, ckpt


def _chunk_fwd(q, k, v, g, beta, s0, scale, gate, norm_w, eps, output, final_state, out, s_out,
               workspace, every, ckpt, stream, prologue=False, noalloc=False):
    lib = load_library()
    if q.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    _need(q, "q", io, (B, T, H, dk), dev)
    _need(k, "k", io, (B, T, H, dk), dev)
    _need(v, "v", io, (B, T, H, dv), dev)
    _need(g, "a" if prologue else "g", io if prologue else torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if s0 is not None:
        _need(s0, "s0", torch.float32, (B, H, dk, dv), dev)
    if gate is not None:
        _need(gate, "gate", io, (B, T, H, dv), dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32, (dv,), dev)
    if output and out is None:
        out = torch.empty((B, T, H, dv), dtype=io, device=dev)
    if not output:
        out = None
    elif out is not None:
        _need(out, "out", io, (B, T, H, dv), dev)
    if final_state and s_out is None:
        s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not final_state:
        s_out = None
    elif s_out is not None:
        _need(s_out, "s_out", torch.float32, (B, H, dk, dv), dev)
    if noalloc:
        st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                       _ptr(out), _ptr(s_out), _ptr(gate), _ptr(norm_w),
                                       float(eps), B, T, H, dk, dv, float(scale), _IO[io],
                                       _stream(dev, stream))
        _check(lib, "kda_chunk_fwd_noalloc", st)
        return out, s_out, None
    ws_bytes = lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, _IO[io])
    if workspace is None and ws_bytes > 0:
        # torch's caching allocator hands out 512-byte aligned blocks
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(out), _ptr(s_out),
            _ptr(gate), _ptr(norm_w), float(eps), B, T, H, dk, dv, float(scale), _IO[io],
            _ptr(workspace), 0 if workspace is None else workspace.numel())
    nck = T // every if every else 0
    if every:
        if ckpt is None:
            ckpt = torch.empty((B, nck, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _need(ckpt, "ckpt", torch.float32, (B, nck, H, dk, dv), dev)
    if prologue:
        st = lib.kda_chunk_fwd_prologue(*args, _stream(dev, stream))
        _check(lib, "kda_chunk_fwd_prologue", st)
        return out, s_out, None
    if nck == 0:  # no checkpoint falls inside the sequence
        _check(lib, "kda_chunk_fwd", lib.kda_chunk_fwd(*args, _stream(dev, stream)))
        return out, s_out, ckpt
    st = lib.kda_chunk_fwd_checkpoints(*args, _ptr(ckpt), int(every), _stream(dev, stream))
    _check(lib, "kda_chunk_fwd_checkpoints", st)
    return out, s_out, ckpt


def decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, gate=None, norm_w=None,
                eps: float = 1e-6, out=None, prologue: bool = False, stream=None) -> torch.Tensor:
    """One token per (b, h) against ``state`` [B, H, dk, dv] (updated in place); returns o.
    ``prologue=True``: raw q, k and the logits a (io dtype) and b in g and beta, as in
    chunk_fwd."""
    lib = load_library()
    if q.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    _need(q, "q", io, (B, H, dk), dev)
    _need(k, "k", io, (B, H, dk), dev)
    _need(v, "v", io, (B, H, dv), dev)
    _need(g, "a" if prologue else "g", io if prologue else torch.float32, (B, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(state, "state", torch.float32, (B, H, dk, dv), dev)
    if gate is not None:
        _need(gate, "gate", io, (B, H, dv), dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32, (dv,), dev)
    if out is None:
        out = torch.empty((B, H, dv), dtype=io, device=dev)
    else:
        _need(out, "out", io, (B, H, dv), dev)
    fn = lib.kda_decode_step_prologue if prologue else lib.kda_decode_step
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out), _ptr(gate),
            _ptr(norm_w), float(eps), B, H, dk, dv, float(scale), _IO[io], _stream(dev, stream))
    _check(lib, "kda_decode_step_prologue" if prologue else "kda_decode_step", st)
    return out


def decode_multi(q, k, v, g, beta, state, n_commit=None, *, scale: float = 1.0, gate=None,
                 norm_w=None, eps: float = 1e-6, output: bool = True, out=None,
                 prologue: bool = False, stream=None) -> Optional[torch.Tensor]:
    """K tokens per sequence ([B, K, H, *] inputs) against ``state`` [B, H, dk, dv].

    Returns the outputs of all K tokens ([B, K, H, dv], or None with
    ``output=False``).  ``state`` is replaced in place by the state after the
    first ``n_commit[b]`` tokens of sequence b (``n_commit``: int32 [B] on the
    device, values clamped into [0, K]; None commits all K tokens).
    ``prologue=True``: raw q, k and the logits a (io dtype) and b in g and beta.
    """
    lib = load_library()
    if q.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev = q.device
    B, K, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    _need(q, "q", io, (B, K, H, dk), dev)
    _need(k, "k", io, (B, K, H, dk), dev)
    _need(v, "v", io, (B, K, H, dv), dev)
    _need(g, "a" if prologue else "g", io if prologue else torch.float32, (B, K, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, K, H), dev)
    _need(state, "state", torch.float32, (B, H, dk, dv), dev)
    if n_commit is not None:
        _need(n_commit, "n_commit", torch.int32, (B,), dev)
    if gate is not None:
        _need(gate, "gate", io, (B, K, H, dv), dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32, (dv,), dev)
    if not output:
        out = None
    elif out is None:
        out = torch.empty((B, K, H, dv), dtype=io, device=dev)
    else:
        _need(out, "out", io, (B, K, H, dv), dev)
    fn = lib.kda_decode_multi_prologue if prologue else lib.kda_decode_multi
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(n_commit),
            _ptr(out), _ptr(gate), _ptr(norm_w), float(eps), B, K, H, dk, dv, float(scale),
            _IO[io], _stream(dev, stream))
    _check(lib, "kda_decode_multi_prologue" if prologue else "kda_decode_multi", st)
    return out


def chunk_workspace_size(B: int, T: int, H: int, dk: int, dv: int, dtype) -> int:
    """Workspace bytes kda_chunk_fwd needs for these sizes (0: none)."""
    return int(load_library().kda_chunk_fwd_workspace_size(int(B), int(T), int(H), int(dk),
                                                           int(dv), _IO[dtype]))


def chunk_launches(B: int, T: int, H: int, dk: int, dv: int, dtype) -> int:
    """Kernel launches one chunk_fwd call makes for these sizes."""
    return int(load_library().kda_chunk_fwd_launches(int(B), int(T), int(H), int(dk), int(dv),
                                                     _IO[dtype]))


def chunk_kernel_name(dk: int, dv: int, dtype) -> Optional[str]:
    """Name of the prefill kernel the library launches for these sizes and io dtype."""
    name = load_library().kda_chunk_fwd_kernel(int(dk), int(dv), _IO[dtype])
    return None if name is None else name.decode()


def gate_rmsnorm(x, gate, norm_w=None, *, eps: float = 1e-6, out=None, stream=None) -> torch.Tensor:
    """Head-wise RMSNorm x sigmoid(gate) over the last axis of ``x``."""
    lib = load_library()
    if x.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev, io = x.device, x.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    dv = x.shape[-1]
    rows = x.numel() // dv
    _need(x, "x", io, x.shape, dev)
    _need(gate, "gate", io, x.shape, dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32, (dv,), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", io, x.shape, dev)
    st = lib.kda_gate_rmsnorm(_ptr(x), _ptr(gate), _ptr(norm_w), _ptr(out), rows, dv, float(eps),
                              _IO[io], _stream(dev, stream))
    _check(lib, "kda_gate_rmsnorm", st)
    return out


def recurrent_bwd(q, k, v, g, beta, dout, s0=None, ds_final=None, *, scale: float = 1.0,
                  workspace=None, stream=None, ckpt=None):
    """Gradients of the token recurrence (kda_recurrent_bwd): q, k, v, dout [B, T, H, 128]
    (io dtype), g [B, T, H, 128] and beta [B, T, H] float32, s0 / ds_final [B, H, 128, 128]
    float32 or None.  ``ckpt``: the forward's states every 64 tokens [B, T // 64, H, 128, 128]
    float32 (kda_chunk_fwd_checkpoints with every = 64), which the chunkwise pass then uses
    instead of recomputing them (kda_recurrent_bwd_ckpt).  Returns (dq, dk, dv, dg, dbeta, ds0)."""
    lib = load_library()
    if q.device.type != "cuda":
        raise ValueError("kda ops need CUDA (HIP) tensors")
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = q.dtype
    if io not in _IO:
        raise TypeError(f"unsupported io dtype {io}")
    _need(q, "q", io, (B, T, H, dk), dev)
    _need(k, "k", io, (B, T, H, dk), dev)
    _need(v, "v", io, (B, T, H, dv), dev)
    _need(dout, "dout", io, (B, T, H, dv), dev)
    _need(g, "g", torch.float32, (B, T, H, dk), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    for t, n in ((s0, "s0"), (ds_final, "ds_final")):
        if t is not None:
            _need(t, n, torch.float32, (B, H, dk, dv), dev)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    ds0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    nws = lib.kda_recurrent_bwd_workspace_size(B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if ckpt is None:
        st = lib.kda_recurrent_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(dout), _ptr(ds_final),
            _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dbeta), _ptr(ds0), B, T, H, dk, dv,
            float(scale), _IO[io], _ptr(workspace), workspace.numel(), _stream(dev, stream))
        _check(lib, "kda_recurrent_bwd", st)
    else:
        _need(ckpt, "ckpt", torch.float32, (B, T // 64, H, dk, dv), dev)
        st = lib.kda_recurrent_bwd_ckpt(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(dout), _ptr(ds_final),
            _ptr(ckpt), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dbeta), _ptr(ds0),
            B, T, H, dk, dv, float(scale), _IO[io], _ptr(workspace), workspace.numel(),
            _stream(dev, stream))
        _check(lib, "kda_recurrent_bwd_ckpt", st)
    return dq, dk_, dv_, dg, dbeta, ds0
