"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function declared in include/kda.h, and
reject bad arguments on the host before any HIP call.  Pointers used here are
fake addresses: every call below fails validation, so nothing is launched and
no pointer is dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, SHAPE, DIM, DTYPE, ALIGN, ALIAS, ARG, LAUNCH, WORKSPACE, INPUT_RANGE = range(11)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_112_amd import load_library
    return load_library()


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ["kda_chunk_fwd", "kda_chunk_fwd_checkpoints", "kda_chunk_fwd_varlen",
              "kda_chunk_fwd_varlen_prologue", "kda_chunk_fwd_workspace_size",
              "kda_chunk_fwd_launches",
              "kda_decode_step", "kda_decode_multi", "kda_chunk_fwd_prologue",
              "kda_decode_step_prologue", "kda_decode_multi_prologue",
              "kda_gate_rmsnorm", "kda_status_string", "kda_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"libkda.so lacks {missing}"


def test_status_strings(lib):
    for s in range(0, 11):
        assert lib.kda_status_string(s)
        assert b"UNKNOWN" not in lib.kda_status_string(s)
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(INPUT_RANGE).startswith(b"KDA_ERR_INPUT_RANGE")
    assert b"UNKNOWN" in lib.kda_status_string(99)
    assert lib.kda_version() >= 100


# Fake, distinct, 16-byte aligned device addresses far apart from each other.
BASE = 1 << 40


def P(i, off=0):
    return ctypes.c_void_p(BASE + (i << 34) + off)


def chunk(lib, *, q=1, k=2, v=3, g=4, beta=5, s0=None, o=6, s_out=7, gate=None, w=None,
          eps=1e-6, B=1, T=16, H=1, dk=16, dv=16, scale=1.0, io=1, ws=None, ws_bytes=0,
          override=None):
    ptrs = dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0, o=o, s_out=s_out, gate=gate, w=w, ws=ws)
    args = {n: (None if x is None else P(x)) for n, x in ptrs.items()}
    if override:
        args.update(override)
    return lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["s0"],
                             args["o"], args["s_out"], args["gate"], args["w"], eps, B, T, H, dk,
                             dv, scale, io, args["ws"], ws_bytes, None)


def test_chunk_null_pointers(lib):
    for name in ["q", "k", "v", "g", "beta"]:
        assert chunk(lib, dk=48, **{name: None}) == NULLP
    assert chunk(lib, o=None, s_out=None) == NULLP


def test_chunk_shapes_dims_dtypes(lib):
    assert chunk(lib, dk=48) == DIM
    assert chunk(lib, dv=256) == DIM
    assert chunk(lib, dk=48, io=2) == DTYPE  # dtype checked before dims
    assert chunk(lib, io=7, dk=16) == DTYPE
    assert chunk(lib, B=0) == SHAPE
    assert chunk(lib, T=0) == SHAPE
    assert chunk(lib, H=-1) == SHAPE
    assert chunk(lib, B=1 << 30, T=1 << 30, H=1 << 10) == SHAPE


def test_chunk_scalars(lib):
    assert chunk(lib, eps=-1.0) == ARG
    assert chunk(lib, eps=float("nan")) == ARG
    assert chunk(lib, scale=float("inf")) == ARG


def test_chunk_alignment(lib):
    assert chunk(lib, override={"q": P(1, 2)}) == ALIGN
    assert chunk(lib, override={"o": P(6, 8)}) == ALIGN
    assert chunk(lib, override={"s0": P(9, 2)}) == ALIGN      # states need 4 bytes
    assert chunk(lib, override={"beta": P(5, 2)}) == ALIGN
    assert chunk(lib, override={"g": P(4, 4)}) == ALIGN       # g tiles move in 16 bytes


def test_chunk_aliasing(lib):
    assert chunk(lib, o=1) == ALIAS                 # o == q
    assert chunk(lib, s_out=2) == ALIAS             # s_out == k
    assert chunk(lib, o=7, s_out=7) == ALIAS        # o == s_out
    assert chunk(lib, gate=8, o=8) == ALIAS
    # s_out == s0 (in place) is allowed (exercised on the GPU); partial overlap is not.
    assert chunk(lib, s0=9, override={"s_out": P(9, 16)}) == ALIAS


def test_chunk_workspace(lib):
    """The matrix-core path (bf16, dk = dv = 128) needs a workspace: missing, too
    small, misaligned or overlapping workspaces are rejected before any launch."""
    size = lib.kda_chunk_fwd_workspace_size
    need = size(1, 4096, 32, 128, 128, 1)
    assert need >= 2 * 28160 * 32 + 32 * 128 * 128 * 4  # two records of one pair of every head
    assert size(1, 4096, 32, 16, 16, 1) == 0          # vector-ALU path: none
    assert size(1, 4096, 32, 128, 128, 0) == 0        # float32 io: vector-ALU path
    assert size(0, 4096, 32, 128, 128, 1) == 0        # invalid sizes
    assert size(1, 4096, 32, 48, 128, 1) == 0
    # two segments of records (at most 256 MiB each) however long the sequence is
    assert size(1, 1 << 20, 96, 128, 128, 1) < (600 << 20)
    assert size(1, 1 << 20, 96, 128, 128, 1) == size(1, 1 << 22, 96, 128, 128, 1)
    kw = dict(B=1, T=4096, H=32, dk=128, dv=128, io=1)
    assert chunk(lib, **kw) == WORKSPACE                             # NULL
    assert chunk(lib, ws=10, ws_bytes=need - 1, **kw) == WORKSPACE   # too small
    assert chunk(lib, ws_bytes=need, override={"ws": P(10, 128)}, **kw) == WORKSPACE
    assert chunk(lib, ws=1, ws_bytes=need, **kw) == ALIAS            # overlaps q
    assert chunk(lib, ws=10, ws_bytes=need, dk=48, B=1, T=16, H=1) == DIM
    launches = lib.kda_chunk_fwd_launches
    launches.restype = ctypes.c_int64
    assert launches(1, 4096, 32, 16, 16, 1) == 1          # vector-ALU path: one kernel
    assert launches(1, 16, 1, 128, 128, 1) == 2           # one segment + its records
    assert launches(1, 1 << 20, 96, 128, 128, 1) > 2
    assert launches(1, 16, 1, 48, 128, 1) == 0


def test_launch_groups(lib):
    """Large batches run in groups of sequences whose state workgroups take
    about 3/8 of the compute units, every segment of every group in one launch
    pipeline: the launch count is one plus the groups' segments, and the
    workspace is sized for one group (host logic; the compute-unit count falls
    back to 256 without a device)."""
    launches = lib.kda_chunk_fwd_launches
    launches.restype = ctypes.c_int64
    ws = lib.kda_chunk_fwd_workspace_size
    ws.restype = ctypes.c_size_t
    one = launches(1, 4096, 96, 128, 128, 1)     # one sequence: one group
    assert one >= 2
    assert launches(16, 4096, 96, 128, 128, 1) == 1 + 16 * (one - 1)
    assert ws(16, 4096, 96, 128, 128, 1) == ws(1, 4096, 96, 128, 128, 1)
    # 32 heads: three sequences per group (96 state workgroups)
    three = launches(3, 4096, 32, 128, 128, 1)
    assert launches(9, 4096, 32, 128, 128, 1) == 1 + 3 * (three - 1)
    assert ws(9, 4096, 32, 128, 128, 1) == ws(3, 4096, 32, 128, 128, 1)


def test_chunk_checkpoints_validation(lib):
    f = lib.kda_chunk_fwd_checkpoints

    def call(ckpt=P(11), every=64, ws=None):
        # vector-path sizes (dk = dv = 16): no workspace needed
        return f(P(1), P(2), P(3), P(4), P(5), None, P(6), P(7), None, None, 1e-6,
                 2, 200, 3, 16, 16, 1.0, 0, ws, 0, ckpt, every, None)

    assert call(ckpt=None) == NULLP
    assert call(every=0) == SHAPE
    assert call(every=48) == SHAPE
    assert call(every=-32) == SHAPE
    assert call(ckpt=P(11, 2)) == ALIGN
    assert call(ckpt=P(1)) == ALIAS          # overlaps q
    assert call(ckpt=P(7)) == ALIAS          # overlaps s_out


def test_chunk_varlen_validation(lib):
    f = lib.kda_chunk_fwd_varlen

    def call(cu=P(12), N=3, total=200, max_len=100, o=6, ckpt=None, every=0):
        # vector-path sizes (dk = dv = 16): no workspace needed
        return f(P(1), P(2), P(3), P(4), P(5), cu, N, total, max_len, None, P(o), P(7), None,
                 None, 1e-6, 3, 16, 16, 1.0, 0, None, 0, ckpt, every, None)

    assert call(cu=None) == NULLP
    assert call(N=0) == SHAPE
    assert call(total=0) == SHAPE
    assert call(max_len=0) == SHAPE
    assert call(cu=P(12, 2)) == ALIGN
    assert call(cu=P(6)) == ALIAS             # cu_seqlens inside o
    assert call(ckpt=P(11), every=40) == SHAPE
    assert call(ckpt=P(1), every=32) == ALIAS   # checkpoints overlap q


def test_chunk_varlen_prologue_validation(lib):
    """The packed entry point from raw projections: a NULL logit array is
    rejected, then kda_chunk_fwd_varlen's checks apply."""
    f = lib.kda_chunk_fwd_varlen_prologue

    def call(a=P(4), cu=P(12), N=3, o=6, ckpt=None, every=0):
        return f(P(1), P(2), P(3), a, P(5), cu, N, 200, 100, None, P(o), P(7), None, None,
                 1e-6, 3, 16, 16, 1.0, 0, None, 0, ckpt, every, None)

    assert call(a=None) == NULLP
    assert call(cu=None) == NULLP
    assert call(N=0) == SHAPE
    assert call(a=P(4, 8)) == ALIGN
    assert call(o=4) == ALIAS                 # o overlaps the logits
    assert call(ckpt=P(11), every=40) == SHAPE


def test_prologue_validation(lib):
    """The prologue entry points: a NULL logit array is rejected, the rest is
    kda_chunk_fwd's and kda_decode_step's validation."""
    f = lib.kda_chunk_fwd_prologue
    args = [P(1), P(2), P(3), P(4), P(5), None, P(6), P(7), None, None, 1e-6, 2, 64, 3, 16, 16,
            1.0, 0, None, 0, None]
    assert f(*args[:3], None, *args[4:]) == NULLP
    assert f(*args[:4], None, *args[5:]) == NULLP
    assert f(*args[:3], P(4, 8), *args[4:]) == ALIGN
    assert f(*args[:3], P(6), *args[4:]) == ALIAS  # o overlaps the logits
    d = lib.kda_decode_step_prologue
    dargs = [P(1), P(2), P(3), P(4), P(5), P(6), P(7), None, None, 1e-6, 1, 1, 16, 16, 1.0, 1,
             None]
    assert d(*dargs[:3], None, *dargs[4:]) == NULLP
    assert d(*dargs[:3], P(7), *dargs[4:]) == ALIAS  # logits == o


def decode(lib, *, q=1, k=2, v=3, g=4, beta=5, state=6, o=7, gate=None, w=None, eps=1e-6,
           B=1, H=1, dk=16, dv=16, scale=1.0, io=1, override=None):
    ptrs = dict(q=q, k=k, v=v, g=g, beta=beta, state=state, o=o, gate=gate, w=w)
    args = {n: (None if x is None else P(x)) for n, x in ptrs.items()}
    if override:
        args.update(override)
    return lib.kda_decode_step(args["q"], args["k"], args["v"], args["g"], args["beta"],
                               args["state"], args["o"], args["gate"], args["w"], eps, B, H, dk,
                               dv, scale, io, None)


def test_decode_validation(lib):
    for name in ["q", "k", "v", "g", "beta", "state", "o"]:
        assert decode(lib, **{name: None}) == NULLP
    assert decode(lib, dk=100) == DIM
    assert decode(lib, io=3) == DTYPE
    assert decode(lib, B=0) == SHAPE
    assert decode(lib, eps=-0.5) == ARG
    assert decode(lib, override={"state": P(6, 4)}) == ALIGN
    assert decode(lib, override={"q": P(1, 1)}) == ALIGN      # bf16 needs 2 bytes
    assert decode(lib, o=6) == ALIAS       # o == state
    assert decode(lib, state=1) == ALIAS   # state == q


def multi(lib, *, q=1, k=2, v=3, g=4, beta=5, state=6, n=8, o=7, gate=None, w=None, eps=1e-6,
          B=2, K=4, H=3, dk=16, dv=16, scale=1.0, io=1, override=None):
    ptrs = dict(q=q, k=k, v=v, g=g, beta=beta, state=state, n=n, o=o, gate=gate, w=w)
    args = {n_: (None if x is None else P(x)) for n_, x in ptrs.items()}
    if override:
        args.update(override)
    return lib.kda_decode_multi(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                args["state"], args["n"], args["o"], args["gate"], args["w"],
                                eps, B, K, H, dk, dv, scale, io, None)


def test_decode_multi_validation(lib):
    for name in ["q", "k", "v", "g", "beta", "state"]:
        assert multi(lib, **{name: None}) == NULLP
    assert multi(lib, dk=100) == DIM
    assert multi(lib, io=3) == DTYPE
    assert multi(lib, K=0) == SHAPE
    assert multi(lib, B=0) == SHAPE
    assert multi(lib, scale=float("inf")) == ARG
    assert multi(lib, override={"state": P(6, 8)}) == ALIGN
    assert multi(lib, override={"n": P(8, 2)}) == ALIGN          # int32 counts
    assert multi(lib, o=6) == ALIAS        # o == state
    assert multi(lib, state=8) == ALIAS    # state == n_commit
    assert multi(lib, n=7) == ALIAS        # n_commit inside o


def test_gate_rmsnorm_validation(lib):
    f = lib.kda_gate_rmsnorm
    assert f(None, P(2), None, P(3), 4, 16, 1e-6, 1, None) == NULLP
    assert f(P(1), P(2), None, P(3), 0, 16, 1e-6, 1, None) == SHAPE
    assert f(P(1), P(2), None, P(3), 4, 24, 1e-6, 1, None) == DIM
    assert f(P(1), P(2), None, P(3), 4, 16, -1.0, 1, None) == ARG
    assert f(P(1), P(2), None, P(2), 4, 16, 1e-6, 1, None) == ALIAS       # y == gate
    assert f(P(1), P(2), None, P(1, 16), 4, 16, 1e-6, 1, None) == ALIAS  # partial y/x overlap
    assert f(P(1, 4), P(2), None, P(3), 4, 16, 1e-6, 1, None) == ALIGN


def test_chunk_kernel_query(lib):
    lib.kda_chunk_fwd_kernel.restype = ctypes.c_char_p
    assert lib.kda_chunk_fwd_kernel(16, 16, 0) in (b"kda_chunk_valu", b"kda_chunk_mfma")
    assert lib.kda_chunk_fwd_kernel(48, 16, 0) is None
    assert lib.kda_chunk_fwd_kernel(16, 16, 5) is None


def test_recurrent_bwd_validation(lib):
    """kda_recurrent_bwd: required pointers, dk = dv = 128 only, workspace size,
    alignment of the float4 state arguments, and no output over an input or
    another output; every rejection happens before any launch."""
    f = lib.kda_recurrent_bwd
    B, T, H = 2, 70, 2
    need = lib.kda_recurrent_bwd_workspace_size(B, T, H, 128, 128)
    # ceil(70 / 64) checkpoints + 64 states per head, then 4 column parts of dq, dk, dg, dbeta
    assert need == (B * H * (2 + 64) * 128 * 128 + 4 * B * T * H * (3 * 128 + 1)) * 4
    assert lib.kda_recurrent_bwd_workspace_size(B, T, H, 64, 64) == 0
    # beyond 2^40 token-heads the size would leave int64: reported as unsupported
    assert lib.kda_recurrent_bwd_workspace_size(1 << 20, 1 << 20, 2, 128, 128) == 0
    # the chunkwise pass needs more than the token-serial one at long T (records and
    # products per tile): the reported size covers the larger
    nl = lib.kda_recurrent_bwd_workspace_size(2, 4096, 32, 128, 128)
    assert nl >= 2 * 32 * (4096 // 16) * (24576 + 2048 + 6784 * 4)

    def call(q=1, dq=9, ds0=14, s0=6, dk=128, ws=15, nws=None, io=0):
        a = {i: P(i) for i in range(1, 16)}
        a[1], a[9], a[14], a[6], a[15] = (None if q is None else P(q)), P(dq), \
            (None if ds0 is None else P(ds0)), (None if s0 is None else P(s0)), \
            (None if ws is None else (P(ws) if isinstance(ws, int) else ws))
        return f(a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], a[10], a[11], a[12],
                 a[13], a[14], B, T, H, dk, dk, 1.0, io, a[15], need if nws is None else nws, None)

    assert call(q=None) == NULLP
    assert call(dk=64) == DIM
    assert call(dk=100) == DIM
    assert call(io=7) == DTYPE
    assert call(ws=None) == WORKSPACE
    assert call(nws=need - 1) == WORKSPACE
    assert call(ws=P(15, 4)) == ALIGN
    assert call(s0=None, ds0=None, dq=1) == ALIAS     # dq over q
    assert call(ds0=9) == ALIAS                        # ds0 over dq


def test_recurrent_bwd_ckpt_validation(lib):
    """kda_recurrent_bwd_ckpt: the checkpoints are required, bfloat16 and 16-byte
    aligned token tensors only (the chunkwise pass), and they may not lie under
    an output; every rejection happens before any launch."""
    f = lib.kda_recurrent_bwd_ckpt
    B, T, H = 1, 256, 2
    need = lib.kda_recurrent_bwd_workspace_size(B, T, H, 128, 128)

    def call(ck=16, io=1, q=P(1), dq=9, dg=P(12)):
        a = {i: P(i) for i in range(1, 17)}
        return f(q, a[2], a[3], a[4], a[5], a[6], a[7], a[8], None if ck is None else P(ck),
                 P(dq), a[10], a[11], dg, a[13], a[14], B, T, H, 128, 128, 1.0, io, a[15],
                 need, None)

    assert call(ck=None) == NULLP
    assert call(io=0) == DTYPE                         # float32: no chunkwise pass
    assert call(q=P(1, 8)) == ALIGN                    # 8 bytes off: not the chunkwise layout
    assert call(dg=P(12, 4)) == ALIGN                  # dg float32-aligned, not 16-byte
    assert call(ck=9) == ALIAS                         # checkpoints under dq
