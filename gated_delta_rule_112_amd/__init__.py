"""KDA (Kimi Delta Attention) layer core for AMD MI355X (gfx950).

Hand-written HIP kernels behind the C ABI in include/kda.h (libkda.so); this
package is the thin Python binding over it plus seeded input generators.
"""
from ._lib import (KDAError, KDA_BF16, KDA_F32, LIB_PATH, chunk_fwd,  # noqa: F401
                   chunk_fwd_checkpoints, chunk_fwd_noalloc, chunk_fwd_varlen, chunk_kernel_name, chunk_launches,
                   chunk_workspace_size, decode_multi, decode_step, gate_rmsnorm, load_library,
                   recurrent_bwd)

__all__ = ["chunk_fwd", "chunk_fwd_checkpoints", "chunk_fwd_noalloc", "chunk_fwd_varlen", "chunk_kernel_name",
           "chunk_launches", "chunk_workspace_size", "decode_multi", "decode_step",
           "gate_rmsnorm", "load_library", "recurrent_bwd", "KDAError", "LIB_PATH", "KDA_F32", "KDA_BF16"]
