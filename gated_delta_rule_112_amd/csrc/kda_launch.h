// Internal launch interface between the C ABI (kda_abi.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* s0;
  void* o;
  float* s_out;
  const void* gate;
  const float* norm_w;
  float eps;
  int64_t B, T, H;
  int dk, dv;
  float scale;
  bool io_bf16;
  void* workspace;  // device scratch of chunk_mfma_workspace() bytes (matrix-core path)
  void* stream;
  // Optional state checkpoints: ckpt [B, T / ckpt_every, H, dk, dv] receives the
  // state after every ckpt_every tokens (a multiple of 32).
  float* ckpt = nullptr;
  int64_t ckpt_every = 0;
  // Checkpoints in accumulator order instead of [dk, dv] (for the backward,
  // which reads them back as whole 16-byte runs per lane): 16-column group
  // w = columns 32 (w / 2) + 8 q + 4 (w % 2) + [0, 4), q < 4, at [w][kb][lane][4]
  // with lane (c, g) holding rows chan(kb, 4 g + r) of column index c.
  bool ckpt_frag = false;
  // Packed sequences: B sequences at rows cu[b] .. cu[b + 1] - 1 of total rows
  // (device array of B + 1 entries), T the longest; NULL for B x T.
  const int* cu = nullptr;
  int64_t total = 0;
  // Gates from logits: ga [rows, H, dk] in the io dtype holds a, and g = -5 sigmoid(a);
  // beta then holds the logit b of the write strength, beta = sigmoid(b).  NULL: g, beta given.
  const void* ga = nullptr;
  // Bytes of the workspace when it is smaller than chunk_mfma_workspace() (at
  // least chunk_mfma_workspace_min()): the matrix-core path then runs shorter
  // segments.  0: the default size.
  int64_t ws_bytes = 0;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  float* state;
  void* o;
  const void* gate;
  const float* norm_w;
  float eps;
  int64_t B, H;
  int dk, dv;
  float scale;
  bool io_bf16;
  void* stream;
  int64_t K = 0;                   // > 0: K tokens per sequence ([B, K, H, ..] inputs)
  const int* n_commit = nullptr;   // with K > 0: tokens to commit per sequence, or NULL = K
  const void* ga = nullptr;        // gates from logits, as in ChunkArgs
};

struct NormArgs {
  const void* x;
  const void* gate;
  const float* norm_w;
  void* y;
  int64_t rows;
  int dv;
  float eps;
  bool io_bf16;
  void* stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_chunk_valu(const ChunkArgs& a);
// Matrix-core prefill (per-pair records and state pass, segment by segment).
// Returns hipErrorNotSupported when it does not cover the shape.
hipError_t launch_chunk_mfma(const ChunkArgs& a);
bool chunk_mfma_supports(int dk, int dv, bool io_bf16);
size_t chunk_mfma_workspace(int64_t B, int64_t T, int64_t H);
// The smallest workspace the matrix-core path runs with (one pair per head per segment).
size_t chunk_mfma_workspace_min(int64_t B, int64_t H);
int64_t chunk_mfma_launches(int64_t B, int64_t T, int64_t H);
hipError_t launch_gate_rmsnorm(const NormArgs& a);

// Backward of the token recurrence (dk = dv = 128): gradients of a loss given
// dO for every token and dS_T for the final state.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* s0;   // NULL: zero initial state
  const void* dout;  // dO [B, T, H, dv]
  const float* ds_final;  // NULL: no final-state term
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* ds0;        // NULL: not written
  int64_t B, T, H;
  float scale;
  bool io_bf16;
  float* workspace;  // bwd_workspace_floats(B, T, H) floats
  void* stream;
  // The caller's forward states after every 64 tokens, [B, T / 64, H, dk, dv]
  // ([dk, dv] row-major), or NULL: recomputed (chunkwise path only).
  const float* ckpt = nullptr;
};
// Pieces of the reverse sweep: the state is checkpointed every kBwdPiece tokens.
constexpr int kBwdPiece = 64;
// Workgroups per (b, h) in the backward pass (each holds 128 / kBwdSplit value columns).
constexpr int kBwdSplit = 4;
int64_t bwd_workspace_floats(int64_t B, int64_t T, int64_t H);
hipError_t launch_recurrent_bwd(const BwdArgs& a);
// Chunkwise backward on the matrix cores (bfloat16 io, 16-byte aligned tensors).
int64_t bwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t H);
hipError_t launch_bwd_chunk(const BwdArgs& a);

}  // namespace kda
