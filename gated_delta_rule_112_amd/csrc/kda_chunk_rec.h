// Matrix-core chunked prefill (bfloat16 io, dk = dv = 128): the per-tile
// record that the tile kernel writes and the state kernel reads, and the small
// device helpers both kernels use.
//
// Chunkwise algebra ("Kimi K3: Engineering a 2.8 Trillion Parameter
// Frontier", section "Dimension 1": 16-token tiles, cumulative log-decay in
// (-80, 0) over a tile, a dense matrix product on every causal tile).  For a
// tile of 16 tokens (rows past the end of the sequence are zero inputs with
// g = beta = 0, which leave the state unchanged) with start state S (dk x dv,
// rows = key channels) and G = in-tile inclusive cumulative sum of g:
//   Qh = scale q e^G,  Kh = k e^G,  Kc = k e^-G,  Kb = k e^(G_15 - G)
//   A  = strict_lower(Diag(beta) Kh Kc^T)     Aqk = lower(Qh Kc^T)
//   T  = (I + A)^-1 Diag(beta)                W = T Kh
//   D  = T V - W S                            O = Qh S + Aqk D
//   S <- Diag(e^G_15) S + Kb^T D
// Everything but the last three lines is independent of the state, so the
// tile kernel computes it for all tiles in parallel and stores it as a record;
// the state kernel then walks the tiles of a head in order.
//
// Record layout.  Matrix operands are stored as the register image of one
// 64-lane wavefront (lane l = 16 g + c, c = l % 16, g = l / 16) so that the
// state kernel moves them with linear 16-byte copies and reads every operand
// with one conflict-free LDS access per lane:
//   Qh   [slab s < 4][lane][8] f16   lane (t, g): Qh[t][32 s + 8 g + e]
//   -W   [slab s < 4][lane][8] f16   lane (i, g): -W[i][32 s + 8 g + e]
//   Kb^T [block b < 8][lane][4] f16  lane (c, g): Kb[4 g + r][chan(b, c)]
//   en   [128] f32                   e^(G_15) per key channel
//   T    [lane][4] f16               lane (i, g): T[i][4 g + r]
//   Aqk  [lane][4] f16               lane (t, g): Aqk[t][4 g + r]
// where chan(b, p) = 32 (b / 2) + 8 (p / 4) + 4 (b % 2) + p % 4 is the key
// channel held in row p of state block b.  The state kernel keeps its state
// rows in that order: the 16x16 accumulator layout gives lane (c, g) rows
// 4 g + r of a block, so the rows of blocks 2s and 2s+1 in one lane are
// exactly channels 32 s + 8 g + 0..7, the k-operand values of that lane in a
// 16x16x32 product over slab s.  The state never moves between lanes.
#pragma once

#include "kda_device.h"

namespace kda {
namespace rec {

constexpr int kC = 16;       // tokens per tile
constexpr int kDK = 128;     // key head size
constexpr int kDV = 128;     // value head size
constexpr int kQh = 0;
constexpr int kW = 4096;
constexpr int kKb = 8192;
constexpr int kEn = 12288;
constexpr int kT = 12800;
constexpr int kAqk = 13312;
constexpr int kBytes = 13824;  // a multiple of 256

__host__ __device__ constexpr int chan(int b, int p) {
  return 32 * (b / 2) + 8 * (p / 4) + 4 * (b % 2) + p % 4;
}

}  // namespace rec

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16x16 matrix-core products, float32 accumulate.  Operand lane (x, g) holds
// row (A) or column (B) x and the k-values listed; the accumulator lane (c, g)
// holds D[4 g + r][c].
//   16x16x32 f16: k = 8 g + e;  16x16x16 f16/bf16: k = 4 g + e;  16x16x4 f32: k = g.
__device__ __forceinline__ f32x4 mma32h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16b(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4f(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
  return f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
}

// LDS writes of one wave made visible to the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cross-lane moves inside each 16-lane DPP row.
template <int CTRL, bool BOUND_ZERO>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, BOUND_ZERO));
}

// Inclusive prefix sum over the 16 lanes of each row (row_shr 1, 2, 4, 8).
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp<0x111, true>(x);
  x += dpp<0x112, true>(x);
  x += dpp<0x114, true>(x);
  x += dpp<0x118, true>(x);
  return x;
}

// Lane M of each row, in every lane of the row (row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(M >= 0 && M < 16, "row lane");
  return dpp<0x150 + M, false>(x);
}

}  // namespace kda
