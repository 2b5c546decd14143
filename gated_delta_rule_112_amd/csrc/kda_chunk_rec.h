// Matrix-core chunked prefill (bfloat16 io, dk = dv = 128): the record that
// the tile builder writes for every pair of 16-token tiles and the state pass
// reads, and the small device helpers both use.
//
// Chunkwise algebra ("Kimi K3: Engineering a 2.8 Trillion Parameter
// Frontier", section "Dimension 1": 16-token tiles, cumulative log-decay in
// (-80, 0) over a tile, a dense matrix product on every causal tile).  For a
// tile of 16 tokens (rows past the end of the sequence are zero inputs with
// g = beta = 0, which leave the state unchanged) with start state S (dk x dv,
// rows = key channels) and G = in-tile inclusive cumulative sum of g:
//   Qh = q e^G,  Kh = k e^G,  Kc = k e^-G,  Kb = k e^(G_15 - G),  E = e^G_15
//   A  = strict_lower(Diag(beta) Kh Kc^T)     Aqk = lower(Qh Kc^T)
//   T  = (I + A)^-1 Diag(beta)                W = T Kh
//   D  = T V - W S                            O = scale (Qh S + Aqk D)
//   S <- Diag(E) S + Kb^T D
// The state pass steps over two tiles a, b at once.  Substituting the state
// after tile a into tile b's lines gives, with every factor bounded by the
// tile-local quantities above (so float16 holds them):
//   D_a = T_a V_a - W_a S
//   D_b = T_b V_b - W_b' S + P D_a           W_b' = W_b Diag(E_a), P = -W_b Kb_a^T
//   O_a = Qh_a S + Aqk_a D_a
//   O_b = Qh_b' S + Q_ba D_a + Aqk_b D_b     Qh_b' = Qh_b Diag(E_a), Q_ba = Qh_b Kb_a^T
//   S  <- Diag(E_a E_b) S + Kb_a'^T D_a + Kb_b^T D_b      Kb_a' = Kb_a Diag(E_b)
// so the state is decayed, converted and updated once per 32 tokens, the
// update being one 32-deep product.  Everything but these lines is
// independent of the state: the tile builder computes it for all pairs in
// parallel and stores it as a record; the state pass walks the pairs of a
// head in order.
//
// Record layout.  Matrix operands are stored as the register image of one
// 64-lane wavefront (lane l = 16 g + c, c = l % 16, g = l / 16) so that the
// state pass moves them with linear 16-byte copies and reads every operand
// with one conflict-free LDS access per lane:
//   -W_a, -W_b'  [slab s < 4][lane][8] f16   lane (i, g): -W[i][32 s + 8 g + e]
//   Qh_a, Qh_b'  [slab s < 4][lane][8] f16   lane (t, g): Qh[t][32 s + 8 g + e]
//   Kb           [block b < 8][lane][8] f16  lane (c, g): Kb_a'[4 g + e][chan(b, c)] (e < 4),
//                                                         Kb_b[4 g + e - 4][chan(b, c)] (e >= 4)
//   en           [128] f32                   E_a E_b per key channel
//   T_a, Aqk_a   [lane][4] f16               lane (i, g): X[i][4 g + r]
//   [T_b | P], [Q_ba | Aqk_b]
//                [lane][8] f16               lane (i, g): X[i][4 g + e] (e < 4),
//                                                         Y[i][4 g + e - 4] (e >= 4)
//   norms        [2][16] f32, f32            1/|q_a|, 1/|q_b| per token, then the largest 1/|k|
//                                            of the pair, when q and k are
//                                            normalised in the kernels (else unused; the key
//                                            norms are then folded into T, W and P, whose rows
//                                            carry 1/|k|, so that D' = Diag(1/|k|) D is what the
//                                            state pass forms)
// (the [T_b | P] and [Q_ba | Aqk_b] blocks are the A and B operands of 32-deep products:
// D_b = [T_b | P] [V_b ; D_a] and O_b^T = ... + [D_a ; D_b]^T [Q_ba | Aqk_b]^T)
// where chan(b, p) = 32 (b / 2) + 8 (p / 4) + 4 (b % 2) + p % 4 is the key
// channel held in row p of state block b.  The state pass keeps its state
// rows in that order: the 16x16 accumulator layout gives lane (c, g) rows
// 4 g + r of a block, so the rows of blocks 2s and 2s+1 in one lane are
// exactly channels 32 s + 8 g + 0..7, the k-operand values of that lane in a
// 16x16x32 product over slab s.  The state never moves between lanes.
#pragma once

#include "kda_device.h"

namespace kda {
namespace rec {

constexpr int kC = 16;       // tokens per tile
constexpr int kP = 32;       // tokens per pair (one state step)
constexpr int kDK = 128;     // key head size
constexpr int kDV = 128;     // value head size
constexpr int kWa = 0;
constexpr int kWb = 4096;
constexpr int kQa = 8192;
constexpr int kQb = 12288;
constexpr int kKb = 16384;
constexpr int kEn = 24576;
constexpr int kTa = 25088;
constexpr int kAa = 25600;
constexpr int kTbP = 26112;
constexpr int kQbaAb = 27136;
constexpr int kNorm = 28160;   // with q and k normalised in the kernels: 1/|q| per token, max 1/|k|
constexpr int kBytes = 28416;  // record stride, a multiple of 256

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

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits
// for every global load and store the wavefront has in flight (vmcnt(0));
// this one leaves them in flight, so loads issued ahead stay ahead.  Data
// that direct-to-LDS loads bring in is covered by the issuing wavefront's own
// vmcnt wait before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest of x over the 64 lanes (x >= 0), in every lane: a max-scan over
// each 16-lane DPP row, then the four row maxima, compared as integers (the
// bit patterns of non-negative floats order like their values).
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, dpp<0x111, true>(x));
  x = fmaxf(x, dpp<0x112, true>(x));
  x = fmaxf(x, dpp<0x114, true>(x));
  x = fmaxf(x, dpp<0x118, true>(x));
  const unsigned b = __builtin_bit_cast(unsigned, x);
  unsigned m = (unsigned)__builtin_amdgcn_readlane((int)b, 15);
  const unsigned m1 = (unsigned)__builtin_amdgcn_readlane((int)b, 31);
  const unsigned m2 = (unsigned)__builtin_amdgcn_readlane((int)b, 47);
  const unsigned m3 = (unsigned)__builtin_amdgcn_readlane((int)b, 63);
  m = m1 > m ? m1 : m;
  m = m2 > m ? m2 : m;
  m = m3 > m ? m3 : m;
  return __builtin_bit_cast(float, m);
}

// Unbiased binary exponent of a non-negative float (x in [2^e, 2^(e+1))),
// or kNoExp for zero.  Denormals read as -127; inf and NaN as 128.
constexpr int kNoExp = -1000;
__device__ __forceinline__ int exp_of(float x) {
  const int b = (int)(__builtin_bit_cast(unsigned, x) >> 23);
  return x == 0.f ? kNoExp : b - 127;
}

// 2^e as a float, e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) {
  return __builtin_bit_cast(float, (unsigned)(e + 127) << 23);
}

// Power-of-two scale of a state wavefront's float16 operands.  The wavefront
// holds sigma S (sigma = 2^sh) and forms sigma V (or the adjoint quantities
// of the backward pass); em is the exponent of the largest
// magnitude among them.  While em stays in [kLoExp, kHiExp] the scale is
// kept; otherwise the returned shift d moves em to kTargetExp (the caller
// multiplies its accumulators by 2^d).  sh stays within [-120, 120].
constexpr int kLoExp = 2, kHiExp = 10, kTargetExp = 9;
__device__ __forceinline__ int scale_shift(int em, int sh) {
  if (em == kNoExp || (em >= kLoExp && em <= kHiExp)) return 0;
  int n = sh + (kTargetExp - em);
  n = n < -120 ? -120 : (n > 120 ? 120 : n);
  return n - sh;
}

}  // namespace kda
