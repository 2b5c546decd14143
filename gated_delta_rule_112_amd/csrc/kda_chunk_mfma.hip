// KDA chunked prefill on the gfx950 matrix cores (bfloat16 io, dk = dv = 128).
//
// Same chunkwise algebra as the vector kernel ("Kimi K3: Engineering a 2.8
// Trillion Parameter Frontier", section "Dimension 1": 16-token tiles whose
// cumulative log-decay stays in (-80, 0), every causal tile a dense matrix
// product).  For one tile of n <= 16 tokens with start state S (dk x dv, rows
// are key channels) and G = in-tile inclusive cumsum of g:
//   Qh = scale q e^G,  Kh = k e^G,  Kc = k e^-G,  Kb = k e^(G_n - G)
//   A  = strict_lower(Diag(beta) Kh Kc^T)     Aqk = lower(Qh Kc^T)
//   T  = (I + A)^-1 Diag(beta)                W = T Kh,   U = T V
//   D  = U - W S                              O = Qh S + Aqk D
//   S <- Diag(e^(G_n)) S + Kb^T D
// A partial last tile is padded with g = beta = 0 and q = k = v = 0 tokens,
// which leave the state unchanged.
//
// Only D, O and the state update depend on the running state; everything
// else about a tile can be computed ahead of it.  One workgroup owns one
// (b, h) and DVW of its dv state columns (all of them, or half when two
// workgroups share a head), with two kinds of waves:
//   state waves (DVW/16): each keeps 16 state columns in matrix-core
//       accumulators for the whole sequence and runs the state-dependent
//       products of tile it-3 in iteration it;
//   builder waves (4, one 32-channel key slab each): in iteration it they
//       build the rescaled operands of tile it (cumulative log-decay,
//       exponentials), form the partial intra-tile products of tile it over
//       their slab, and two blocks of W = T Kh for tile it-2; builder 3 also
//       sums the partials of tile it-1 and solves the 16x16 unit-lower-
//       triangular system for T by forward substitution in float32.
// Each wave kind runs its own loop; every iteration is two phases separated
// by workgroup barriers (each wave executes exactly the same barriers), and
// the inputs are prefetched into registers two iterations before they are
// staged in LDS.  HBM latency, the operand arithmetic and the solve therefore
// overlap the serial state chain.  The output tile of x is normalised/gated and
// written one iteration after its state step, once the head's row sums of
// squares are complete.
//
// Precision.  Outputs of this layer have a max/RMS ratio of 12-16, so a
// single bfloat16 rounding on the path from an input to an output already
// costs up to ~3% of the output RMS at the largest elements.  Operands that
// multiply the state or the delta are therefore float16 (11-bit significand);
// the product that involves e^-G (up to e^80, outside float16 range) and
// feeds the output directly, Qh Kc^T, uses bfloat16 split into high and low
// parts (16 significand bits).  Accumulation is float32 throughout and the
// state never leaves float32 accumulators.  float16 operands require the
// state, the values and the delta to stay below 65504 in magnitude.
//
// The state is contracted over its rows (dk) with the 16x16x32 instruction.
// Its accumulator layout gives lane (c, g) the rows 16b + 4g + r (r = 0..3);
// the 32-row slab s of the contraction is fed with the lane's own rows of
// blocks 2s and 2s+1, and the left operand (W or Qh) is read with the same
// permutation of its columns, so the state is never shuffled between lanes.
#include <stdlib.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kC = 16;         // tokens per tile
constexpr int kDK = 128;       // key head size served by this kernel
// LDS row paddings, chosen so that the matrix-operand reads and writes of a
// wave spread over all banks: 2-byte [token][channel] tiles, float32
// [token][channel] tiles, [.][16] 2-byte tiles and [16][16] float32 tiles.
constexpr int kRow = kDK + 8;   // read and written 16 bytes at a time
constexpr int kRowH = kDK + 4;  // read and written 8 bytes at a time
constexpr int kRowF = kDK + 4;
constexpr int kR16 = 20;
constexpr int kR16F = 20;
constexpr int kNB = 4;         // builder waves, one 32-channel key slab each
constexpr int kLead = 2;       // register prefetch slots (iterations of lead)
constexpr int kLagS = 3;       // the state chain runs tile it - kLagS in iteration it

template <int DVW>
struct Cfg {
  static constexpr int NS = DVW / 16;  // state waves
  static constexpr int NT = 64 * (NS + kNB);
};

__device__ __forceinline__ f32x4 mma32h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32b(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
  return f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS writes of one wave made visible to the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
  int v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));
  return x;
}

// Sum over the 16 lanes of each DPP row, result in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  int v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x122, 0xf, 0xf, false));
  v = __builtin_bit_cast(int, x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x121, 0xf, 0xf, false));
  return x;
}

// Value of lane 15 of each DPP row, in every lane of the row.
__device__ __forceinline__ float row_last16(float x) {
  const int v = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x15F, 0xf, 0xf, false));
}

template <int DVW>
struct Smem {
  static constexpr int NS = Cfg<DVW>::NS;
  // Raw input tiles (rows past the end of the sequence are zero).
  bf16_t rq[kC][kRow];
  bf16_t rk[kC][kRow];
  float rg[kC][kRowF];
  float rb[kC];
  bf16_t rv[2][kC][DVW + 4];     // tile x % 2
  bf16_t rgate[2][kC][DVW + 4];  // tile x % 2
  // Builder outputs consumed by the partial intra-tile products (same iteration).
  bf16_t qhh[kC][kRow];   // Qh, bfloat16 high part
  bf16_t qhl[kC][kRow];   //     bfloat16 low part
  bf16_t khb[kC][kRow];   // Kh, bfloat16
  bf16_t kch[kC][kRow];   // Kc high part
  bf16_t kcl[kC][kRow];   // Kc low part
  // Builder outputs consumed later by W and by the state waves.
  f16 khT[3][kDK][kR16];  // Kh^T, float16        (tile x % 3)
  f16 qh16[4][kC][kRowH]; // Qh, float16          (tile x % 4)
  f16 kbT[4][kDK][kR16];  // Kb^T, float16        (tile x % 4)
  float en[4][kDK];       // e^(G_n)              (tile x % 4)
  float betab[2][kC];     // beta                 (tile x % 2)
  // Partial products over key slab p, transposed: part[p][j][i] = (X Kc^T)[i][j].
  float partA[2][kNB][kC][kR16F];  // (tile x % 2)
  float partQ[2][kNB][kC][kR16F];
  float aT[kC][kR16F];    // A^T, float32, input of the forward substitution
  f16 t16[2][kC][kR16];   // T                    (tile x % 2)
  f16 aqk16[2][kC][kR16]; // Aqk                  (tile x % 2)
  f16 wneg[2][kC][kRowH]; // -W                   (tile x % 2)
  float rsT[NS][kC];      // row sums of squares of the output, per state wave
  bf16_t otile[kC][DVW + 4];  // finished output tile
};

template <int DV, int DVW, bool GATE>
__global__ void __launch_bounds__(Cfg<DVW>::NT, 1)
kda_chunk_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ beta, const float* __restrict__ s0,
                      bf16_t* __restrict__ o, float* __restrict__ s_out,
                      const bf16_t* __restrict__ gate, const float* __restrict__ norm_w,
                      float eps, int64_t T, int64_t H, int64_t BH, float scale) {
  using CF = Cfg<DVW>;
  constexpr int NS = CF::NS;
  constexpr int NSPLIT = DV / DVW;
  constexpr int NKB = kDK / 16;   // 16-row accumulator blocks of the state
  constexpr int NKS = kDK / 32;   // 32-row contraction slabs
  static_assert(DVW % 64 == 0 && DV % DVW == 0, "bad column split");
  static_assert(!GATE || NSPLIT == 1, "the gated RMSNorm needs a head's full dv row");
  static_assert(kNB * 32 == kDK && 2 * kNB == NKB, "builder slabs must cover the key channels");

  __shared__ Smem<DVW> sm;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int lc = lane % 16;  // column (or row) index inside a 16x16 tile
  const int lg = lane / 16;  // lane group: 4 rows, or 4 / 8 contraction values

  // Workgroups are dealt round-robin over the 8 XCDs; keep the NSPLIT
  // workgroups of one head on the same XCD so its q/k/g tiles are shared in L2.
  int64_t wg = blockIdx.x;
  const int64_t total = BH * NSPLIT;
  if (NSPLIT > 1 && total % 8 == 0) wg = (wg % 8) * (total / 8) + wg / 8;
  const int64_t bh = wg / NSPLIT;
  const int col0 = (int)(wg % NSPLIT) * DVW;  // first dv column of this workgroup
  const int64_t b = bh / H, h = bh % H;
  const int64_t nchunks = (T + kC - 1) / kC;
  const int64_t niter = nchunks + kLagS + 1;
  const bool write_o = (o != nullptr);

  // Element offset of token t (clamped into the sequence) of this head in a
  // [B, T, H, *] tensor, per channel.  Loads are issued for every tile slot,
  // in range or not, so every wave has the same loads in flight; rows outside
  // the sequence are zeroed when staged.
  auto tokoff = [&](int64_t t) {
    t = t < 0 ? 0 : (t >= T ? T - 1 : t);
    return (b * T + t) * H + h;
  };

  if (wave < NS) {
    // ============================================================ state waves
    const int wcol = wave * 16;  // first column of this wave within DVW
    // State lane tid moves one 16-byte unit of the v (or gate) tile.
    const int s_which = tid / (2 * DVW);
    const int s_row = (tid % (2 * DVW)) / (DVW / 8);
    const int s_c8 = ((tid % (2 * DVW)) % (DVW / 8)) * 8;
    const bf16_t* s_src = (GATE && s_which == 1) ? gate : v;
    auto load_s = [&](int64_t x) {
      return *(const bf16x8*)(s_src + tokoff(x * kC + s_row) * DV + col0 + s_c8);
    };
    // Rows past the end of the sequence hold a clamped copy of the last row:
    // finite values that meet zero columns of T (beta = 0) or are never stored.
    auto stage_s = [&](int64_t x, bf16x8 r) {
      bf16_t* dst = (s_which == 0) ? &sm.rv[x & 1][s_row][s_c8] : &sm.rgate[x & 1][s_row][s_c8];
      *(bf16x4*)dst = bf16x4{r[0], r[1], r[2], r[3]};
      *(bf16x4*)(dst + 4) = bf16x4{r[4], r[5], r[6], r[7]};
    };

    f32x4 S[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x4 x = zero4();
      if (s0 != nullptr) {
        const float* p = s0 + (bh * kDK + 16 * kb + 4 * lg) * DV + col0 + wcol + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = p[(int64_t)r * DV];
      }
      S[kb] = x;
    }
    const float wn = (GATE && norm_w != nullptr) ? norm_w[col0 + wcol + lc] : 1.f;
    f32x4 O = zero4(), Oprev = zero4();
    f16x4 d16 = {};
    // Slot u is staged in iteration i0 + u as tile it - 2 (loaded kLead iterations before).
    bf16x8 ps[kLead];
#pragma unroll
    for (int u = 0; u < kLead; ++u) ps[u] = load_s(u - 2);
    __syncthreads();

    for (int64_t i0 = 0; i0 < niter; i0 += kLead) {
#pragma unroll
      for (int u = 0; u < kLead; ++u) {
        const int64_t it = i0 + u;
        if (it >= niter) break;
        const int64_t xs = it - kLagS;      // tile in the state chain
        const int64_t xf = it - kLagS - 1;  // tile whose output is finished
        const bool run_s = xs >= 0 && xs < nchunks;
        const bool run_f = write_o && xf >= 0 && xf < nchunks;

        // ---- phase A: finish tile xf; D and O of tile xs
        if (run_f) {
          float y[4] = {Oprev[0], Oprev[1], Oprev[2], Oprev[3]};
          if (GATE) {
            f32x4 ss = zero4();
#pragma unroll
            for (int w = 0; w < NS; ++w) ss += *(const f32x4*)&sm.rsT[w][4 * lg];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float inv = rsqrtf(ss[r] * (1.f / (float)DV) + eps);
              const float gt = (float)sm.rgate[xf & 1][4 * lg + r][wcol + lc];
              const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-gt));
              y[r] = y[r] * inv * wn * sg;
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.otile[4 * lg + r][wcol + lc] = (bf16_t)y[r];
        }
        if (run_s) {
          const int xs4 = (int)(xs & 3), xs2 = (int)(xs & 1);
          // The state as float16 right operands, slab s = rows of blocks 2s, 2s+1.
          f16x8 sop[NKS];
#pragma unroll
          for (int s = 0; s < NKS; ++s) sop[s] = cat8(to_h4(S[2 * s]), to_h4(S[2 * s + 1]));
          // U = T V
          const f16x4 ta = *(const f16x4*)&sm.t16[xs2][lc][4 * lg];
          f16x4 vb;
#pragma unroll
          for (int e = 0; e < 4; ++e) vb[e] = (f16)(float)sm.rv[xs2][4 * lg + e][wcol + lc];
          f32x4 d0 = mma16h(ta, vb, zero4());
          f32x4 d1 = zero4(), o0 = zero4(), o1 = zero4();
          // D = U - W S and O = Qh S, two accumulation chains each.
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
            const f16x8 wa = cat8(*(const f16x4*)&sm.wneg[xs2][lc][32 * s + 4 * lg],
                                  *(const f16x4*)&sm.wneg[xs2][lc][32 * s + 16 + 4 * lg]);
            const f16x8 qa = cat8(*(const f16x4*)&sm.qh16[xs4][lc][32 * s + 4 * lg],
                                  *(const f16x4*)&sm.qh16[xs4][lc][32 * s + 16 + 4 * lg]);
            if (s & 1) {
              d1 = mma32h(wa, sop[s], d1);
              o1 = mma32h(qa, sop[s], o1);
            } else {
              d0 = mma32h(wa, sop[s], d0);
              o0 = mma32h(qa, sop[s], o0);
            }
          }
          d16 = to_h4(d0 + d1);
          // O += Aqk D
          const f16x4 qk = *(const f16x4*)&sm.aqk16[xs2][lc][4 * lg];
          O = mma16h(qk, d16, o0 + o1);
        }
        __syncthreads();

        // ---- phase B: state update of tile xs; write tile xf; stage v / gate
        if (run_s) {
          const int xs4 = (int)(xs & 3);
          // S <- e^(G_n) S + Kb^T D
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const f32x4 e4 = *(const f32x4*)&sm.en[xs4][16 * kb + 4 * lg];
            const f16x4 ka = *(const f16x4*)&sm.kbT[xs4][16 * kb + lc][4 * lg];
            S[kb] = mma16h(ka, d16, S[kb] * e4);
          }
          if (GATE) {
            // Row sums of squares of this wave's 16 output columns.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ss = row_sum16(O[r] * O[r]);
              if (lc == 0) sm.rsT[wave][4 * lg + r] = ss;
            }
          }
          Oprev = O;
        }
        if (run_f) {
          // 16-byte stores of whole rows of the finished tile.
          constexpr int TPR = DVW / 8;  // lanes per row
          if (tid < kC * TPR) {
            const int row = tid / TPR, c8 = (tid % TPR) * 8;
            if (xf * kC + row < T) {
              const bf16x4 a = *(const bf16x4*)&sm.otile[row][c8];
              const bf16x4 z = *(const bf16x4*)&sm.otile[row][c8 + 4];
              *(bf16x8*)(o + tokoff(xf * kC + row) * DV + col0 + c8) =
                  bf16x8{a[0], a[1], a[2], a[3], z[0], z[1], z[2], z[3]};
            }
          }
        }
        stage_s(it - 2, ps[u]);
        ps[u] = load_s(it - 2 + kLead);
        __syncthreads();
      }
    }

    if (s_out != nullptr) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float* p = s_out + (bh * kDK + 16 * kb + 4 * lg) * DV + col0 + wcol + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[(int64_t)r * DV] = S[kb][r];
      }
    }
  } else {
    // ============================================================ builder waves
    const int bw = wave - NS;            // key slab 32 bw .. 32 bw + 31
    const int bl = tid - NS * 64;        // builder lane 0..255: tile row bl / 16,
    const int b_row = bl / 16;           //   channels 8 (bl % 16) .. + 7
    const int b_c8 = (bl % 16) * 8;
    struct PfB {
      bf16x8 q, k;
      f32x4 g0, g1;
      float beta;
    };
    auto load_b = [&](int64_t x) {
      PfB r;
      const int64_t off = tokoff(x * kC + b_row) * kDK + b_c8;
      r.q = *(const bf16x8*)(q + off);
      r.k = *(const bf16x8*)(k + off);
      r.g0 = *(const f32x4*)(g + off);
      r.g1 = *(const f32x4*)(g + off + 4);
      r.beta = beta[tokoff(x * kC + (bl % kC))];
      return r;
    };
    // Staged unmasked; the operand build zeroes the rows past the sequence end.
    auto stage_b = [&](const PfB& r) {
      *(bf16x8*)&sm.rq[b_row][b_c8] = r.q;
      *(bf16x8*)&sm.rk[b_row][b_c8] = r.k;
      *(f32x4*)&sm.rg[b_row][b_c8] = r.g0;
      *(f32x4*)&sm.rg[b_row][b_c8 + 4] = r.g1;
      if (bl < kC) sm.rb[bl] = r.beta;
    };

    // Right operands selecting slab channels 16 hh + c into column c.
    f16x8 ident[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) ident[hh][e] = (f16)((8 * lg + e == lc + 16 * hh) ? 1.f : 0.f);

    // Tile 0 staged now; slot u is staged in iteration i0 + u as tile it + 1.
    stage_b(load_b(0));
    PfB pb[kLead];
#pragma unroll
    for (int u = 0; u < kLead; ++u) pb[u] = load_b(u + 1);
    __syncthreads();

    for (int64_t i0 = 0; i0 < niter; i0 += kLead) {
#pragma unroll
      for (int u = 0; u < kLead; ++u) {
        const int64_t it = i0 + u;
        if (it >= niter) break;
        const int64_t xb = it;      // tile being built
        const int64_t xw = it - 2;  // tile whose W this wave helps form
        const int64_t xv = it - 1;  // tile solved by builder kNB - 1
        const bool run_b = xb < nchunks;
        const bool run_w = xw >= 0 && xw < nchunks;
        const bool run_v = bw == kNB - 1 && xv >= 0 && xv < nchunks;

        // ---- phase A: two blocks of W for tile xw; rescaled operands of tile xb
        if (run_w) {
          // W^T = Kh^T T^T: block kb holds W[i = lc][16kb + 4lg + r]; store -W.
          const int xw2 = (int)(xw & 1), xw3 = (int)(xw % 3);
          const f16x4 tb = *(const f16x4*)&sm.t16[xw2][lc][4 * lg];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int kb = 2 * bw + kk;
            const f16x4 ka = *(const f16x4*)&sm.khT[xw3][16 * kb + lc][4 * lg];
            const f32x4 w = mma16h(ka, tb, zero4());
            *(f16x4*)&sm.wneg[xw2][lc][16 * kb + 4 * lg] = to_h4(-w);
          }
        }
        if (run_b) {
          // Lane = (token t, 8 channels of this wave's slab); the scan runs over the 16-lane row.
          const int t = lane % 16;
          const int ch = 32 * bw + 8 * (lane / 16);
          const int xb4 = (int)(xb & 3), xb3 = (int)(xb % 3), xb2 = (int)(xb & 1);
          // Tokens past the sequence end become g = 0, beta = 0, q = k = 0: the identity.
          const bool live = xb * kC + t < T;
          bf16x8 qv = *(const bf16x8*)&sm.rq[t][ch];
          bf16x8 kv = *(const bf16x8*)&sm.rk[t][ch];
          f32x4 g0 = *(const f32x4*)&sm.rg[t][ch];
          f32x4 g1 = *(const f32x4*)&sm.rg[t][ch + 4];
          if (!live) {
            qv = bf16x8{};
            kv = bf16x8{};
            g0 = zero4();
            g1 = zero4();
          }
          float gam[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) gam[e] = row_scan16(gam[e]);
          bf16x8 qhh, qhl, khb, kch, kcl;
          f16x8 qh16, kh16, kb16;
          float en8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float eg = __expf(gam[e]);
            const float ieg = __expf(-gam[e]);
            en8[e] = row_last16(eg);  // e^(G_n) of this channel
            const float kk = (float)kv[e];
            const float qhat = scale * (float)qv[e] * eg;
            const float khat = kk * eg;
            const float kchk = kk * ieg;
            qh16[e] = (f16)qhat;
            qhh[e] = (bf16_t)qhat;
            qhl[e] = (bf16_t)(qhat - (float)qhh[e]);
            khb[e] = (bf16_t)khat;
            kch[e] = (bf16_t)kchk;
            kcl[e] = (bf16_t)(kchk - (float)kch[e]);
            kh16[e] = (f16)khat;
            kb16[e] = (f16)(kchk * en8[e]);  // k e^(G_n - G_t) <= |k|
          }
          // Channel-major copies of Kh and Kb: the lane's 8 channels of token t form
          // the left operand of a product with a 0/1 selection matrix, whose
          // accumulator holds 4 tokens of one channel per lane (exact in float32).
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x4 th = mma32h(kh16, ident[hh], zero4());
            const f32x4 tb = mma32h(kb16, ident[hh], zero4());
            const int chl = 32 * bw + 16 * hh + lc;
            *(f16x4*)&sm.khT[xb3][chl][4 * lg] = to_h4(th);
            *(f16x4*)&sm.kbT[xb4][chl][4 * lg] = to_h4(tb);
          }
          *(bf16x8*)&sm.qhh[t][ch] = qhh;
          *(bf16x8*)&sm.qhl[t][ch] = qhl;
          *(bf16x8*)&sm.khb[t][ch] = khb;
          *(bf16x8*)&sm.kch[t][ch] = kch;
          *(bf16x8*)&sm.kcl[t][ch] = kcl;
          *(f16x4*)&sm.qh16[xb4][t][ch] = f16x4{qh16[0], qh16[1], qh16[2], qh16[3]};
          *(f16x4*)&sm.qh16[xb4][t][ch + 4] = f16x4{qh16[4], qh16[5], qh16[6], qh16[7]};
          if (t == 15) {
            *(f32x4*)&sm.en[xb4][ch] = f32x4{en8[0], en8[1], en8[2], en8[3]};
            *(f32x4*)&sm.en[xb4][ch + 4] = f32x4{en8[4], en8[5], en8[6], en8[7]};
          }
          if (bw == 0 && lane < kC) sm.betab[xb2][lane] = live ? sm.rb[lane] : 0.f;
        }
        __syncthreads();

        // ---- phase B: partial intra-tile products of tile xb; solve tile xv; stage inputs
        if (run_b) {
          const int xb2 = (int)(xb & 1);
          const int c0 = 32 * bw + 8 * lg;
          const bf16x8 ah = *(const bf16x8*)&sm.qhh[lc][c0];
          const bf16x8 al = *(const bf16x8*)&sm.qhl[lc][c0];
          const bf16x8 ak = *(const bf16x8*)&sm.khb[lc][c0];
          const bf16x8 bh8 = *(const bf16x8*)&sm.kch[lc][c0];
          const bf16x8 bl8 = *(const bf16x8*)&sm.kcl[lc][c0];
          const f32x4 pa = mma32b(ak, bh8, zero4());
          f32x4 pq = mma32b(ah, bh8, zero4());
          pq = mma32b(ah, bl8, pq);
          pq = mma32b(al, bh8, pq);
          *(f32x4*)&sm.partA[xb2][bw][lc][4 * lg] = pa;
          *(f32x4*)&sm.partQ[xb2][bw][lc][4 * lg] = pq;
        }
        if (run_v) {
          // Sum the slab partials of tile xv, apply beta and the causal masks.
          const int xv2 = (int)(xv & 1);
          const int j = lc, i0r = 4 * lg;
          f32x4 pa = zero4(), pq = zero4();
#pragma unroll
          for (int p = 0; p < kNB; ++p) {
            pa += *(const f32x4*)&sm.partA[xv2][p][j][i0r];
            pq += *(const f32x4*)&sm.partQ[xv2][p][j][i0r];
          }
          const f32x4 bi = *(const f32x4*)&sm.betab[xv2][i0r];
          f32x4 at;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0r + r;
            at[r] = (j < i) ? bi[r] * pa[r] : 0.f;  // select: masked entries may be huge
            sm.aqk16[xv2][i][j] = (f16)((j <= i) ? pq[r] : 0.f);
          }
          *(f32x4*)&sm.aT[j][i0r] = at;
          wave_lds_sync();
          // T = (I + A)^-1 Diag(beta): lane j < 16 solves column j by forward
          // substitution; the rows of A^T are read three steps ahead of use.
          if (lane < kC) {
            float y[kC];
#pragma unroll
            for (int i = 0; i < kC; ++i) y[i] = (i == lane) ? 1.f : 0.f;
            constexpr int kAhead = 3;
            f32x4 rowbuf[kAhead][kC / 4];
#pragma unroll
            for (int m = 0; m < kAhead; ++m)
#pragma unroll
              for (int q = 0; q < kC / 4; ++q) rowbuf[m][q] = *(const f32x4*)&sm.aT[m][4 * q];
#pragma unroll
            for (int m = 0; m < kC - 1; ++m) {
              float a[kC];
#pragma unroll
              for (int q = 0; q < kC / 4; ++q) {
                a[4 * q] = rowbuf[m % kAhead][q][0];
                a[4 * q + 1] = rowbuf[m % kAhead][q][1];
                a[4 * q + 2] = rowbuf[m % kAhead][q][2];
                a[4 * q + 3] = rowbuf[m % kAhead][q][3];
              }
              if (m + kAhead < kC - 1) {
#pragma unroll
                for (int q = 0; q < kC / 4; ++q)
                  rowbuf[m % kAhead][q] = *(const f32x4*)&sm.aT[m + kAhead][4 * q];
              }
              const float ym = y[m];
#pragma unroll
              for (int i = m + 1; i < kC; ++i) y[i] = fmaf(-a[i], ym, y[i]);
            }
            const float bj = sm.betab[xv2][lane];
#pragma unroll
            for (int i = 0; i < kC; ++i) sm.t16[xv2][i][lane] = (f16)(bj * y[i]);
          }
        }
        stage_b(pb[u]);
        pb[u] = load_b(it + 1 + kLead);
        __syncthreads();
      }
    }
  }
}

template <int DV, int DVW, bool GATE>
hipError_t launch_t(const ChunkArgs& a) {
  const int64_t nblk = a.B * a.H * (DV / DVW);
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kda_chunk_mfma_kernel<DV, DVW, GATE>), dim3((unsigned)nblk),
                     dim3(Cfg<DVW>::NT), 0, (hipStream_t)a.stream, (const bf16_t*)a.q,
                     (const bf16_t*)a.k, (const bf16_t*)a.v, a.g, a.beta, a.s0, (bf16_t*)a.o,
                     a.s_out, (const bf16_t*)a.gate, a.norm_w, a.eps, a.T, a.H, a.B * a.H,
                     a.scale);
  return hipGetLastError();
}

// Columns per workgroup: a head's whole dv row when the gated norm is fused
// (it needs the row), otherwise half of it when that is what fills the GPU.
int split_for(const ChunkArgs& a) {
  if (a.gate != nullptr) return 1;
  if (const char* e = getenv("KDA_CHUNK_SPLIT")) {
    const int s = atoi(e);
    if (s == 1 || s == 2) return s;
  }
  return (a.B * a.H < 256) ? 2 : 1;
}

}  // namespace

bool chunk_mfma_supports(int dk, int dv, bool io_bf16) {
  return io_bf16 && dk == kDK && dv == 128;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  if (!chunk_mfma_supports(a.dk, a.dv, a.io_bf16)) return hipErrorNotSupported;
  if (a.gate != nullptr) return launch_t<128, 128, true>(a);
  return split_for(a) == 2 ? launch_t<128, 64, false>(a) : launch_t<128, 128, false>(a);
}

}  // namespace kda
