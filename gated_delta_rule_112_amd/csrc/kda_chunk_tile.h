// Tile builder of the matrix-core chunked prefill: everything about a 16-token
// tile that does not depend on the running state (kda_chunk_rec.h), computed
// by one wavefront per tile.
//
// Lane (t, g) = (lane % 16, lane / 16) holds token t and, for each 32-channel
// slab s, the key channels 32 s + 8 g + 0..7.  Per slab it forms the in-tile
// cumulative log-decay (a prefix sum over the 16 lanes of a DPP row), the
// exponentials and the rescaled operands, and accumulates the two intra-tile
// products over the slab on the matrix cores in float32 (16x16x4: each k step
// is one of the lane's channels, so the operands come straight from
// registers):
//   lane (i, g) accumulates (Kh Kc^T)[i][4 g + r] and (Qh Kc^T)[i][4 g + r].
// Kh and Kb are transposed to channel-major 16x16 blocks by a product with a
// 0/1 selection matrix (exact).  The 16x16 unit-lower-triangular system
// (I + A) Y = I is solved by forward substitution, lane (i, g) holding rows i
// of columns 4 g + 0..3 and the pivot row broadcast over each DPP row; then
// T = Y Diag(beta) and W = T Kh.  The results are stored as the tile's record.
//
// Precision: all sums over key channels and the solve are float32; the stored
// matrix operands are float16 (11-bit significand), e^G_15 is float32.
#pragma once

#include "kda_chunk_rec.h"

namespace kda {
namespace tile {

constexpr float kLog2e = 1.4426950408889634f;

struct Args {
  const bf16_t* q;
  const bf16_t* k;
  const float* g;
  const float* beta;
  unsigned char* recs;  // records of the segment, [head][tile]
  int64_t T, H, BH;
  int64_t x0, nseg;     // first tile and tile count of the segment
  float scale;
};

// One lane's inputs of one tile.
struct Inputs {
  bf16x8 q[4], k[4];
  f32x4 g[4][2];
  float beta;
};

struct Scratch {  // per wavefront
  float a[16][20];  // A = strict_lower(Diag(beta) Kh Kc^T), row-major, padded rows
  float beta[16];
};

// Loads tile w = (head, tile of the segment) < BH * nseg.  Rows past the end
// of the sequence are clamped copies (zeroed by build()).
__device__ __forceinline__ void load(Inputs& in, const Args& a, int64_t w, int lane) {
  const int64_t bh = w / a.nseg, xl = w % a.nseg;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int t = lane % 16, lg = lane / 16;
  int64_t tok = (a.x0 + xl) * rec::kC + t;
  tok = tok < a.T ? tok : a.T - 1;
  const int64_t row = (b * a.T + tok) * a.H + h;
  const bf16_t* qp = a.q + row * rec::kDK + 8 * lg;
  const bf16_t* kp = a.k + row * rec::kDK + 8 * lg;
  const float* gp = a.g + row * rec::kDK + 8 * lg;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    in.q[s] = __builtin_nontemporal_load((const bf16x8*)(qp + 32 * s));
    in.k[s] = __builtin_nontemporal_load((const bf16x8*)(kp + 32 * s));
    in.g[s][0] = __builtin_nontemporal_load((const f32x4*)(gp + 32 * s));
    in.g[s][1] = __builtin_nontemporal_load((const f32x4*)(gp + 32 * s + 4));
  }
  in.beta = a.beta[row];
}

// One step of the forward substitution: column values y[e] of rows i (this
// lane's row) receive -A[i][M] * y_M, with y_M broadcast from lane M of the row.
template <int M>
__device__ __forceinline__ void forward_sub(float (&y)[4], const f32x4 (&arow)[4]) {
  const float aim = arow[M / 4][M % 4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = fmaf(-aim, row_bcast<M>(y[e]), y[e]);
  if constexpr (M + 1 < 15) forward_sub<M + 1>(y, arow);
}

// Builds and stores the record of tile w from its inputs.
__device__ __forceinline__ void build(const Inputs& in, const Args& a, int64_t w, Scratch& sm,
                                      int lane) {
  const int t = lane % 16, lg = lane / 16;
  const int64_t xl = w % a.nseg;
  const bool live = (a.x0 + xl) * rec::kC + t < a.T;
  const float lv = live ? 1.f : 0.f;  // tokens past the end: q = k = g = beta = 0
  const float bt = in.beta * lv;
  unsigned char* R = a.recs + w * (int64_t)rec::kBytes;

  // Selection matrix for the transposes: B[k = 4 g + e][c] = (k == c).
  f16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (f16)((4 * lg + e == t) ? 1.f : 0.f);

  f32x4 acc_a = zero4();  // lane (i, g): (Kh Kc^T)[i][4 g + r]
  f32x4 acc_q = zero4();  // lane (t, g): (Qh Kc^T)[t][4 g + r]
  f16x4 khT[8];           // Kh^T blocks: lane (c, g): Kh[4 g + r][chan(b, c)]
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float gm[8] = {in.g[s][0][0], in.g[s][0][1], in.g[s][0][2], in.g[s][0][3],
                         in.g[s][1][0], in.g[s][1][1], in.g[s][1][2], in.g[s][1][3]};
    float kh[8], kc[8], qh[8], kb[8], en8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gl = row_scan16(gm[e] * (kLog2e * lv));  // G in log2 units
      const float eg = __builtin_amdgcn_exp2f(gl);          // e^G    <= 1
      const float ieg = __builtin_amdgcn_exp2f(-gl);        // e^-G   <  e^80
      en8[e] = row_bcast<15>(eg);                           // e^G_15 of this channel
      const float kf = (float)in.k[s][e] * lv;
      const float qf = (float)in.q[s][e] * (a.scale * lv);
      kh[e] = kf * eg;
      kc[e] = kf * ieg;
      qh[e] = qf * eg;
      kb[e] = kc[e] * en8[e];  // k e^(G_15 - G_t) <= |k|
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc_a = mma4f(kc[e], kh[e], acc_a);
      acc_q = mma4f(kc[e], qh[e], acc_q);
    }
    // Qh image of slab s.
    *(f16x8*)(R + rec::kQh + s * 1024 + lane * 16) =
        f16x8{(f16)qh[0], (f16)qh[1], (f16)qh[2], (f16)qh[3],
              (f16)qh[4], (f16)qh[5], (f16)qh[6], (f16)qh[7]};
    // Channel-major blocks 2s (channels 32 s + 8 g + 0..3) and 2s+1 (+ 4..7).
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const f16x4 kh4 = {(f16)kh[4 * hb], (f16)kh[4 * hb + 1], (f16)kh[4 * hb + 2],
                         (f16)kh[4 * hb + 3]};
      const f16x4 kb4 = {(f16)kb[4 * hb], (f16)kb[4 * hb + 1], (f16)kb[4 * hb + 2],
                         (f16)kb[4 * hb + 3]};
      khT[2 * s + hb] = to_h4(mma16h(kh4, ident, zero4()));
      *(f16x4*)(R + rec::kKb + (2 * s + hb) * 512 + lane * 8) = to_h4(mma16h(kb4, ident, zero4()));
    }
    if (t == 15) {
      f32x4* ep = (f32x4*)(R + rec::kEn + (32 * s + 8 * lg) * 4);
      ep[0] = f32x4{en8[0], en8[1], en8[2], en8[3]};
      ep[1] = f32x4{en8[4], en8[5], en8[6], en8[7]};
    }
  }

  // Causal masks (selects: masked entries may be huge products of e^-G).
  f32x4 am;
  f16x4 aq;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * lg + r;
    am[r] = (j < t) ? bt * acc_a[r] : 0.f;
    aq[r] = (f16)((j <= t) ? acc_q[r] : 0.f);
  }
  *(f16x4*)(R + rec::kAqk + lane * 8) = aq;
  *(f32x4*)&sm.a[t][4 * lg] = am;
  if (lg == 0) sm.beta[t] = bt;
  wave_lds_sync();

  // (I + A) Y = I by forward substitution; lane (i, g): Y[i][4 g + e].
  f32x4 arow[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) arow[c4] = *(const f32x4*)&sm.a[t][4 * c4];
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (t == 4 * lg + e) ? 1.f : 0.f;
  forward_sub<0>(y, arow);
  const f32x4 bj = *(const f32x4*)&sm.beta[4 * lg];
  wave_lds_sync();  // the scratch is reused by the wavefront's next tile
  const f16x4 tb = {(f16)(y[0] * bj[0]), (f16)(y[1] * bj[1]), (f16)(y[2] * bj[2]),
                    (f16)(y[3] * bj[3])};  // lane (i, g): T[i][4 g + e]
  *(f16x4*)(R + rec::kT + lane * 8) = tb;

  // W^T block b = Kh^T_b T^T: lane (i, g) receives W[i][chan(b, 4 g + r)].
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x4 w0 = mma16h(khT[2 * s], tb, zero4());
    const f32x4 w1 = mma16h(khT[2 * s + 1], tb, zero4());
    *(f16x8*)(R + rec::kW + s * 1024 + lane * 16) = cat8(to_h4(-w0), to_h4(-w1));
  }
}

// Tiles first, first + stride, ... < BH * nseg of one wavefront, each tile's
// inputs loaded while the previous tile is built.  Loads are issued for
// clamped tile indices so that every iteration has the same memory operations.
__device__ __forceinline__ void build_range(const Args& a, int64_t first, int64_t stride,
                                            Scratch& sm, int lane) {
  const int64_t total = a.BH * a.nseg;
  if (first >= total) return;
  auto clampw = [&](int64_t w) { return w < total ? w : total - 1; };
  Inputs in0, in1;
  load(in0, a, first, lane);
  for (int64_t w = first; w < total; w += 2 * stride) {
    load(in1, a, clampw(w + stride), lane);
    build(in0, a, w, sm, lane);
    if (w + stride >= total) break;
    load(in0, a, clampw(w + 2 * stride), lane);
    build(in1, a, w + stride, sm, lane);
  }
}

}  // namespace tile
}  // namespace kda
