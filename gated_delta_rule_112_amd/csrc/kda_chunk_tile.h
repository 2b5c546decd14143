// Tile builder of the matrix-core chunked prefill: everything about a 16-token
// tile that does not depend on the running state (kda_chunk_rec.h).
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
// 0/1 selection matrix (exact).  With the products summed over all slabs, the
// 16x16 unit-lower-triangular system (I + A) Y = I is solved by forward
// substitution, lane (i, g) holding rows i of columns 4 g + 0..3 and the pivot
// row broadcast over each DPP row; then T = Y Diag(beta) and W = T Kh, one
// 32-channel slab of W at a time.
//
// The pieces are used whole (one wavefront builds a tile and stores its
// record in memory) and sliced (four wavefronts build one slab each and
// write the record into LDS).
//
// Precision: all sums over key channels and the solve are float32; the stored
// matrix operands are float16 (11-bit significand), e^G_15 is float32.
#pragma once

#include "kda_chunk_rec.h"

namespace kda {

// LDS accesses issued directly.  Wavefronts that also have direct-to-LDS
// loads in flight use these: for a plain LDS access the compiler would first
// wait for every load in flight (it cannot tell that they target other
// bytes).  Within one wavefront, LDS accesses complete in issue order.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void ds_write16(unsigned a, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_write8(unsigned a, f32x2 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_write4(unsigned a, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4 ds_read16(unsigned a) {
  f32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
template <typename V>
__device__ __forceinline__ f32x4 as_f4(V x) { return __builtin_bit_cast(f32x4, x); }
template <typename V>
__device__ __forceinline__ f32x2 as_f2(V x) { return __builtin_bit_cast(f32x2, x); }

namespace tile {

constexpr float kLog2e = 1.4426950408889634f;

// One lane's inputs of one 32-channel slab of a tile.
struct SlabIn {
  bf16x8 q, k;
  f32x4 g0, g1;
};

// One lane's results of one slab, in the record's operand images.
struct SlabOut {
  f16x8 qh;      // Qh image of the slab
  f16x4 kbT[2];  // Kb^T blocks 2s, 2s+1
  f16x4 khT[2];  // Kh^T blocks 2s, 2s+1 (kept for W)
  f32x4 en[2];   // e^G_15 of the lane's 8 channels (stored from lanes t == 15)
};

struct Scratch {  // per wavefront, for the solve
  float a[16][20];  // A = strict_lower(Diag(beta) Kh Kc^T), row-major, padded rows
  float beta[16];
};

// Element offset of the row of token `tok` (clamped into the sequence) of head (b, h).
__device__ __forceinline__ int64_t row_of(int64_t b, int64_t h, int64_t tok, int64_t T,
                                          int64_t H) {
  tok = tok < T ? tok : T - 1;
  return (b * T + tok) * H + h;
}

__device__ __forceinline__ void load_slab(SlabIn& in, const bf16_t* q, const bf16_t* k,
                                          const float* g, int64_t row, int s, int lane) {
  const int64_t off = row * rec::kDK + 32 * s + 8 * (lane / 16);
  in.q = __builtin_nontemporal_load((const bf16x8*)(q + off));
  in.k = __builtin_nontemporal_load((const bf16x8*)(k + off));
  in.g0 = __builtin_nontemporal_load((const f32x4*)(g + off));
  in.g1 = __builtin_nontemporal_load((const f32x4*)(g + off + 4));
}

// Selection matrix for the transposes: B[k = 4 g + e][c] = (k == c).
__device__ __forceinline__ f16x4 selection(int lane) {
  f16x4 id;
#pragma unroll
  for (int e = 0; e < 4; ++e) id[e] = (f16)((4 * (lane / 16) + e == lane % 16) ? 1.f : 0.f);
  return id;
}

// Builds one slab.  lv = 1 for a token of the sequence, 0 past its end (then
// q = k = g = 0); FULL tiles skip that mask.
template <bool FULL>
__device__ __forceinline__ void build_slab(const SlabIn& in, float lv, float scale, f16x4 ident,
                                           f32x4& acc_a, f32x4& acc_q, SlabOut& out) {
  const float gm[8] = {in.g0[0], in.g0[1], in.g0[2], in.g0[3],
                       in.g1[0], in.g1[1], in.g1[2], in.g1[3]};
  const float gs = FULL ? kLog2e : kLog2e * lv;
  const float qs = FULL ? scale : scale * lv;
  float kh[8], kc[8], qh[8], kb[8], en8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gl = row_scan16(gm[e] * gs);         // G in log2 units
    const float eg = __builtin_amdgcn_exp2f(gl);     // e^G    <= 1
    const float ieg = __builtin_amdgcn_exp2f(-gl);   // e^-G   <  e^80
    en8[e] = row_bcast<15>(eg);                      // e^G_15 of this channel
    const float kf = FULL ? (float)in.k[e] : (float)in.k[e] * lv;
    kh[e] = kf * eg;
    kc[e] = kf * ieg;
    qh[e] = (float)in.q[e] * qs * eg;
    kb[e] = kc[e] * en8[e];  // k e^(G_15 - G_t) <= |k|
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc_a = mma4f(kc[e], kh[e], acc_a);
    acc_q = mma4f(kc[e], qh[e], acc_q);
  }
  out.qh = f16x8{(f16)qh[0], (f16)qh[1], (f16)qh[2], (f16)qh[3],
                 (f16)qh[4], (f16)qh[5], (f16)qh[6], (f16)qh[7]};
  // Channel-major blocks 2s (channels 32 s + 8 g + 0..3) and 2s+1 (+ 4..7).
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const f16x4 kh4 = {(f16)kh[4 * hb], (f16)kh[4 * hb + 1], (f16)kh[4 * hb + 2],
                       (f16)kh[4 * hb + 3]};
    const f16x4 kb4 = {(f16)kb[4 * hb], (f16)kb[4 * hb + 1], (f16)kb[4 * hb + 2],
                       (f16)kb[4 * hb + 3]};
    out.khT[hb] = to_h4(mma16h(kh4, ident, zero4()));
    out.kbT[hb] = to_h4(mma16h(kb4, ident, zero4()));
  }
  out.en[0] = f32x4{en8[0], en8[1], en8[2], en8[3]};
  out.en[1] = f32x4{en8[4], en8[5], en8[6], en8[7]};
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

// From the intra-tile products summed over all slabs: the causal masks, the
// solve and T.  bt = beta of this lane's token (0 past the sequence end).
// Returns this lane's T image (lane (i, g): T[i][4 g + e]) and Aqk image.
__device__ __forceinline__ void finish(f32x4 acc_a, f32x4 acc_q, float bt, Scratch* sm, int lane,
                                       f16x4& tb, f16x4& aq) {
  const int t = lane % 16, lg = lane / 16;
  f32x4 am;  // selects: masked entries may be huge products of e^-G
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * lg + r;
    am[r] = (j < t) ? bt * acc_a[r] : 0.f;
    aq[r] = (f16)((j <= t) ? acc_q[r] : 0.f);
  }
  const unsigned arow_addr = lds_addr(&sm->a[t][0]);
  ds_write16(lds_addr(&sm->a[t][4 * lg]), am);
  if (lg == 0) ds_write4(lds_addr(&sm->beta[t]), bt);
  // (I + A) Y = I by forward substitution; lane (i, g): Y[i][4 g + e].
  f32x4 arow[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %4 offset:32\n\t"
      "ds_read_b128 %3, %4 offset:48\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(arow[0]), "=v"(arow[1]), "=v"(arow[2]), "=v"(arow[3])
      : "v"(arow_addr)
      : "memory");
  const f32x4 bj = ds_read16(lds_addr(&sm->beta[4 * lg]));
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (t == 4 * lg + e) ? 1.f : 0.f;
  forward_sub<0>(y, arow);
  tb = f16x4{(f16)(y[0] * bj[0]), (f16)(y[1] * bj[1]), (f16)(y[2] * bj[2]), (f16)(y[3] * bj[3])};
}

// W^T blocks 2s, 2s+1 = Kh^T T^T: the lane's (i, g) image of -W for slab s,
// -W[i][32 s + 8 g + e].
__device__ __forceinline__ f16x8 w_slab(const f16x4 (&khT)[2], f16x4 tb) {
  const f32x4 w0 = mma16h(khT[0], tb, zero4());
  const f32x4 w1 = mma16h(khT[1], tb, zero4());
  return cat8(to_h4(-w0), to_h4(-w1));
}

// ---------------------------------------------------------------- whole tiles

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

// Position of a tile: head (b, h) and tile xl of the segment.
struct Pos {
  int64_t b, h, xl;
};

__device__ __forceinline__ int64_t tile_row(const Args& a, const Pos& p, int lane) {
  return row_of(p.b, p.h, (a.x0 + p.xl) * rec::kC + lane % 16, a.T, a.H);
}

// Tiles first, first + stride, ... < BH * nseg of one wavefront, numbered
// head-fastest (tile w is tile w / BH of head w % BH), so that the wavefronts
// working at one time read neighbouring heads of the same tokens, which are
// adjacent in memory; every record goes to memory.  PIPE: software pipelined
// over slabs (as soon as slab s of a tile is built, slab s of the wavefront's
// next tile is loaded into the same registers, so one tile's inputs are in
// flight while the rest of the current tile is built; past the last tile the
// loads repeat the last tile).  Without PIPE each tile loads its own inputs
// first (for workgroups with enough wavefronts per SIMD to cover the latency,
// and too few registers per wavefront to hold a second tile's inputs).
template <bool PIPE>
__device__ __forceinline__ void build_range(const Args& a, int64_t first, int64_t stride,
                                            Scratch* sm, int lane) {
  const int64_t total = a.BH * a.nseg;
  if (first >= total) return;
  const int t = lane % 16, lg = lane / 16;
  const f16x4 ident = selection(lane);
  const int64_t B = a.BH / a.H;
  // w = xl BH + b H + h; the stride split the same way, advanced without divisions
  const int64_t sxl = stride / a.BH, sbh = stride - sxl * a.BH;
  const int64_t sb = sbh / a.H, sh = sbh - sb * a.H;
  Pos p;
  {
    p.xl = first / a.BH;
    const int64_t bh = first - p.xl * a.BH;
    p.b = bh / a.H;
    p.h = bh - p.b * a.H;
  }
  const Pos last{B - 1, a.H - 1, a.nseg - 1};
  SlabIn in[4];
  float beta;
  if constexpr (PIPE) {
    const int64_t row = tile_row(a, p, lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) load_slab(in[s], a.q, a.k, a.g, row, s, lane);
    beta = a.beta[row];
  }
  for (int64_t w = first; w < total; w += stride) {
    if constexpr (!PIPE) {
      const int64_t row = tile_row(a, p, lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) load_slab(in[s], a.q, a.k, a.g, row, s, lane);
      beta = a.beta[row];
    }
    // the wavefront's next tile (clamped to the last tile)
    Pos n{p.b + sb, p.h + sh, p.xl + sxl};
    if (n.h >= a.H) {
      n.h -= a.H;
      ++n.b;
    }
    if (n.b >= B) {
      n.b -= B;
      ++n.xl;
    }
    const int64_t nrow =
        PIPE ? (w + stride < total ? tile_row(a, n, lane) : tile_row(a, last, lane)) : 0;
    const int64_t xl = p.xl, bh = p.b * a.H + p.h;

    const int64_t tok0 = (a.x0 + xl) * rec::kC;
    const bool full = tok0 + rec::kC <= a.T;
    const float lv = tok0 + t < a.T ? 1.f : 0.f;
    unsigned char* R = a.recs + (bh * a.nseg + xl) * (int64_t)rec::kBytes;
    f32x4 acc_a = zero4(), acc_q = zero4();
    f16x4 khT[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      SlabOut so;
      if (full)
        build_slab<true>(in[s], 1.f, a.scale, ident, acc_a, acc_q, so);
      else
        build_slab<false>(in[s], lv, a.scale, ident, acc_a, acc_q, so);
      if constexpr (PIPE) load_slab(in[s], a.q, a.k, a.g, nrow, s, lane);
      *(f16x8*)(R + rec::kQh + s * 1024 + lane * 16) = so.qh;
      *(f16x4*)(R + rec::kKb + (2 * s) * 512 + lane * 8) = so.kbT[0];
      *(f16x4*)(R + rec::kKb + (2 * s + 1) * 512 + lane * 8) = so.kbT[1];
      if (t == 15) {
        f32x4* ep = (f32x4*)(R + rec::kEn + (32 * s + 8 * lg) * 4);
        ep[0] = so.en[0];
        ep[1] = so.en[1];
      }
      khT[s][0] = so.khT[0];
      khT[s][1] = so.khT[1];
    }
    f16x4 tb, aq;
    finish(acc_a, acc_q, beta * lv, sm, lane, tb, aq);
    if constexpr (PIPE) beta = a.beta[nrow];
    *(f16x4*)(R + rec::kAqk + lane * 8) = aq;
    *(f16x4*)(R + rec::kT + lane * 8) = tb;
#pragma unroll
    for (int s = 0; s < 4; ++s) *(f16x8*)(R + rec::kW + s * 1024 + lane * 16) = w_slab(khT[s], tb);
    p = n;
  }
}

}  // namespace tile
}  // namespace kda
