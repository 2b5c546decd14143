// Tile builder of the matrix-core chunked prefill: everything about a pair of
// 16-token tiles that does not depend on the running state (kda_chunk_rec.h).
//
// Lane (t, g) = (lane % 16, lane / 16) holds token t and, for each 32-channel
// slab s, the key channels 32 s + 8 g + 0..7.  Per slab and tile it forms the
// in-tile cumulative log-decay (a prefix sum over the 16 lanes of a DPP row),
// the exponentials and the rescaled operands, and accumulates the two
// intra-tile products over the slab on the matrix cores in float32 (16x16x4:
// each k step is one of the lane's channels, so the operands come straight
// from registers):
//   lane (i, g) accumulates (Kh Kc^T)[i][4 g + r] and (Qh Kc^T)[i][4 g + r].
// Kh and Kb are transposed to channel-major 16x16 blocks through LDS with the
// transpose read of gfx950 (exact).  With the products summed over all slabs, the
// 16x16 unit-lower-triangular system (I + A) Y = I is solved by forward
// substitution, lane (i, g) holding rows i of columns 4 g + 0..3 and the pivot
// row broadcast over each DPP row; then T = Y Diag(beta) and W = T Kh, one
// 32-channel slab of W at a time.  The two tiles of a pair are built slab by
// slab side by side, so that the cross terms (Kb_a scaled by E_b, Qh_b scaled
// by E_a, Q_ba = Qh_b Kb_a^T, M = Kh_b Kb_a^T) come from registers;
// P = -W_b Kb_a^T = -T_b M and W_b scaled by E_a follow tile b's solve.
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

// One lane's inputs of one 32-channel slab of a tile: g, or its logits.
struct SlabIn {
  bf16x8 q, k;
  f32x4 g0, g1;
  bf16x8 ga;
};

struct Scratch {  // per wavefront
  f16x4 tr[2][64];  // staging of the transposes, [half slab][lane]
  float a[16][20];  // -A = -strict_lower(Diag(beta) Kh Kc^T), row-major, padded rows
  float beta[16];
  float rk[16];     // 1/|k| per token of the tile being finished (keys normalised here)
  float en_a[rec::kDK];  // E_a of the pair being built, per key channel
};

// Row index (into [rows, H, *] tensors) of token `tok` of head (b, h), the
// token clamped into its sequence.
template <bool PACKED>
__device__ __forceinline__ int64_t row_of(const Seqs<PACKED>& sq, int64_t b, int64_t h,
                                          int64_t tok, int64_t H) {
  return sq.row(b, tok) * H + h;
}

// This lane's q and k of slab s (and of slab s + 1, into q1 / k1) and g of slab
// s.  A slab of q or k is 64 bytes of a token row, half a 128-byte line: the
// two slabs of a line are loaded by back-to-back instructions, so that each
// line leaves memory once (loaded a slab apart, the first half's line was
// often gone when the second half was read).
template <bool LOGITS>
__device__ __forceinline__ void load_slab(SlabIn& in, bf16x8& q1, bf16x8& k1, const bf16_t* q,
                                          const bf16_t* k, const float* g, const bf16_t* ga,
                                          int64_t row, int s, int lane) {
  const int64_t off = row * rec::kDK + 32 * s + 8 * (lane / 16);
  if (s % 2 == 0) {
    in.q = __builtin_nontemporal_load((const bf16x8*)(q + off));
    q1 = __builtin_nontemporal_load((const bf16x8*)(q + off + 32));
    in.k = __builtin_nontemporal_load((const bf16x8*)(k + off));
    k1 = __builtin_nontemporal_load((const bf16x8*)(k + off + 32));
  }
  if constexpr (LOGITS) {
    in.ga = __builtin_nontemporal_load((const bf16x8*)(ga + off));
  } else {
    in.g0 = __builtin_nontemporal_load((const f32x4*)(g + off));
    in.g1 = __builtin_nontemporal_load((const f32x4*)(g + off + 4));
  }
}

// sigmoid(x) with the hardware exponential and reciprocal.
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// One lane's rescaled values of one slab of one tile (channels 32 s + 8 g + e).
struct SlabVals {
  float kh[8], kc[8], qh[8], kb[8], en[8];
};

// The rescaled values of one slab, and its contribution to the two
// intra-tile products.  lv = 1 for a token of the sequence, 0 past its end
// (then q = k = g = 0); FULL tiles skip that mask.
// With LOGITS, nq and nk also accumulate this lane's part of |q|^2 and |k|^2.
template <bool FULL, bool LOGITS>
__device__ __forceinline__ void slab_vals(const SlabIn& in, float lv, SlabVals& o,
                                          f32x4& acc_a, f32x4& acc_q, float& nq, float& nk) {
  float gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (LOGITS)
      gm[e] = -5.f * fast_sigmoid((float)in.ga[e]);  // the decay floor: g = -5 sigmoid(a)
    else
      gm[e] = e < 4 ? in.g0[e] : in.g1[e - 4];
  }
  const float gs = FULL ? kLog2e : kLog2e * lv;
  const float qs = FULL ? 1.f : lv;  // the output scale is applied by the state pass
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gl = row_scan16(gm[e] * gs);         // G in log2 units
    const float eg = __builtin_amdgcn_exp2f(gl);     // e^G    <= 1
    const float ieg = __builtin_amdgcn_exp2f(-gl);   // e^-G   <  e^80
    o.en[e] = row_bcast<15>(eg);                     // e^G_15 of this channel
    const float kf = FULL ? (float)in.k[e] : (float)in.k[e] * lv;
    const float qf = (float)in.q[e];
    if constexpr (LOGITS) {
      nq = fmaf(qf, qf, nq);
      nk = fmaf(kf, kf, nk);
    }
    o.kh[e] = kf * eg;
    o.kc[e] = kf * ieg;
    o.qh[e] = qf * qs * eg;
    o.kb[e] = o.kc[e] * o.en[e];  // k e^(G_15 - G_t) <= |k|
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc_a = mma4f(o.kc[e], o.kh[e], acc_a);
    acc_q = mma4f(o.kc[e], o.qh[e], acc_q);
  }
}

template <bool LOGITS>
__device__ __forceinline__ void slab_vals_any(bool full, const SlabIn& in, float lv,
                                              SlabVals& o, f32x4& acc_a, f32x4& acc_q, float& nq,
                                              float& nk) {
  if (full)
    slab_vals<true, LOGITS>(in, 1.f, o, acc_a, acc_q, nq, nk);
  else
    slab_vals<false, LOGITS>(in, lv, o, acc_a, acc_q, nq, nk);
}

__device__ __forceinline__ f16x8 to_h8(const float (&x)[8]) {
  return f16x8{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3],
               (f16)x[4], (f16)x[5], (f16)x[6], (f16)x[7]};
}

// Channel-major blocks 2s (channels 32 s + 8 g + 0..3) and 2s+1 (+ 4..7) of a
// token-major slab: out[hb] lane (c, g) = x[token 4 g + r][chan(2 s + hb, c)],
// through LDS.  Each lane stores its 4 channels of a half slab (8 bytes, in
// lane order); lane 16 g + j then reads the 4 channels 32 s + 8 (j % 4) +
// 4 hb + 0..3 of token 4 g + j / 4 with the transpose read
// (ds_read_b64_tr_b16), which hands lane i of each 16-lane group element
// i % 4 of what lane 4 e + i / 4 of its group read, as its element e.
__device__ __forceinline__ void transpose_slab(const float (&x)[8], Scratch* sm, int lane,
                                               f16x4 (&out)[2]) {
  const int j = lane % 16, g = lane / 16;
  const int src = (j % 4) * 16 + 4 * g + j / 4;  // lane (token 4 g + j / 4, group j % 4)
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
    sm->tr[hb][lane] = f16x4{(f16)x[4 * hb], (f16)x[4 * hb + 1], (f16)x[4 * hb + 2],
                             (f16)x[4 * hb + 3]};
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
    out[hb] = __builtin_bit_cast(
        f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) i16x4*)(
                       (__attribute__((address_space(3))) f16x4*)&sm->tr[hb][0] + src)));
}

// Forward substitution for (I + A) Y = I, A strictly lower triangular:
// y[e] (this lane's row i, column 4 g + e) receives -A[i][M] y_M for
// M = 0..14, y_M taken from lane M of the row.  One fused DPP multiply-add
// per column and step (the broadcast is the first source operand of
// v_fmac_f32_dpp); `an` holds -A[i][0..15].  The four columns of a step are
// independent, so each broadcast read comes at least three instructions
// after the write of the value it reads (DPP needs two), and the block
// opens with the two wait states its first reads need.
__device__ __forceinline__ void forward_sub(float (&y)[4], const f32x4 (&an)[4]) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %0, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
      : "v"(an[0][0]), "v"(an[0][1]), "v"(an[0][2]), "v"(an[0][3]), "v"(an[1][0]),
        "v"(an[1][1]), "v"(an[1][2]), "v"(an[1][3]), "v"(an[2][0]), "v"(an[2][1]),
        "v"(an[2][2]), "v"(an[2][3]), "v"(an[3][0]), "v"(an[3][1]), "v"(an[3][2]));
}

// From the intra-tile products summed over all slabs: the causal masks, the
// solve and T.  bt = beta of this lane's token (0 past the sequence end).
// Returns this lane's T image (lane (i, g): T[i][4 g + e]) and Aqk image (and,
// when the keys are not normalised here, T in float32 through tf and
// (I + A)^-1 through mf, when given).
// NORM: the keys are normalised here, rkt = 1/|k| of this lane's token and
// sm->rk holds it for every token of the tile.  A takes the norms of its row
// and column (the products were formed from the raw keys); tb receives
// Diag(1/|k|) T and tw Diag(1/|k|) T Diag(1/|k|), the factor that turns the raw
// keys into Diag(1/|k|) W, so that the state pass computes D' = Diag(1/|k|) D,
// the operand the raw keys Kb and Kc need, with no extra step.
template <bool NORM>
__device__ __forceinline__ void finish(f32x4 acc_a, f32x4 acc_q, float bt, float rkt,
                                       Scratch* sm, int lane, f16x4& tb, f16x4& aq, f16x4& tw,
                                       f32x4* tf = nullptr, f32x4* mf = nullptr) {
  const int t = lane % 16, lg = lane / 16;
  f32x4 rkj = {1.f, 1.f, 1.f, 1.f};  // 1/|k| of columns 4 g + r
  if constexpr (NORM) rkj = ds_read16(lds_addr(&sm->rk[4 * lg]));
  f32x4 am;  // -A; selects: masked entries may be huge products of e^-G
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 4 * lg + r;
    am[r] = (j < t) ? -bt * (NORM ? rkt * rkj[r] : 1.f) * acc_a[r] : 0.f;
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
  forward_sub(y, arow);
  if constexpr (NORM) {
    tb = f16x4{(f16)(y[0] * bj[0] * rkt), (f16)(y[1] * bj[1] * rkt), (f16)(y[2] * bj[2] * rkt),
               (f16)(y[3] * bj[3] * rkt)};
    tw = f16x4{(f16)(y[0] * bj[0] * rkt * rkj[0]), (f16)(y[1] * bj[1] * rkt * rkj[1]),
               (f16)(y[2] * bj[2] * rkt * rkj[2]), (f16)(y[3] * bj[3] * rkt * rkj[3])};
  } else {
    tb = f16x4{(f16)(y[0] * bj[0]), (f16)(y[1] * bj[1]), (f16)(y[2] * bj[2]), (f16)(y[3] * bj[3])};
    tw = tb;
    if (tf != nullptr) *tf = f32x4{y[0] * bj[0], y[1] * bj[1], y[2] * bj[2], y[3] * bj[3]};
    if (mf != nullptr) *mf = f32x4{y[0], y[1], y[2], y[3]};
  }
}

// W^T blocks 2s, 2s+1 = Kh^T T^T: lane (i, g) gets -W[i][32 s + 8 g + e],
// e < 4 in w[0], e >= 4 in w[1].
__device__ __forceinline__ void w_slab(const f16x4 (&khT)[2], f16x4 tb, f32x4 (&w)[2]) {
  w[0] = -mma16h(khT[0], tb, zero4());
  w[1] = -mma16h(khT[1], tb, zero4());
}

// ---------------------------------------------------------------- pairs

// LOGITS: g and beta come as logits (ga [rows, H, dk] bfloat16, beta the
// float32 logit of the write strength) and are formed here.
template <bool PACKED, bool LOGITS = false>
struct Args {
  const bf16_t* q;
  const bf16_t* k;
  const float* g;
  const float* beta;
  const bf16_t* ga;
  unsigned char* recs;  // records of the segment, [head][pair]
  Seqs<PACKED> seqs;    // where each sequence's tokens are; seqs.T = longest length
  int64_t H, BH;
  int64_t x0, nseg;     // first pair and pair count of the segment
};

// Position of a pair: head (b, h) and pair xl of the segment.
struct Pos {
  int64_t b, h, xl;
};

// Inputs of one slab of both tiles of a pair, and the rows they come from.
struct PairIn {
  SlabIn a, b;
  bf16x8 qa1, ka1, qb1, kb1;  // q and k of the odd slab that follows an even one
};

struct PairRows {
  int64_t a, b;  // element offsets of this lane's token rows (clamped into the sequence)
};

template <bool PACKED, bool LOGITS>
__device__ __forceinline__ PairRows pair_rows(const Args<PACKED, LOGITS>& a, const Pos& p,
                                              int lane) {
  const int64_t tok0 = (a.x0 + p.xl) * rec::kP + lane % 16;
  return PairRows{row_of(a.seqs, p.b, p.h, tok0, a.H),
                  row_of(a.seqs, p.b, p.h, tok0 + rec::kC, a.H)};
}

template <bool PACKED, bool LOGITS>
__device__ __forceinline__ void load_pair_slab(PairIn& x, const Args<PACKED, LOGITS>& a,
                                               const PairRows& r, int s, int lane) {
  load_slab<LOGITS>(x.a, x.qa1, x.ka1, a.q, a.k, a.g, a.ga, r.a, s, lane);
  load_slab<LOGITS>(x.b, x.qb1, x.kb1, a.q, a.k, a.g, a.ga, r.b, s, lane);
}

// Builds pair p of head (b, h) and stores its record.  On entry `cur` holds
// slab 0 of pair p (and the q and k of its slab 1); the next slab's inputs are always in flight while a slab
// is built, and on return `cur` holds slab 0 of pair `pn` (the wavefront's
// next pair, or any valid pair when there is none).
template <bool PACKED, bool LOGITS>
__device__ __forceinline__ void build_pair(const Args<PACKED, LOGITS>& a, const Pos& p,
                                           const Pos& pn, PairIn& cur, Scratch* sm, int lane) {
  const int t = lane % 16, lg = lane / 16;
  const int64_t tok0 = (a.x0 + p.xl) * rec::kP;
  const PairRows rows = pair_rows(a, p, lane), nrows = pair_rows(a, pn, lane);
  const int64_t T = a.seqs.len(p.b);  // tokens past it are identity (g = beta = k = q = 0)
  const bool fulla = tok0 + rec::kC <= T, fullb = tok0 + rec::kP <= T;
  const float lva = tok0 + t < T ? 1.f : 0.f;
  const float lvb = tok0 + rec::kC + t < T ? 1.f : 0.f;
  float betaa = a.beta[rows.a], betab = a.beta[rows.b];
  if constexpr (LOGITS) {
    betaa = fast_sigmoid(betaa);
    betab = fast_sigmoid(betab);
  }
  betaa *= lva;
  betab *= lvb;
  unsigned char* R = a.recs + ((p.b * a.H + p.h) * a.nseg + p.xl) * (int64_t)rec::kBytes;

  f32x4 aa = zero4(), qa = zero4(), ab = zero4(), qb = zero4(), qba = zero4(), mba = zero4();
  f16x4 khTa[4][2], khTb[4][2];
  float nqa = 0.f, nka = 0.f, nqb = 0.f, nkb = 0.f;  // this lane's part of |q|^2, |k|^2
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    PairIn nxt;
    if (s < 3)
      load_pair_slab(nxt, a, rows, s + 1, lane);
    else
      load_pair_slab(nxt, a, nrows, 0, lane);
    if (s % 2 == 0) {  // the odd slab's q and k came with this one's
      nxt.a.q = cur.qa1;
      nxt.a.k = cur.ka1;
      nxt.b.q = cur.qb1;
      nxt.b.k = cur.kb1;
    }
    // tile a: its values, then everything that needs only them
    SlabVals va;
    slab_vals_any<LOGITS>(fulla, cur.a, lva, va, aa, qa, nqa, nka);
    transpose_slab(va.kh, sm, lane, khTa[s]);
    const f16x8 kba = to_h8(va.kb);  // Kb_a, token-major
    *(f16x8*)(R + rec::kQa + s * 1024 + lane * 16) = to_h8(va.qh);
    if (t == 0) {
      const unsigned ea = lds_addr(&sm->en_a[32 * s + 8 * lg]);
      ds_write16(ea, f32x4{va.en[0], va.en[1], va.en[2], va.en[3]});
      ds_write16(ea + 16, f32x4{va.en[4], va.en[5], va.en[6], va.en[7]});
    }
    // tile b, and the cross terms
    SlabVals vb;
    slab_vals_any<LOGITS>(fullb, cur.b, lvb, vb, ab, qb, nqb, nkb);
    transpose_slab(vb.kh, sm, lane, khTb[s]);
    // Q_ba^T: lane (i, g) accumulates (Qh_b Kb_a^T)[i][4 g + r];
    // M = Kh_b Kb_a^T: lane (j, g) accumulates M[4 g + r][j]
    qba = mma32h(kba, to_h8(vb.qh), qba);
    mba = mma32h(to_h8(vb.kh), kba, mba);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = vb.qh[e] * va.en[e];
    *(f16x8*)(R + rec::kQb + s * 1024 + lane * 16) = to_h8(x);
    f16x4 kta[2], ktb[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = va.kb[e] * vb.en[e];
    transpose_slab(x, sm, lane, kta);
    transpose_slab(vb.kb, sm, lane, ktb);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      *(f16x8*)(R + rec::kKb + (2 * s + hb) * 1024 + lane * 16) = cat8(kta[hb], ktb[hb]);
    if (t == 15) {
      f32x4* ep = (f32x4*)(R + rec::kEn + (32 * s + 8 * lg) * 4);
      ep[0] = f32x4{va.en[0] * vb.en[0], va.en[1] * vb.en[1], va.en[2] * vb.en[2],
                    va.en[3] * vb.en[3]};
      ep[1] = f32x4{va.en[4] * vb.en[4], va.en[5] * vb.en[5], va.en[6] * vb.en[6],
                    va.en[7] * vb.en[7]};
    }
    cur = nxt;
  }

  // 1/|q|, 1/|k| per token: the four lanes of a token hold a quarter each
  float rqa = 1.f, rka = 1.f, rqb = 1.f, rkb = 1.f;
  if constexpr (LOGITS) {
    nqa += __shfl_xor(nqa, 16);
    nka += __shfl_xor(nka, 16);
    nqb += __shfl_xor(nqb, 16);
    nkb += __shfl_xor(nkb, 16);
    nqa += __shfl_xor(nqa, 32);
    nka += __shfl_xor(nka, 32);
    nqb += __shfl_xor(nqb, 32);
    nkb += __shfl_xor(nkb, 32);
    rqa = rsqrtf(fmaxf(nqa, 1e-24f));
    rqb = rsqrtf(fmaxf(nqb, 1e-24f));
    // A zero key (also every token past the sequence's end) writes nothing:
    // every use of its row of D' = Diag(1/|k|) D is multiplied by the key, so
    // the row is set to zero rather than to an overflowing 1e12 D.
    rka = nka > 0.f ? rsqrtf(fmaxf(nka, 1e-24f)) : 0.f;
    rkb = nkb > 0.f ? rsqrtf(fmaxf(nkb, 1e-24f)) : 0.f;
    // the largest 1/|k| of the pair: the state pass forms D' = Diag(1/|k|) D
    // and scales its float16 operands for it
    float rkm = fmaxf(rka, rkb);
    rkm = fmaxf(rkm, dpp<0x111, true>(rkm));
    rkm = fmaxf(rkm, dpp<0x112, true>(rkm));
    rkm = fmaxf(rkm, dpp<0x114, true>(rkm));
    rkm = fmaxf(rkm, dpp<0x118, true>(rkm));
    if (lg == 0) {
      float* nr = (float*)(R + rec::kNorm);
      nr[t] = rqa;
      nr[16 + t] = rqb;
      if (t == 15) nr[32] = rkm;
      ds_write4(lds_addr(&sm->rk[t]), rka);
    }
  }

  f16x4 ta, aqa, tb, aqb, twa, twb;
  finish<LOGITS>(aa, qa, betaa, rka, sm, lane, ta, aqa, twa);
  *(f16x4*)(R + rec::kTa + lane * 8) = ta;
  *(f16x4*)(R + rec::kAa + lane * 8) = aqa;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f32x4 w[2];
    w_slab(khTa[s], twa, w);
    *(f16x8*)(R + rec::kWa + s * 1024 + lane * 16) = cat8(to_h4(w[0]), to_h4(w[1]));
  }
  if constexpr (LOGITS) {
    if (lg == 0) ds_write4(lds_addr(&sm->rk[t]), rkb);
  }
  finish<LOGITS>(ab, qb, betab, rkb, sm, lane, tb, aqb, twb);
  // P = -W_b Kb_a^T = -T_b M, formed as (M^T T_b^T)^T: lane (i, g) gets P[i][4 g + r]
  // (with normalised keys, Diag(1/|k_b|) P Diag(|k_a|): it multiplies D_a' and gives D_b')
  const f32x4 pm = -mma16h(to_h4(mba), twb, zero4());
  *(f16x8*)(R + rec::kTbP + lane * 16) = cat8(tb, to_h4(pm));
  *(f16x8*)(R + rec::kQbaAb + lane * 16) = cat8(to_h4(qba), aqb);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f32x4 w[2];
    w_slab(khTb[s], twb, w);
    const unsigned ea = lds_addr(&sm->en_a[32 * s + 8 * lg]);
    f32x4 e0, e1;
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(e0), "=v"(e1)
        : "v"(ea)
        : "memory");
    *(f16x8*)(R + rec::kWb + s * 1024 + lane * 16) = cat8(to_h4(w[0] * e0), to_h4(w[1] * e1));
  }
}

// Pairs first, first + stride, ... < BH * nseg of one wavefront, numbered
// head-fastest (pair w is pair w / BH of head w % BH), so that the wavefronts
// working at one time read neighbouring heads of the same tokens, which are
// adjacent in memory.
template <bool PACKED, bool LOGITS>
__device__ __forceinline__ void build_range(const Args<PACKED, LOGITS>& a, int64_t first,
                                            int64_t stride, Scratch* sm, int lane) {
  const int64_t total = a.BH * a.nseg;
  if (first >= total) return;
  // w = xl BH + b H + h; the stride split the same way, advanced without divisions
  const int64_t B = a.BH / a.H;
  const int64_t sxl = stride / a.BH, sbh = stride - sxl * a.BH;
  const int64_t sb = sbh / a.H, sh = sbh - sb * a.H;
  auto advance = [&](Pos q) {
    q.b += sb;
    q.h += sh;
    q.xl += sxl;
    if (q.h >= a.H) {
      q.h -= a.H;
      ++q.b;
    }
    if (q.b >= B) {
      q.b -= B;
      ++q.xl;
    }
    return q;
  };
  Pos p;
  p.xl = first / a.BH;
  {
    const int64_t bh = first - p.xl * a.BH;
    p.b = bh / a.H;
    p.h = bh - p.b * a.H;
  }
  PairIn cur;
  load_pair_slab(cur, a, pair_rows(a, p, lane), 0, lane);
  for (int64_t w = first; w < total; w += stride) {
    const Pos pn = w + stride < total ? advance(p) : p;  // past the last pair: reload this one
    // a pair past the end of its sequence is never read: no record for it
    if ((a.x0 + p.xl) * rec::kP < a.seqs.len(p.b))
      build_pair(a, p, pn, cur, sm, lane);
    else
      load_pair_slab(cur, a, pair_rows(a, pn, lane), 0, lane);
    p = pn;
  }
}

}  // namespace tile
}  // namespace kda
