// Backward of the KDA layer core on the matrix cores (bfloat16 io,
// dk = dv = 128), chunkwise in 16-token tiles.
//
// The forward over a tile of C = 16 tokens with start state S (dk x dv, rows
// are key channels) and G the in-tile cumulative sum of g ("Kimi K3:
// Engineering a 2.8 Trillion Parameter Frontier", section "Dimension 1":
// 16-token tiles whose cumulative log-decay stays in (-80, 0)):
//   Kh = k e^G, Kc = k e^-G, Qh = q e^G, Kb = k e^(G_15 - G), E = e^G_15
//   P = Kh Kc^T, A = strict_lower(Diag(beta) P), M = (I + A)^-1, T = M Diag(beta)
//   Aqk = lower(Qh Kc^T)
//   X = V - Kh S,  Delta = T X,  O = scale (Qh S + Aqk Delta),  S' = Diag(E) S + Kb^T Delta
// The pages give no backward pass; these are the plain gradients of a loss
// given dO for every token and dS_T for the final state.  With dO' = scale dO
// and dS' the adjoint of the tile's end state, the adjoint of the tile is
//   dDelta = Aqk^T dO' + Kb dS'          dX = T^T dDelta          dV = dX
//   dS     = Diag(E) dS' + Qh^T dO' - Kh^T dX                     (the previous tile's dS')
//   Y1 = dO' S^T,  Y2 = dX S^T,  Y3 = Delta dS'^T,  dE = rowsum(S * dS')
//   dT = dDelta X^T,  dAqk = lower(dO' Delta^T)
// and, per tile from those (float32):
//   dM = dT Diag(beta),  dbeta_j = sum_i dT_ij M_ij + sum_k dA_jk P_jk,
//   dA = strict_lower(-M^T dM M^T),  dP = Diag(beta) dA
//   dq  = e^G (Y1 + dAqk Kc)
//   dk  = e^G (-Y2 + dP Kc) + e^-G (dAqk^T Qh + dP^T Kh) + e^(G_15 - G) Y3
//   dG  = k (dk_h - dk_c - dk_b) + q dq  (the three parts of dk), dG_15 += sum_rows k dk_b + dE E
//   dg  = reverse cumulative sum of dG over the tile.
// Every product with a factor e^-G (up to e^80) is formed in float32 with the
// masked (causal) entries only, so each term carries e^(G_i - G_j) <= 1.
//
// The pass runs as five steps on the caller's stream.  (Running step 1 on a
// second stream beside steps 2 and 3 saved about 0.1 ms of 1.8 at B=2, H=32,
// T=4096, but the extra hardware queue slowed later kernels of the process:
// the decode step by 4 %.)
//   1. the matrix-core forward, state only, with the state kept every 64
//      tokens (a block of four tiles);
//   2. kda_bwd_rec_kernel: per tile and in parallel, the operands of the two
//      chains (the record below), as float16 matrix-core operand images;
//   3. kda_bwd_chain_kernel: per head (its value columns split over four
//      workgroups), the tiles last to first, dS' resident in matrix-core
//      accumulators; it keeps dS' at the end of every block and returns dS_0;
//   4. kda_bwd_block_kernel: per head and block, in parallel: for each tile
//      of the block (last to first) the forward state recomputed from the
//      block's start state, the tile's adjoint step, the products Y1, Y2, Y3,
//      dE, dT, dAqk over all value columns (float32, summed in a fixed order,
//      so the pass is deterministic) and dV;
//   5. kda_bwd_fin_kernel: per tile, the float32 part above (P and M come
//      from the record builder).
// The state and its adjoint enter the products as float16 with a power-of-two
// scale per wavefront (scale_shift), as in the forward's state pass; the
// method is linear in the forward values and in the adjoint values, and each
// wavefront divides what it contributes by both scales.
#include "kda_chunk_rec.h"
#include "kda_chunk_tile.h"
#include "kda_launch.h"

namespace kda {
namespace bwd {

constexpr int kC = 16, kDK = 128, kDV = 128;
constexpr int64_t kDD = (int64_t)kDK * kDV;
constexpr int kBlkTiles = 4;                 // tiles per block
constexpr int kBlkTok = kBlkTiles * kC;      // 64 tokens

// Record of one tile (float16 operand images of one 64-lane wavefront,
// lane l = 16 g + c; chan(b, p) is the key channel of row p of state block b):
constexpr int kKh = 0;        // [slab < 4][lane][8]  lane (t, g): Kh[t][32 s + 8 g + e]
constexpr int kKb = 4096;     // [slab < 4][lane][8]  lane (t, g): Kb[t][32 s + 8 g + e]
constexpr int kQK = 8192;     // [block < 8][lane][8] lane (c, g): Qh[4 g + e][chan(b, c)] (e < 4),
                              //                      -Kh[4 g + e - 4][chan(b, c)] (e >= 4)
constexpr int kKbC = 16384;   // [block < 8][lane][4] lane (c, g): Kb[4 g + e][chan(b, c)]
constexpr int kT = 20480;     // [lane][4]            lane (i, g): T[i][4 g + e]
constexpr int kTt = 20992;    // [lane][4]            T[4 g + e][i]
constexpr int kAqkT = 21504;  // [lane][4]            Aqk[4 g + e][i]
constexpr int kE = 22016;     // [128] f32            E per key channel
constexpr int kTlo = 22528;   // [lane][4]            T - kT (the float16 rounding of T)
// the float16 roundings (x - float16(x)) of two of the adjoint step's operands
constexpr int kTtlo = 23040;  // [lane][4]            of kTt
constexpr int kAqkTlo = 23552;  // [lane][4]          of kAqkT
constexpr int kRecBytes = 24576;  // a whole number of 1 KB blocks

// Products of one tile (float32), from the block kernel to the finishing kernel:
// Y1, Y2, Y3 are [16 tokens][128 channels] each, in accumulator order: token t,
// channel 16 w + c at 256 w + 4 (c + 16 (t / 4)) + t % 4.
constexpr int kY1 = 0, kY2 = 2048, kY3 = 4096;
constexpr int kDE = 6144;                       // [128]
constexpr int kDT = 6272, kDAqk = 6528;         // [16][16] each
constexpr int kYFloats = 6784;

__device__ __forceinline__ f16x8 lo8(f16x4 x) {
  return f16x8{x[0], x[1], x[2], x[3], (f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
}
__device__ __forceinline__ f16x8 ld16h(const unsigned char* p) { return *(const f16x8*)p; }
__device__ __forceinline__ f16x4 ld8h(const unsigned char* p) { return *(const f16x4*)p; }

// X transposed: lane (i, g) holds X[i][4 g + e] on entry and X[4 g + e][i] on return.
__device__ __forceinline__ f16x4 transpose16(f16x4 x, tile::Scratch* sm, int lane) {
  f16* buf = (f16*)&sm->tr[0][0];
  const int i = lane % 16, g = lane / 16;
  wave_lds_sync();
  *(f16x4*)(buf + i * 16 + 4 * g) = x;
  wave_lds_sync();
  f16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = buf[(4 * g + e) * 16 + i];
  wave_lds_sync();
  return y;
}

// ------------------------------------------------------------------ 2. records
struct RecArgs {
  const bf16_t* q;
  const bf16_t* k;
  const float* g;
  const float* beta;
  unsigned char* recs;  // [B H][nt][kRecBytes]
  float* pm;            // [B H][nt][2][16][16]: P = Kh Kc^T and M = (I + A)^-1, float32
  int64_t B, T, H, nt;
};

// The record of tile x of head bh, built by one wavefront.  Lane (t, g) holds
// token t and, per 32-channel slab s, channels 32 s + 8 g + 0..7.
__device__ __forceinline__ void build_tile(const RecArgs& a, int64_t bh, int64_t x,
                                           tile::Scratch* sm, int lane) {
  const int t = lane % 16, lg = lane / 16;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t tok0 = x * kC, tok = tok0 + t;
  const bool full = tok0 + kC <= a.T;
  const float lv = tok < a.T ? 1.f : 0.f;  // tokens past the end: identity tokens
  const int64_t row = (b * a.T + (tok < a.T ? tok : a.T - 1)) * a.H + h;
  const float bt = a.beta[row] * lv;
  unsigned char* R = a.recs + (bh * a.nt + x) * (int64_t)kRecBytes;
  f32x4 acc_a = zero4(), acc_q = zero4();
  float nq = 0.f, nk = 0.f;
  tile::SlabIn in;
  bf16x8 q1, k1;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 qn, kn;
    tile::load_slab<false>(in, qn, kn, a.q, a.k, a.g, nullptr, row, s, lane);
    if (s % 2 == 0) {
      q1 = qn;
      k1 = kn;
    } else {
      in.q = q1;
      in.k = k1;
    }
    tile::SlabVals v;
    tile::slab_vals_any<false>(full, in, lv, v, acc_a, acc_q, nq, nk);
    *(f16x8*)(R + kKh + s * 1024 + lane * 16) = tile::to_h8(v.kh);
    *(f16x8*)(R + kKb + s * 1024 + lane * 16) = tile::to_h8(v.kb);
    f16x4 kbT[2], qT[2], khT[2];
    tile::transpose_slab(v.kb, sm, lane, kbT);
    tile::transpose_slab(v.qh, sm, lane, qT);
    tile::transpose_slab(v.kh, sm, lane, khT);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      *(f16x4*)(R + kKbC + (2 * s + hb) * 512 + lane * 8) = kbT[hb];
      *(f16x8*)(R + kQK + (2 * s + hb) * 1024 + lane * 16) = cat8(qT[hb], -khT[hb]);
    }
    if (t == 15) {
      f32x4* ep = (f32x4*)(R + kE + (32 * s + 8 * lg) * 4);
      ep[0] = f32x4{v.en[0], v.en[1], v.en[2], v.en[3]};
      ep[1] = f32x4{v.en[4], v.en[5], v.en[6], v.en[7]};
    }
  }
  f16x4 tb, aq, tw;
  f32x4 tf, mf;
  tile::finish<false>(acc_a, acc_q, bt, 1.f, sm, lane, tb, aq, tw, &tf, &mf);
  {  // lane (i, g) holds row i, columns 4 g .. 4 g + 3 of P and of M
    float* pm = a.pm + (bh * a.nt + x) * 512 + t * 16 + 4 * lg;
    *(f32x4*)pm = acc_a;
    *(f32x4*)(pm + 256) = mf;
  }
  const f16x4 tlo = to_h4(tf - f32x4{(float)tb[0], (float)tb[1], (float)tb[2], (float)tb[3]});
  f32x4 aqlo;  // Aqk - float16(Aqk), Aqk = lower(Qh Kc^T) as finish() masks it
#pragma unroll
  for (int r = 0; r < 4; ++r) aqlo[r] = (4 * lg + r <= t ? acc_q[r] : 0.f) - (float)aq[r];
  *(f16x4*)(R + kT + lane * 8) = tb;
  *(f16x4*)(R + kTlo + lane * 8) = tlo;
  *(f16x4*)(R + kTt + lane * 8) = transpose16(tb, sm, lane);
  *(f16x4*)(R + kTtlo + lane * 8) = transpose16(tlo, sm, lane);
  *(f16x4*)(R + kAqkT + lane * 8) = transpose16(aq, sm, lane);
  *(f16x4*)(R + kAqkTlo + lane * 8) = transpose16(to_h4(aqlo), sm, lane);
}

__global__ void __launch_bounds__(256) kda_bwd_rec_kernel(RecArgs a) {
  __shared__ tile::Scratch scratch[4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int64_t total = a.B * a.H * a.nt;
  for (int64_t w = (int64_t)blockIdx.x * 4 + wave; w < total; w += (int64_t)gridDim.x * 4)
    build_tile(a, w % (a.B * a.H), w / (a.B * a.H), &scratch[wave], lane);
}

// --------------------------------------------- scale of a wavefront's operands
// The wavefront holds sigma Z (sigma = 2^sh) in f32 accumulators Z[8] and forms
// sigma W from w (16 values per lane); returns the rescale already applied.
struct Scale {
  int sh = 0;
  float sig = 1.f, isig = 1.f;
};

// Whether scale_shift() keeps the scale, given each lane's largest magnitude
// m (>= 0): the wavefront's largest lies in [2^kLoExp, 2^(kHiExp + 1)), or
// every value is zero.  Three lane votes instead of a reduction across lanes.
__device__ __forceinline__ bool scale_kept(float m) {
  static_assert(kLoExp >= 0 && kHiExp + 1 < 31, "bounds as integers");
  constexpr float kLo = (float)(1 << kLoExp), kHi = (float)(1 << (kHiExp + 1));
  if (__builtin_amdgcn_ballot_w64(m >= kHi) != 0) return false;
  return __builtin_amdgcn_ballot_w64(m >= kLo) != 0 || __builtin_amdgcn_ballot_w64(m > 0.f) == 0;
}

// Chooses the scale for accumulators z and incoming values w (unscaled) of a
// wavefront that holds N 16-column blocks (one scale for all), rescales z
// when the scale moves, and sets ws[n] = sigma w[n].
template <int N>
__device__ __forceinline__ void rescale_n(Scale& sc, f32x4 (&z)[N][8], const f32x4 (&w)[N],
                                          f32x4 (&ws)[N]) {
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    ws[n] = w[n] * sc.sig;
#pragma unroll
    for (int r = 0; r < 4; ++r) m0 = fmaxf(m0, fabsf(ws[n][r]));
#pragma unroll
    for (int kb = 0; kb < 8; kb += 2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m0 = fmaxf(m0, fabsf(z[n][kb][r]));
        m1 = fmaxf(m1, fabsf(z[n][kb + 1][r]));
      }
  }
  if (scale_kept(fmaxf(m0, m1))) return;
  const int em = exp_of(wave_max_nonneg(fmaxf(m0, m1)));
  if (scale_shift(em, sc.sh) != 0) {  // rare: measured again with w unscaled
    float mz = 0.f, mw = 0.f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mw = fmaxf(mw, fabsf(w[n][r]));
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mz = fmaxf(mz, fabsf(z[n][kb][r]));
    }
    const int ez = exp_of(wave_max_nonneg(mz));
    int ew = exp_of(wave_max_nonneg(mw));
    ew = ew == kNoExp ? kNoExp : ew + sc.sh;
    const int d = scale_shift(ez > ew ? ez : ew, sc.sh);
    if (d != 0) {
      const float f = exp2i(d);
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) z[n][kb] *= f;
      sc.sh += d;
      sc.sig = exp2i(sc.sh);
      sc.isig = exp2i(-sc.sh);
    }
#pragma unroll
    for (int n = 0; n < N; ++n) ws[n] = w[n] * sc.sig;
  }
}

// rescale_n() for one block: returns sigma w.
__device__ __forceinline__ f32x4 rescale(Scale& sc, f32x4 (&z)[8], f32x4 w) {
  f32x4(&zn)[1][8] = *reinterpret_cast<f32x4(*)[1][8]>(&z);
  const f32x4 wn[1] = {w};
  f32x4 ws[1];
  rescale_n<1>(sc, zn, wn, ws);
  return ws[0];
}

// The k-operand image of a wavefront's 16 value columns of a [dk, dv] state
// in accumulators (lane (c, g) of block kb: rows chan(kb, 4 g + r), column c).
__device__ __forceinline__ void state_op(const f32x4 (&z)[8], f16x8 (&op)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) op[s] = cat8(to_h4(z[2 * s]), to_h4(z[2 * s + 1]));
}

// The value columns of wavefront w: column index c (lane (c, g) of an
// accumulator) is column 32 (w / 2) + 8 (c / 4) + 4 (w % 2) + c % 4, the
// forward's state pass numbering, so that its checkpoints in accumulator
// order load here as they are; a lane (t, g) of a row operand holds the four
// adjacent columns of indices 4 g .. 4 g + 3, from row_col(w, g) on.
__device__ __forceinline__ int acc_col(int wave, int c) {
  return 32 * (wave / 2) + 8 * (c / 4) + 4 * (wave % 2) + c % 4;
}
__device__ __forceinline__ int row_col(int wave, int g) {
  return 32 * (wave / 2) + 8 * g + 4 * (wave % 2);
}

// A wavefront's columns of a [dk][dv] row-major state (caller buffers).
__device__ __forceinline__ void load_state(f32x4 (&z)[8], const float* p, int wave, int lane) {
  const int lc = lane % 16, lg = lane / 16;
  if (p == nullptr) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) z[kb] = zero4();
    return;
  }
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) z[kb][r] = p[rec::chan(kb, 4 * lg + r) * kDV + acc_col(wave, lc)];
}

__device__ __forceinline__ void store_state(float* p, const f32x4 (&z)[8], float f, int wave,
                                            int lane) {
  const int lc = lane % 16, lg = lane / 16;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) p[rec::chan(kb, 4 * lg + r) * kDV + acc_col(wave, lc)] = z[kb][r] * f;
}

// A state held by the eight wavefronts in accumulator order, for buffers that
// only these kernels read: wavefront w's block kb at [w][kb][lane][4], so
// every lane moves 16 contiguous bytes (a [dk][dv] row-major layout takes
// four times as many narrower accesses).
__device__ __forceinline__ void store_frag(float* p, const f32x4 (&z)[8], float f, int wave,
                                           int lane) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) *(f32x4*)(p + 2048 * wave + 4 * (64 * kb + lane)) = z[kb] * f;
}

__device__ __forceinline__ void load_frag(f32x4 (&z)[8], const float* p, int wave, int lane) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) z[kb] = *(const f32x4*)(p + 2048 * wave + 4 * (64 * kb + lane));
}

// Selection matrix for moving 16 token rows into the k-operand layout:
// B[k = 4 g + e][c] = (k == c).
__device__ __forceinline__ bf16x4 ident_op(int lane) {
  bf16x4 id;
#pragma unroll
  for (int e = 0; e < 4; ++e) id[e] = (bf16_t)((4 * (lane / 16) + e == lane % 16) ? 1.f : 0.f);
  return id;
}

// -------------------------------------------------------------- 3. the chain
struct ChainArgs {
  const unsigned char* recs;
  const bf16_t* dout;
  const float* dsf;  // [B H][dk][dv] or NULL
  float* ds_blk;     // [B H][nblk] states in accumulator order: dS' at the end of every block
  float* ds0;        // [B H][dk][dv] or NULL
  int64_t B, T, H, nt, nblk;
  float scale;
};

// The value columns of the adjoint recurrence are independent of each other
// (every product acts on them column by column), so each head's walk is split
// over kChainSplit workgroups of 128 / kChainSplit columns.
constexpr int kChainSplit = 4;
constexpr int kChainCols = kDV / kChainSplit;
constexpr int kRowBytes = kChainCols * 2;  // a dO row of one workgroup's columns
// The chain's part of a tile in an LDS slot, in 1 KB blocks: record blocks
// 4 .. 15 (Kb, then [Qh^T | -Kh^T]), record blocks 20 and 21 (T, T^T, Aqk^T,
// E), then the workgroup's columns of the tile's 16 dO rows.
constexpr int kSlotKb = 0, kSlotQK = 4096, kSlotTt = 12288 + (kTt - 20480),
              kSlotAqkT = 12288 + (kAqkT - 20480), kSlotE = 12288 + (kE - 20480), kSlotDO = 14336;
constexpr int kChainDOBlocks = 16 * kRowBytes / 1024;
constexpr int kChainBlocks = 14 + kChainDOBlocks, kChainSlot = kChainBlocks * 1024;
constexpr int kChainRing = 8;     // slots: seven tiles in flight ahead of the one in use
constexpr int kChainNcb = 1;      // 16-column blocks per compute wavefront
constexpr int kChainWaves = kChainCols / 16 / kChainNcb;  // compute wavefronts
constexpr int kChainLoaders = 3;  // loader wavefronts
constexpr int kChainPer = kChainBlocks / kChainLoaders;  // loads per loader wavefront per tile
static_assert(kChainDOBlocks * 1024 == 16 * kRowBytes && kChainWaves * kChainNcb * 16 == kChainCols,
              "whole dO blocks and column blocks");
static_assert(kKb == 4096 && kQK == 8192 && kKbC == 16384 && kT == 20480 && kTlo == 22528,
              "the chain's record blocks");
static_assert(kChainPer * kChainLoaders == kChainBlocks, "whole loads per loader wavefront");
static_assert((kChainRing - 1) * kChainPer <= 63, "loads in flight per wavefront exceed vmcnt");

// z * E for rows 4 g + r of state block KB (r < 4), from the two values per
// lane described at the chain's E read: four multiplies whose first source
// is lane 2 KB + r / 2 of the DPP row (row_newbcast), so the broadcast costs
// no instruction of its own.  The s_nops cover the wait states of a DPP
// source after a vector-ALU write of it and of a matrix-core operand after
// the multiplies that write it (the compiler does not see into the block).
template <int KB>
__device__ __forceinline__ f32x4 decay_rows(f32x2 e2, f32x4 z) {
  f32x4 y;
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %4, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %5, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %4, %9 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %5, %10 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])
      : "v"(e2[0]), "v"(e2[1]), "v"(z[0]), "v"(z[1]), "i"(2 * KB), "v"(z[2]), "v"(z[3]),
        "i"(2 * KB + 1));
  return y;
}

// f(integral_constant<int, KB>) for KB = 0 .. 7.
template <int KB = 0, class F>
__device__ __forceinline__ void unroll8(F&& f) {
  if constexpr (KB < 8) {
    f(std::integral_constant<int, KB>{});
    unroll8<KB + 1>(f);
  }
}

// s_waitcnt with vmcnt = N, the other counters left alone (gfx9 encoding).
constexpr unsigned vmcnt_only(int n) {
  return (unsigned)((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// kChainSplit workgroups per (b, h), each on its own kChainCols value
// columns: its compute wavefronts (kChainNcb 16-column blocks each) walk the
// tiles last to first, while its loader wavefronts keep the next seven tiles'
// record parts and dO columns streaming into a ring of LDS slots with
// direct-to-LDS loads.  One barrier per tile: after it, the tile just used
// frees its slot and the next tile is in LDS.  The workgroups of one head
// get block indices equal modulo 8, which places them on one XCD (blocks are
// dealt to the XCDs in turn), so that the head's records are read from HBM
// once and from that XCD's L2 by the others (a matter of speed only: the
// results do not depend on where the blocks run).
__global__ void __launch_bounds__(64 * (kChainWaves + kChainLoaders), 1)
kda_bwd_chain_kernel(ChainArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kChainRing][kChainSlot];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, lc = lane % 16, lg = lane / 16;
  // block -> (head, part): groups of 8 heads take 8 kChainSplit consecutive
  // blocks, head j of a group at blocks j + 8 part (a last, smaller group
  // when B H is not a multiple of 8 takes its blocks in head order)
  const int64_t BH = a.B * a.H, grp = blockIdx.x / (8 * kChainSplit);
  const int64_t in_grp = blockIdx.x % (8 * kChainSplit);
  int64_t bh;
  int part;
  if ((grp + 1) * 8 <= BH) {
    bh = grp * 8 + in_grp % 8;
    part = (int)(in_grp / 8);
  } else {
    bh = grp * 8 + in_grp / kChainSplit;
    part = (int)(in_grp % kChainSplit);
  }
  const int64_t b = bh / a.H, h = bh % a.H;
  const int cg0 = part * (kChainCols / 16) + wave * kChainNcb;  // first 16-column group

  if (wave >= kChainWaves) {  // -------------------------------- loader waves
    const int lw = wave - kChainWaves;
    auto issue = [&](int64_t x) {
      const unsigned char* R = a.recs + (bh * a.nt + x) * (int64_t)kRecBytes;
      unsigned char* slot = lds[x % kChainRing];
#pragma unroll
      for (int i = 0; i < kChainPer; ++i) {
        const int blk = lw + kChainLoaders * i;
        const unsigned char* src;
        if (blk < 12) {
          src = R + 4096 + blk * 1024 + lane * 16;
        } else if (blk < 14) {
          src = R + 20480 + (blk - 12) * 1024 + lane * 16;
        } else {  // 16-byte chunks of dO rows, kRowBytes / 16 per row
          constexpr int kLanesPerRow = kRowBytes / 16, kRowsPerBlock = 64 / kLanesPerRow;
          int64_t tok = x * kC + (blk - 14) * kRowsPerBlock + lane / kLanesPerRow;
          tok = tok < a.T ? tok : a.T - 1;
          src = (const unsigned char*)(a.dout + ((b * a.T + tok) * a.H + h) * kDV +
                                       part * kChainCols + (lane % kLanesPerRow) * 8);
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(slot +
                                                                                   blk * 1024),
                                         16, 0, 0);
      }
    };
    // tiles nt - 1 .. nt - 7 in flight, then wait for the first
    for (int64_t i = 0; i < kChainRing - 1 && i < a.nt; ++i) issue(a.nt - 1 - i);
    if (a.nt >= kChainRing - 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_only((kChainRing - 2) * kChainPer));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    // A bare barrier: these waves touch LDS only through their direct-to-LDS
    // loads, whose completion the vmcnt waits above establish; a fence here
    // would also wait for the tiles still in flight.
    __builtin_amdgcn_s_barrier();
    for (int64_t x = a.nt - 1; x >= 0; --x) {
      // the slot of tile x + 1 is free: it takes tile x - 7
      if (x - (kChainRing - 1) >= 0) issue(x - (kChainRing - 1));
      // tile x - 1 in LDS: the loads issued after it are those of tiles
      // x - 2 .. max(x - 7, 0)
      if (x - 1 >= kChainRing - 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_only((kChainRing - 2) * kChainPer));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    return;
  }

  // --------------------------------------------------------- compute waves
  // The adjoint quantities are held in units of scale / sigma, so that dO
  // (bfloat16) enters the float16 operands exactly: sigma dO instead of a
  // rounded sigma scale dO.  so = scale, or 1 with dO dropped when scale = 0.
  // Column block n of this wavefront is 16-column group cg0 + n.
  const float so = a.scale != 0.f ? a.scale : 1.f, dmul = a.scale != 0.f ? 1.f : 0.f;
  f32x4 dS[kChainNcb][8];
#pragma unroll
  for (int n = 0; n < kChainNcb; ++n) {
    load_state(dS[n], a.dsf != nullptr ? a.dsf + bh * kDD : nullptr, cg0 + n, lane);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) dS[n][kb] *= 1.f / so;
  }
  Scale sc;
  const bf16x4 ident = ident_op(lane);
  // dS' at the end of block blk (the state entering its last tile)
  auto store_ds = [&](int64_t blk) {
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n)
      store_frag(a.ds_blk + (bh * a.nblk + blk) * kDD, dS[n], so * sc.isig, cg0 + n, lane);
  };
  store_ds(a.nblk - 1);
  lds_barrier();  // tile nt - 1 is in LDS
  for (int64_t x = a.nt - 1; x >= 0; --x) {
    const unsigned char* R = lds[x % kChainRing];
    // All of the tile's operand reads first (16 with one column block: the
    // first is waited for at the LDS counter's largest value, 15), those of
    // the first products first: their latency is then exposed once, and the
    // state update's operands arrive during the dependent chain.
    bf16x4 dor[kChainNcb];  // dO rows: lane (c, g): dO[c][4 g + e] of block n's columns
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n)
      dor[n] = *(const bf16x4*)(R + kSlotDO + lc * kRowBytes +
                                (row_col(cg0 + n, lg) - part * kChainCols) * 2);
    f16x8 kbo[4], qk[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) kbo[s] = ld16h(R + kSlotKb + s * 1024 + lane * 16);
    const f16x8 aq = lo8(ld8h(R + kSlotAqkT + lane * 8)), tt = lo8(ld8h(R + kSlotTt + lane * 8));
    // E of the channels of row group g, two per lane: lane (c, g) holds
    // E[32 (c / 4) + 8 g + 2 (c % 4) + {0, 1}], so that the value for row
    // 4 g + r of block kb sits in lane 2 kb + r / 2 of the same DPP row
    const f32x2 e2 = *(const f32x2*)(R + kSlotE + 4 * (32 * (lc / 4) + 8 * lg + 2 * (lc % 4)));
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qk[kb] = ld16h(R + kSlotQK + kb * 1024 + lane * 16);
    // keep the reads here: neither the compiler's code motion nor its
    // scheduler may move them down to their uses
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // dO in the k-operand layout: lane (c, g): dO[4 g + r][column index c]
    f32x4 dof[kChainNcb], dos[kChainNcb];
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n) dof[n] = mma16b(dor[n], ident, zero4()) * dmul;
    rescale_n<kChainNcb>(sc, dS, dof, dos);
    f16x4 do16[kChainNcb];
    f16x8 sop[kChainNcb][4];
    f32x4 dd[kChainNcb];
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n) {
      do16[n] = to_h4(dos[n]);
      state_op(dS[n], sop[n]);
      dd[n] = zero4();
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int n = 0; n < kChainNcb; ++n) dd[n] = mma32h(kbo[s], sop[n][s], dd[n]);
    f16x8 bop[kChainNcb];
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n) {
      dd[n] = mma32h(aq, cat8(do16[n], do16[n]), dd[n]);
      const f16x4 dd16 = to_h4(dd[n]);
      const f32x4 dx = mma32h(tt, cat8(dd16, dd16), zero4());
      bop[n] = cat8(do16[n], to_h4(dx));
    }
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n) {
      dS[n][0] = mma32h(qk[0], bop[n], decay_rows<0>(e2, dS[n][0]));
      dS[n][1] = mma32h(qk[1], bop[n], decay_rows<1>(e2, dS[n][1]));
      dS[n][2] = mma32h(qk[2], bop[n], decay_rows<2>(e2, dS[n][2]));
      dS[n][3] = mma32h(qk[3], bop[n], decay_rows<3>(e2, dS[n][3]));
      dS[n][4] = mma32h(qk[4], bop[n], decay_rows<4>(e2, dS[n][4]));
      dS[n][5] = mma32h(qk[5], bop[n], decay_rows<5>(e2, dS[n][5]));
      dS[n][6] = mma32h(qk[6], bop[n], decay_rows<6>(e2, dS[n][6]));
      dS[n][7] = mma32h(qk[7], bop[n], decay_rows<7>(e2, dS[n][7]));
    }
    // dS' entering tile x - 1, the last tile of block x / kBlkTiles - 1
    if (x > 0 && x % kBlkTiles == 0) store_ds(x / kBlkTiles - 1);
    lds_barrier();
  }
  if (a.ds0 != nullptr) {
#pragma unroll
    for (int n = 0; n < kChainNcb; ++n)
      store_state(a.ds0 + bh * kDD, dS[n], so * sc.isig, cg0 + n, lane);
  }
}

// ---------------------------------------------------------- 4. block products
struct BlockArgs {
  const unsigned char* recs;
  const bf16_t* v;
  const bf16_t* dout;
  const float* s0;      // [B H][dk][dv] or NULL
  const float* s_ck;    // [B][T / 64][H] states: the state after every 64 tokens
  bool ck_rowmajor;     // s_ck [dk][dv] row-major (the caller's); else in accumulator order
  const float* ds_blk;  // [B H][nblk] states in accumulator order
  bf16_t* dv;
  float* ybuf;          // [B H][nt][kYFloats]
  int64_t B, T, H, nt, nblk, nck;
  float scale;
};

// Staging of one tile's operands for the products over value columns, every
// value unscaled float32, chunk w = the 16 value columns of wavefront w.
// The record parts the forward steps use, per tile of the block (shared by
// the eight wavefronts): Kh, Kb^T, T, T - float16(T), E.
constexpr int kFwKh = 0, kFwKbC = 4096, kFwT = 8192, kFwTlo = 8704, kFwE = 9216;
constexpr int kFwBytes = 9728;
// The staged operands are bfloat16 pairs: h = bfloat16(x) and l = bfloat16(x - h)
// (x = h + l to about 2^-17 relative); a product takes hh + hl + lh.
struct BlockSmem {
  bf16_t sth[8][kDK * 16], stl[8][kDK * 16];  // chunk w of S_t, then of dS', row-major [c][j]
  bf16_t sxh[8][5][kC * 16], sxl[8][5][kC * 16];  // chunk w of dO', dX, Delta, dDelta, X: [t][j]
  float dep[8][kDK];                          // chunk w's part of dE
  unsigned char fw[kBlkTiles][kFwBytes];
};

// One exchange of a reduce-scatter over the 16 lanes of a DPP row: the lane
// keeps half BIT of its N values (the lower half when its lane bit is 0) and
// adds the same half from its partner (CTRL pairs lanes that differ in that bit).
template <int CTRL, int N>
__device__ __forceinline__ void rs_half(const float* v, float* out, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float own = upper ? v[N / 2 + i] : v[i], snd = upper ? v[i] : v[N / 2 + i];
    out[i] = own + dpp<CTRL, false>(snd);
  }
}

// Sums of 32 values per lane over the 16 lanes of each DPP row: lane c of the
// row returns those of indices 2 c and 2 c + 1.  Partners in turn: the row
// mirrored (lane bit 3 differs), each half mirrored (bit 2), quad_perm
// [2, 3, 0, 1] (bit 1) and [1, 0, 3, 2] (bit 0); 90 instructions instead of
// 32 prefix sums of 4 steps each.
__device__ __forceinline__ f32x2 row_reduce_scatter32(const float (&p)[32], int c) {
  float a[16], b[8], q[4], d[2];
  rs_half<0x140, 32>(p, a, (c & 8) != 0);
  rs_half<0x141, 16>(a, b, (c & 4) != 0);
  rs_half<0x4E, 8>(b, q, (c & 2) != 0);
  rs_half<0xB1, 4>(q, d, (c & 1) != 0);
  return f32x2{d[0], d[1]};
}

__device__ __forceinline__ f32x4 to_f4(f16x4 x) {
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// A token row of v or dO (bfloat16) as the A operand of the selection-matrix
// product: lane (t, g) the four columns from c0 on of token t, zero past the end.
__device__ __forceinline__ bf16x4 token_row4(const bf16_t* p, int64_t tok, int64_t T, int64_t b,
                                             int64_t h, int64_t H, int c0) {
  bf16x4 r{};
  if (tok < T) r = *(const bf16x4*)(p + ((b * T + tok) * H + h) * kDV + c0);
  return r;
}

__device__ __forceinline__ f32x4 mma32b(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pairs x = h + l with h = bfloat16(x), l = bfloat16(x - h) (x = h + l to
// about 2^-17 relative), two values per conversion.
__device__ __forceinline__ void split2(f32x2 x, bf16x2& h, bf16x2& l) {
  h = __builtin_convertvector(x, bf16x2);
  l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2), bf16x2);
}

// This wavefront's accumulators (lane (c, g) of block kb: rows chan(kb, 4 g + r),
// column c) to row-major [channel][c] bfloat16 pairs, as held (the caller
// moves the wavefront's scale onto the other operand of each product; a
// power-of-two factor commutes with the bfloat16 rounding).
__device__ __forceinline__ void stage_state(bf16_t* sh, bf16_t* sl, const f32x4 (&z)[8], int lane) {
  const int lc = lane % 16, lg = lane / 16;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
      bf16x2 h, l;
      split2(f32x2{z[kb][r], z[kb][r + 1]}, h, l);
      const int i = rec::chan(kb, 4 * lg + r) * 16 + lc;  // rows r, r + 1: channels i, i + 1
      sh[i] = h[0];
      sh[i + 16] = h[1];
      sl[i] = l[0];
      sl[i + 16] = l[1];
    }
}

// A [16 tokens][16 columns] accumulator (lane (c, g): rows 4 g + r) times f to
// row-major bfloat16 pairs.
__device__ __forceinline__ void stage_small(bf16_t* sh, bf16_t* sl, f32x4 z, float f, int lane) {
#pragma unroll
  for (int r = 0; r < 4; r += 2) {
    bf16x2 h, l;
    split2(f32x2{z[r] * f, z[r + 1] * f}, h, l);
    const int i = (4 * (lane / 16) + r) * 16 + lane % 16;
    sh[i] = h[0];
    sh[i + 16] = h[1];
    sl[i] = l[0];
    sl[i + 16] = l[1];
  }
}

// Out[4 g + r][c] of A B^T summed over all 128 value columns, in four 32-deep
// steps over chunks 2s, 2s + 1 (fixed order), each as hh + hl + lh: lane
// (x, g) takes row x, columns 8 (g % 2) .. + 7 of chunk 2 s + g / 2; A chunk w
// at A0 + w * as, B chunk w at B0 + w * bs (h and l arrays alike).
__device__ __forceinline__ f32x4 prod128(const bf16_t* Ah, const bf16_t* Al, int as,
                                         const bf16_t* Bh, const bf16_t* Bl, int bs, int lane) {
  const int off = (lane % 16) * 16 + 8 * ((lane / 16) % 2), wg = (lane / 16) / 2;
  f32x4 o = zero4();
  // The compiler keeps this loop rolled (it refuses the partial unroll: the
  // matrix-core builtins are convergent).  Unrolled whole it spills; unrolled
  // by two by hand, with two steps' eight reads ahead of their six products,
  // it measured the same, bit for bit and in time.
#pragma unroll 2
  for (int s = 0; s < 4; ++s) {
    const int w = 2 * s + wg;
    const bf16x8 ah = *(const bf16x8*)(Ah + w * as + off), al = *(const bf16x8*)(Al + w * as + off);
    const bf16x8 bh = *(const bf16x8*)(Bh + w * bs + off), bl = *(const bf16x8*)(Bl + w * bs + off);
    o = mma32b(ah, bh, o);
    o = mma32b(ah, bl, o);
    o = mma32b(al, bh, o);
  }
  return o;
}

__global__ void __launch_bounds__(512, 1) kda_bwd_block_kernel(BlockArgs a) {
  __shared__ __attribute__((aligned(16))) BlockSmem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, lc = lane % 16, lg = lane / 16;
  const int64_t bh = blockIdx.x / a.nblk, blk = blockIdx.x % a.nblk;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int rc0 = row_col(wave, lg);  // this lane's first column in row layout
  const int64_t x0 = blk * kBlkTiles;
  const int ntl = (int)(a.nt - x0 < kBlkTiles ? a.nt - x0 : kBlkTiles);
  // the forward-step parts of the block's records, moved to LDS once for all
  // wavefronts; then dS' at the block's end, the v rows and the block's start
  // state, which stay in flight over the barrier
  constexpr int kFwChunks = kFwBytes / 16, kFwPer = (kBlkTiles * kFwChunks + 511) / 512;
  {
    f32x4 fwv[kFwPer];  // all loads in flight at once, then the LDS stores
#pragma unroll
    for (int j = 0; j < kFwPer; ++j) {
      const int i = tid + 512 * j;
      if (i < ntl * kFwChunks) {
        const int u = i / kFwChunks, o = 16 * (i % kFwChunks);
        const unsigned char* Ru = a.recs + (bh * a.nt + x0 + u) * (int64_t)kRecBytes;
        const int src = o < kFwKbC ? kKh + o
                      : o < kFwT   ? kKbC + (o - kFwKbC)
                      : o < kFwTlo ? kT + (o - kFwT)
                      : o < kFwE   ? kTlo + (o - kFwTlo)
                                   : kE + (o - kFwE);
        fwv[j] = *(const f32x4*)(Ru + src);
      }
    }
#pragma unroll
    for (int j = 0; j < kFwPer; ++j) {
      const int i = tid + 512 * j;
      if (i < ntl * kFwChunks) *(f32x4*)&sm.fw[i / kFwChunks][16 * (i % kFwChunks)] = fwv[j];
    }
  }
  // keeps the loads below from being scheduled into the staging above, where
  // they would hold registers the staging needs
  __builtin_amdgcn_sched_barrier(0);
  f32x4 dS[8];
  load_frag(dS, a.ds_blk + (bh * a.nblk + blk) * kDD, wave, lane);
  // the block's start state: the caller's s0 ([dk][dv]) for the first block,
  // else the forward's checkpoint (accumulator order)
  const float* s_start = blk == 0 ? (a.s0 != nullptr ? a.s0 + bh * kDD : nullptr)
                                  : a.s_ck + ((b * a.nck + blk - 1) * a.H + h) * kDD;
  auto load_start = [&](f32x4 (&z)[8]) {
    if (blk == 0 || a.ck_rowmajor)
      load_state(z, s_start, wave, lane);
    else
      load_frag(z, s_start, wave, lane);
  };
  // every v row this wavefront reads, loaded once (a load issued after the
  // stores of a tile waits for those stores)
  bf16x4 vrow[kBlkTiles];
#pragma unroll
  for (int u = 0; u < kBlkTiles; ++u)
    vrow[u] = token_row4(a.v, (x0 + u) * kC + lc, a.T, b, h, a.H, rc0);
  f32x4 S[8];  // S_tl; reloaded for the next tile once it is staged
  load_start(S);
  lds_barrier();

  const bf16x4 ident = ident_op(lane);
  // adjoint quantities in units of scale / sigma (see the chain kernel)
  const float so = a.scale != 0.f ? a.scale : 1.f, dmul = a.scale != 0.f ? 1.f : 0.f;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) dS[kb] *= 1.f / so;
  Scale sd;

  for (int tl = ntl - 1; tl >= 0; --tl) {
    const int64_t x = x0 + tl;
    // the tile's dO rows, needed after the forward steps
    const bf16x4 drow = token_row4(a.dout, x * kC + lc, a.T, b, h, a.H, rc0);
    // ---- forward: S_tl from the block's start state.  T, X and Delta enter
    // their products as float16 pairs (value and rounding error).
    Scale sf;
    f32x4 X = zero4(), Dl = zero4();
    // unrolled, so that vrow[u] is a register and not a select over the array
#pragma unroll
    for (int u = 0; u < kBlkTiles; ++u) {
      if (u > tl) break;
      const unsigned char* Ru = sm.fw[u];
      const f32x4 vs = rescale(sf, S, mma16b(vrow[u], ident, zero4()));
      f16x8 sopS[4];
      state_op(S, sopS);
      f32x4 y = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) y = mma32h(ld16h(Ru + kFwKh + s * 1024 + lane * 16), sopS[s], y);
      X = vs - y;
      const f16x4 xh = to_h4(X), xl = to_h4(X - to_f4(xh));
      // T (xh + xl) in one product (both halves of k hold T), then T_lo xh
      const f16x4 t4 = ld8h(Ru + kFwT + lane * 8);
      Dl = mma32h(cat8(t4, t4), cat8(xh, xl), zero4());
      Dl = mma32h(lo8(ld8h(Ru + kFwTlo + lane * 8)), cat8(xh, xh), Dl);
      if (u < tl) {
        const f16x4 dh = to_h4(Dl), dlo = to_h4(Dl - to_f4(dh));
        const f32x2 e2 = *(const f32x2*)(Ru + kFwE + 4 * (32 * (lc / 4) + 8 * lg + 2 * (lc % 4)));
        unroll8([&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
          const f16x4 k4 = ld8h(Ru + kFwKbC + kb * 512 + lane * 8);
          S[kb] = mma32h(cat8(k4, k4), cat8(dh, dlo), decay_rows<kb>(e2, S[kb]));  // Kb^T (dh + dlo)
        });
      }
    }
    // ---- the adjoint step of tile tl
    const unsigned char* R = a.recs + (bh * a.nt + x) * (int64_t)kRecBytes;
    const f32x4 dos = rescale(sd, dS, mma16b(drow, ident, zero4()) * dmul);
    const f16x4 do16 = to_h4(dos);  // exact: sigma dO with dO in bfloat16
    // dDelta and dX with dS', Aqk, dDelta and T as float16 pairs (value and
    // rounding error; Kb alone stays one float16 rounding): the largest
    // gradients come from the final-state term in the last tiles, and four
    // float16 roundings there would cost a few times their rounding relative
    // to gradients 100 times their RMS.
    f16x8 sopD[4], sopDl[4];
    state_op(dS, sopD);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      f16x4 l0, l1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        l0[e] = (f16)(dS[2 * s2][e] - (float)sopD[s2][e]);
        l1[e] = (f16)(dS[2 * s2 + 1][e] - (float)sopD[s2][4 + e]);
      }
      sopDl[s2] = cat8(l0, l1);
    }
    f32x4 dd = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 kbh = ld16h(R + kKb + s * 1024 + lane * 16);
      dd = mma32h(kbh, sopD[s], dd);
      dd = mma32h(kbh, sopDl[s], dd);
    }
    // Aqk^T dO' (dO' exact in float16): value and rounding in one product
    dd = mma32h(cat8(ld8h(R + kAqkT + lane * 8), ld8h(R + kAqkTlo + lane * 8)),
                cat8(do16, do16), dd);
    const f16x4 dd16 = to_h4(dd), ddl = to_h4(dd - to_f4(dd16));
    const f16x4 tt4 = ld8h(R + kTt + lane * 8);
    f32x4 dx = mma32h(cat8(tt4, tt4), cat8(dd16, ddl), zero4());  // T^T (dd16 + ddl)
    dx = mma32h(lo8(ld8h(R + kTtlo + lane * 8)), cat8(dd16, dd16), dx);
    const float ff = sf.isig, fd = so * sd.isig;  // back to unscaled units
    float* Y = a.ybuf + (bh * a.nt + x) * (int64_t)kYFloats;

    // dE = rowsum(S_t * dS') in float32: each lane's column, summed over the
    // 16 lanes of its row group; lane c then holds the channels of rows
    // 4 g + 2 (c % 2) + {0, 1} of block c / 2 (adjacent channels)
    {
      float p[32];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[4 * kb + r] = S[kb][r] * dS[kb][r];
      *(f32x2*)&sm.dep[wave][rec::chan(lc / 2, 4 * lg + 2 * (lc % 2))] =
          row_reduce_scatter32(p, lc) * (ff * fd);
    }

    // ---- the products over the 128 value columns, float32: every chunk
    // staged unscaled, then wavefront w forms output columns 16 w .. 16 w + 15
    // (channels) summing the chunks in order
    // S as held (sigma_f S): its factor ff moves to dO' and dX; Delta as held
    // for dO' Delta^T, with dO' carrying ff (ff is a power of two)
    stage_state(sm.sth[wave], sm.stl[wave], S, lane);
    stage_small(sm.sxh[wave][0], sm.sxl[wave][0], dos, fd * ff, lane);
    stage_small(sm.sxh[wave][1], sm.sxl[wave][1], dx, fd * ff, lane);
    stage_small(sm.sxh[wave][2], sm.sxl[wave][2], Dl, 1.f, lane);
    stage_small(sm.sxh[wave][3], sm.sxl[wave][3], dd, fd, lane);
    stage_small(sm.sxh[wave][4], sm.sxl[wave][4], X, ff, lane);
    lds_barrier();
    constexpr int kXs = 5 * kC * 16, kSs = kDK * 16;
    const int srow = 16 * wave * 16;  // this wavefront's 16 output channels
    const f32x4 y1 = prod128(sm.sxh[0][0], sm.sxl[0][0], kXs, sm.sth[0] + srow, sm.stl[0] + srow,
                             kSs, lane);  // dO S^T
    const f32x4 y2 = prod128(sm.sxh[0][1], sm.sxl[0][1], kXs, sm.sth[0] + srow, sm.stl[0] + srow,
                             kSs, lane);  // dX S^T
    f32x4 ysm = zero4();  // wave 0: dDelta X^T, wave 1: dO Delta^T, wave 2: dE
    if (wave == 0) {
      ysm = prod128(sm.sxh[0][3], sm.sxl[0][3], kXs, sm.sxh[0][4], sm.sxl[0][4], kXs, lane);
    } else if (wave == 1) {
      ysm = prod128(sm.sxh[0][0], sm.sxl[0][0], kXs, sm.sxh[0][2], sm.sxl[0][2], kXs, lane);
    } else if (wave == 2) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int w = 0; w < 8; ++w) ysm[m] += sm.dep[w][lane + 64 * m];
      }
    }
    // [Qh^T | -Kh^T] for the update of dS' at the end, loaded now so that the
    // last product hides the wait
    f16x8 qk[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qk[kb] = ld16h(R + kQK + kb * 1024 + lane * 16);
    lds_barrier();
    // dS' as held: its factor fd moves to Delta
    stage_state(sm.sth[wave], sm.stl[wave], dS, lane);
    stage_small(sm.sxh[wave][2], sm.sxl[wave][2], Dl, ff * fd, lane);
    lds_barrier();
    const f32x4 y3 = prod128(sm.sxh[0][2], sm.sxl[0][2], kXs, sm.sth[0] + srow, sm.stl[0] + srow,
                             kSs, lane);  // Delta dS'^T
    // dV = dX in bfloat16: lane (t, g) holds the four columns from rc0 on of
    // token t, moved there by the selection-matrix product (exact: the
    // operand is already bfloat16)
    const f32x4 dvt = mma16b(
        bf16x4{(bf16_t)(dx[0] * fd), (bf16_t)(dx[1] * fd), (bf16_t)(dx[2] * fd), (bf16_t)(dx[3] * fd)},
        ident, zero4());
    const bf16x4 dvo = {(bf16_t)dvt[0], (bf16_t)dvt[1], (bf16_t)dvt[2], (bf16_t)dvt[3]};
    // dS' of the tile before (the adjoint of this tile's start state)
    {
      const f16x8 bop = cat8(do16, to_h4(dx));
      const f32x2 e2 =
          *(const f32x2*)(sm.fw[tl] + kFwE + 4 * (32 * (lc / 4) + 8 * lg + 2 * (lc % 4)));
      unroll8([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        dS[kb] = mma32h(qk[kb], bop, decay_rows<kb>(e2, dS[kb]));
      });
    }
    // the next tile's start state, loaded before this tile's stores so that
    // its wait does not take them in
    if (tl > 0) load_start(S);
    *(f32x4*)(Y + kY1 + 256 * wave + 4 * lane) = y1;
    *(f32x4*)(Y + kY2 + 256 * wave + 4 * lane) = y2;
    *(f32x4*)(Y + kY3 + 256 * wave + 4 * lane) = y3;
    if (wave < 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[(wave == 0 ? kDT : kDAqk) + (4 * lg + r) * 16 + lc] = ysm[r];
    } else if (wave == 2) {
      Y[kDE + lane] = ysm[0];
      Y[kDE + lane + 64] = ysm[1];
    }
    if (x * kC + lc < a.T)
      *(bf16x4*)(a.dv + ((b * a.T + x * kC + lc) * a.H + h) * kDV + rc0) = dvo;
    lds_barrier();  // the staging is free for the next tile
  }
}

// ------------------------------------------------------------ 5. finishing
struct FinArgs {
  const bf16_t* q;
  const bf16_t* k;
  const float* g;
  const float* beta;
  const float* ybuf;
  const float* pm;
  bf16_t* dq;
  bf16_t* dk;
  float* dg;
  float* dbeta;
  int64_t B, T, H, nt;
};

struct FinSmem {
  float k[kC][kDK], q[kC][kDK], dG[kC][kDK];
  float P[kC][kC + 1], M[kC][kC + 1], dM[kC][kC + 1], Z[kC][kC + 1];
  // dP and dAqk and their transposes, rows of 16 read whole (broadcast) by a wavefront
  __attribute__((aligned(16))) float dP[kC][kC], dAq[kC][kC], dPT[kC][kC], dAqT[kC][kC];
  float beta[kC], dbT[kC], dbA[kC];
  float kdkb[2][kDK];
  __attribute__((aligned(16))) bf16_t dqo[kC][kDK], dko[kC][kDK];  // dq, dk on their way out
};

// One workgroup per tile (256 threads), float32 throughout.  Every global
// load is issued before the arithmetic that needs it, with rows clamped into
// the sequence and tokens past its end zeroed by a factor (no load behind a
// branch), so a workgroup waits for memory a few times, not once per token.
__global__ void __launch_bounds__(256) kda_bwd_fin_kernel(FinArgs a) {
  __shared__ FinSmem sm;
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / a.nt, x = blockIdx.x % a.nt;
  const int64_t b = bh / a.H, h = bh % a.H;
  const float* __restrict__ Y = a.ybuf + (bh * a.nt + x) * (int64_t)kYFloats;
  const float* __restrict__ PM = a.pm + (bh * a.nt + x) * 512;
  const bf16_t* __restrict__ qp = a.q;
  const bf16_t* __restrict__ kp = a.k;
  const float* __restrict__ gp = a.g;
  auto row_of = [&](int t) {
    int64_t tok = x * kC + t;
    tok = tok < a.T ? tok : a.T - 1;
    return (b * a.T + tok) * a.H + h;
  };
  auto valid = [&](int t) { return x * kC + t < a.T; };

  // Y1, Y2, Y3 of thread (c, half): tokens 8 half + 4 m .. + 3 of channel c,
  // loaded first and waited for last
  const int c = tid % kDK, half = tid / kDK;
  f32x4 y1[2], y2[2], y3[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int o = 256 * (c / 16) + 4 * (c % 16 + 16 * (2 * half + m));
    y1[m] = *(const f32x4*)(Y + kY1 + o);
    y2[m] = *(const f32x4*)(Y + kY2 + o);
    y3[m] = *(const f32x4*)(Y + kY3 + o);
  }
  // the tile's inputs, 16-byte accesses: thread tid takes token tid / 16,
  // channels c8 .. c8 + 7 (the same split stores dq, dk and dg at the end)
  const int t8 = tid / 16, c8 = 8 * (tid % 16);
  {
    const int64_t r = row_of(t8);
    const bf16x8 kv = *(const bf16x8*)(kp + r * kDK + c8);
    const bf16x8 qv = *(const bf16x8*)(qp + r * kDK + c8);
    const f32x4 g0 = *(const f32x4*)(gp + r * kDK + c8), g1 = *(const f32x4*)(gp + r * kDK + c8 + 4);
    const float lv = valid(t8) ? 1.f : 0.f;
    *(f32x4*)&sm.k[t8][c8] = f32x4{(float)kv[0], (float)kv[1], (float)kv[2], (float)kv[3]} * lv;
    *(f32x4*)&sm.k[t8][c8 + 4] = f32x4{(float)kv[4], (float)kv[5], (float)kv[6], (float)kv[7]} * lv;
    *(f32x4*)&sm.q[t8][c8] = f32x4{(float)qv[0], (float)qv[1], (float)qv[2], (float)qv[3]} * lv;
    *(f32x4*)&sm.q[t8][c8 + 4] = f32x4{(float)qv[4], (float)qv[5], (float)qv[6], (float)qv[7]} * lv;
    *(f32x4*)&sm.dG[t8][c8] = g0 * lv;  // g for now
    *(f32x4*)&sm.dG[t8][c8 + 4] = g1 * lv;
    const int i = tid / kC, j = tid % kC;
    sm.P[i][j] = PM[tid];
    sm.M[i][j] = PM[256 + tid];
    const float dT = Y[kDT + tid], dAq = Y[kDAqk + tid];
    if (tid < kC) sm.beta[tid] = valid(tid) ? a.beta[row_of(tid)] : 0.f;
    lds_barrier();
    sm.dM[i][j] = dT * sm.beta[j];
    sm.dAq[i][j] = sm.dAqT[j][i] = j <= i ? dAq : 0.f;
    sm.Z[i][j] = dT * sm.M[i][j];  // for dbeta from T = M Diag(beta): column sums
  }
  // e^G and e^-G of channel c at every token of the tile (G the cumulative
  // log-decay), in registers: both threads of a channel form their own copy
  float egr[kC], iegr[kC];
  {
    float G = 0.f;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      G += sm.dG[t][c];
      egr[t] = __expf(G);
      iegr[t] = __expf(-G);
    }
  }
  lds_barrier();
  const int i = tid / kC, j = tid % kC;  // a (row, column) of a 16 x 16 matrix
  if (tid < kC) {
    float s = 0.f;
    for (int r = 0; r < kC; ++r) s += sm.Z[r][tid];
    sm.dbT[tid] = s;
  }
  lds_barrier();
  {
    float z = 0.f;  // Z = dM M^T
    for (int c = 0; c < kC; ++c) z = fmaf(sm.dM[i][c], sm.M[j][c], z);
    sm.Z[i][j] = z;
  }
  lds_barrier();
  {
    float d = 0.f;  // dA = strict_lower(-M^T Z)
    if (j < i)
      for (int c = 0; c < kC; ++c) d -= sm.M[c][i] * sm.Z[c][j];
    sm.dP[i][j] = sm.dPT[j][i] = sm.beta[i] * d;  // dP = Diag(beta) dA
    sm.dM[i][j] = d * sm.P[i][j];  // dM is spent: row sums of dA * P, for dbeta
  }
  lds_barrier();
  if (tid < kC) {
    float s = 0.f;
    for (int c = 0; c < kC; ++c) s += sm.dM[tid][c];
    sm.dbA[tid] = s;
  }

  // per (token, channel): thread (c, half) takes tokens 8 half .. 8 half + 7;
  // channel c's Kc, Kh and Qh at every token of the tile in registers, the rows
  // of dP, dAqk and their transposes read whole (the token is wavefront-uniform)
  float kcr[kC], khr[kC], qhr[kC];
#pragma unroll
  for (int jj = 0; jj < kC; ++jj) {
    const float kj = sm.k[jj][c];
    kcr[jj] = kj * iegr[jj];
    khr[jj] = kj * egr[jj];
    qhr[jj] = sm.q[jj][c] * egr[jj];
  }
  float kdkb = 0.f;
  // the token index as a constant in each of the two copies, so that egr[t]
  // and iegr[t] are registers (half is the same across a wavefront)
  auto tokens = [&](auto hc) {
    constexpr int kHalf = decltype(hc)::value;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 8 * kHalf + u;
      float i1 = 0.f, i2 = 0.f, i3 = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < kC / 4; ++j4) {
        const f32x4 p4 = *(const f32x4*)&sm.dP[t][4 * j4], a4 = *(const f32x4*)&sm.dAq[t][4 * j4];
        const f32x4 pt4 = *(const f32x4*)&sm.dPT[t][4 * j4], at4 = *(const f32x4*)&sm.dAqT[t][4 * j4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 4 * j4 + e;
          i1 = fmaf(p4[e], kcr[jj], i1);   // (dP Kc)[t]:     jj < t
          i2 = fmaf(a4[e], kcr[jj], i2);   // (dAqk Kc)[t]:   jj <= t
          i3 = fmaf(at4[e], qhr[jj], fmaf(pt4[e], khr[jj], i3));  // (dAqk^T Qh + dP^T Kh)[t]
        }
      }
      const float egt = egr[t], iegt = iegr[t];
      const float dq = egt * (y1[u / 4][u % 4] + i2);
      const float dkh = egt * (i1 - y2[u / 4][u % 4]);
      const float dkc = iegt * i3;
      const float dkb = egr[kC - 1] * iegt * y3[u / 4][u % 4];
      const float kt = sm.k[t][c];
      kdkb = fmaf(kt, dkb, kdkb);
      sm.dG[t][c] = kt * (dkh - dkc - dkb) + sm.q[t][c] * dq;
      sm.dqo[t][c] = (bf16_t)dq;
      sm.dko[t][c] = (bf16_t)(dkh + dkc + dkb);
    }
  };
  if (__builtin_amdgcn_readfirstlane(half) == 0)
    tokens(std::integral_constant<int, 0>{});
  else
    tokens(std::integral_constant<int, 1>{});
  sm.kdkb[half][c] = kdkb;
  lds_barrier();
  if (tid < kDK) {  // dG_15 += sum_rows k dk_b + dE E, then dg = reverse cumulative sum
    float acc = sm.kdkb[0][c] + sm.kdkb[1][c] + Y[kDE + c] * egr[kC - 1];
#pragma unroll
    for (int t = kC - 1; t >= 0; --t) {
      acc += sm.dG[t][c];
      sm.dG[t][c] = acc;
    }
  } else if (tid < kDK + kC) {
    const int t = tid - kDK;
    if (valid(t)) a.dbeta[row_of(t)] = sm.dbT[t] + sm.dbA[t];
  }
  const bool live8 = valid(t8);
  const int64_t r8 = row_of(t8);
  if (live8) {
    *(bf16x8*)(a.dq + r8 * kDK + c8) = *(const bf16x8*)&sm.dqo[t8][c8];
    *(bf16x8*)(a.dk + r8 * kDK + c8) = *(const bf16x8*)&sm.dko[t8][c8];
  }
  lds_barrier();
  if (live8) {
    *(f32x4*)(a.dg + r8 * kDK + c8) = *(const f32x4*)&sm.dG[t8][c8];
    *(f32x4*)(a.dg + r8 * kDK + c8 + 4) = *(const f32x4*)&sm.dG[t8][c8 + 4];
  }
}

}  // namespace bwd

// Workspace of the chunkwise backward, in 256-byte aligned parts.
struct BwdChunkWs {
  int64_t fwd, s_tmp, s_ck, ds_blk, recs, pm, ybuf, total;
};

static int64_t al256(int64_t n) { return (n + 255) / 256 * 256; }

static BwdChunkWs bwd_chunk_layout(int64_t B, int64_t T, int64_t H) {
  using namespace bwd;
  const int64_t BH = B * H, nt = (T + kC - 1) / kC, nblk = (nt + kBlkTiles - 1) / kBlkTiles;
  BwdChunkWs w;
  w.fwd = 0;
  w.s_tmp = al256((int64_t)chunk_mfma_workspace(B, T, H));
  w.s_ck = w.s_tmp + al256(BH * kDD * 4);
  w.ds_blk = w.s_ck + al256(B * (T / kBlkTok) * H * kDD * 4);
  w.recs = w.ds_blk + al256(BH * nblk * kDD * 4);
  w.pm = w.recs + al256(BH * nt * (int64_t)kRecBytes);
  w.ybuf = w.pm + al256(BH * nt * 512 * 4);
  w.total = w.ybuf + al256(BH * nt * (int64_t)kYFloats * 4);
  return w;
}

int64_t bwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t H) {
  return bwd_chunk_layout(B, T, H).total;
}

hipError_t launch_bwd_chunk(const BwdArgs& a) {
  using namespace bwd;
  const int64_t BH = a.B * a.H, nt = (a.T + kC - 1) / kC;
  const int64_t nblk = (nt + kBlkTiles - 1) / kBlkTiles, nck = a.T / kBlkTok;
  if (BH * nt > 0x7fffffffLL || BH * nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const BwdChunkWs w = bwd_chunk_layout(a.B, a.T, a.H);
  unsigned char* ws = (unsigned char*)a.workspace;
  hipStream_t st = (hipStream_t)a.stream;

  // 1. forward states every 64 tokens (unless the caller brings them)
  hipError_t e;
  if (a.ckpt == nullptr) {
    ChunkArgs ca{a.q, a.k, a.v, a.g, a.beta, a.s0, nullptr, (float*)(ws + w.s_tmp), nullptr,
                 nullptr, 0.f, a.B, a.T, a.H, kDK, kDV, 1.f, true, ws + w.fwd, a.stream};
    ca.total = a.B * a.T;
    if (nck > 0) {
      ca.ckpt = (float*)(ws + w.s_ck);
      ca.ckpt_every = kBlkTok;
      ca.ckpt_frag = true;
    }
    if ((e = launch_chunk_mfma(ca)) != hipSuccess) return e;
  }

  // 2. records
  RecArgs ra{(const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.beta, ws + w.recs,
             (float*)(ws + w.pm), a.B, a.T, a.H, nt};
  int64_t nrec = (BH * nt + 3) / 4;
  nrec = nrec < 16384 ? nrec : 16384;
  hipLaunchKernelGGL(kda_bwd_rec_kernel, dim3((unsigned)nrec), dim3(256), 0, st, ra);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 3. the adjoint chain
  ChainArgs cha{ws + w.recs, (const bf16_t*)a.dout, a.ds_final, (float*)(ws + w.ds_blk), a.ds0,
                a.B, a.T, a.H, nt, nblk, a.scale};
  hipLaunchKernelGGL(kda_bwd_chain_kernel, dim3((unsigned)(BH * kChainSplit)),
                     dim3(64 * (kChainWaves + kChainLoaders)), 0,
                     st, cha);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 4. block products
  BlockArgs ba{ws + w.recs, (const bf16_t*)a.v, (const bf16_t*)a.dout, a.s0,
               a.ckpt != nullptr ? a.ckpt : (const float*)(ws + w.s_ck), a.ckpt != nullptr,
               (const float*)(ws + w.ds_blk), (bf16_t*)a.dv,
               (float*)(ws + w.ybuf), a.B, a.T, a.H, nt, nblk, nck, a.scale};
  hipLaunchKernelGGL(kda_bwd_block_kernel, dim3((unsigned)(BH * nblk)), dim3(512), 0, st, ba);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // 5. finishing
  FinArgs fa{(const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.beta, (const float*)(ws + w.ybuf),
             (const float*)(ws + w.pm), (bf16_t*)a.dq, (bf16_t*)a.dk, a.dg, a.dbeta,
             a.B, a.T, a.H, nt};
  hipLaunchKernelGGL(kda_bwd_fin_kernel, dim3((unsigned)(BH * nt)), dim3(256), 0, st, fa);
  return hipGetLastError();
}

}  // namespace kda
