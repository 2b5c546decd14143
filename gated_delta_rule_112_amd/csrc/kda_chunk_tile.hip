// Tile kernel of the matrix-core chunked prefill: everything about a 16-token
// tile that does not depend on the running state, for all tiles at once.
//
// One wavefront per tile.  Lane (t, g) = (lane % 16, lane / 16) holds token t
// and, for each 32-channel slab s, the key channels 32 s + 8 g + 0..7.  Per
// slab it forms the in-tile cumulative log-decay (a prefix sum over the 16
// lanes of a DPP row), the exponentials and the rescaled operands, and
// accumulates the two intra-tile products over the slab on the matrix cores in
// float32 (16x16x4: each k step is one of the lane's channels, so the
// operands come straight from registers):
//   lane (i, g) accumulates (Kh Kc^T)[i][4 g + r] and (Qh Kc^T)[i][4 g + r].
// Kh and Kb are transposed to channel-major 16x16 blocks by a product with a
// 0/1 selection matrix (exact).  The 16x16 unit-lower-triangular system
// (I + A) Y = I is solved by forward substitution, lane (i, g) holding rows i
// of columns 4 g + 0..3 and the pivot row broadcast over each DPP row; then
// T = Y Diag(beta) and W = T Kh.  The results are stored as one record per
// tile in the layout the state kernel consumes (kda_chunk_rec.h).
//
// Precision: all sums over key channels and the solve are float32; the stored
// matrix operands are float16 (11-bit significand), e^G_15 is float32.
#include "kda_chunk_rec.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kWaves = 4;  // tiles per workgroup, one wavefront each
constexpr float kLog2e = 1.4426950408889634f;

struct WaveSmem {
  float a[16][20];  // A = strict_lower(Diag(beta) Kh Kc^T), row-major, padded rows
  float beta[16];
};

// One step of the forward substitution: column values y[e] of rows i (this
// lane's row) receive -A[i][M] * y_M, with y_M broadcast from lane M of the row.
template <int M>
__device__ __forceinline__ void forward_sub(float (&y)[4], const f32x4 (&arow)[4]) {
  const float aim = arow[M / 4][M % 4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = fmaf(-aim, row_bcast<M>(y[e]), y[e]);
  if constexpr (M + 1 < 15) forward_sub<M + 1>(y, arow);
}

__global__ void __launch_bounds__(64 * kWaves)
kda_tile_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const float* __restrict__ g, const float* __restrict__ beta,
                unsigned char* __restrict__ recs, int64_t T, int64_t H, int64_t BH,
                int64_t x0, int64_t nseg, float scale) {
  __shared__ WaveSmem smem[kWaves];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int64_t w = (int64_t)blockIdx.x * kWaves + wave;  // (head, tile of the segment)
  if (w >= BH * nseg) return;  // whole wavefront; no workgroup barrier follows
  WaveSmem& sm = smem[wave];

  const int64_t bh = w / nseg, xl = w % nseg;
  const int64_t b = bh / H, h = bh % H;
  const int t = lane % 16, lg = lane / 16;
  const int64_t tok = (x0 + xl) * rec::kC + t;
  const bool live = tok < T;
  const int64_t row = (b * T + (live ? tok : T - 1)) * H + h;  // clamped: always in bounds
  unsigned char* R = recs + w * (int64_t)rec::kBytes;

  // All loads first: 4 slabs x (8 q, 8 k, 8 g) values of token t.
  bf16x8 qv[4], kv[4];
  f32x4 gv[4][2];
  {
    const bf16_t* qp = q + row * rec::kDK + 8 * lg;
    const bf16_t* kp = k + row * rec::kDK + 8 * lg;
    const float* gp = g + row * rec::kDK + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qv[s] = __builtin_nontemporal_load((const bf16x8*)(qp + 32 * s));
      kv[s] = __builtin_nontemporal_load((const bf16x8*)(kp + 32 * s));
      gv[s][0] = __builtin_nontemporal_load((const f32x4*)(gp + 32 * s));
      gv[s][1] = __builtin_nontemporal_load((const f32x4*)(gp + 32 * s + 4));
    }
  }
  const float bt = live ? beta[row] : 0.f;
  const float lv = live ? 1.f : 0.f;  // tokens past the end: q = k = g = 0

  // Selection matrix for the transposes: B[k = 4 g + e][c] = (k == c).
  f16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (f16)((4 * lg + e == t) ? 1.f : 0.f);

  f32x4 acc_a = zero4();  // lane (i, g): (Kh Kc^T)[i][4 g + r]
  f32x4 acc_q = zero4();  // lane (t, g): (Qh Kc^T)[t][4 g + r]
  f16x4 khT[8];           // Kh^T blocks: lane (c, g): Kh[4 g + r][chan(b, c)]
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float gm[8] = {gv[s][0][0], gv[s][0][1], gv[s][0][2], gv[s][0][3],
                   gv[s][1][0], gv[s][1][1], gv[s][1][2], gv[s][1][3]};
    float kh[8], kc[8], qh[8], kb[8], en8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gl = row_scan16(gm[e] * (kLog2e * lv));  // G in log2 units
      const float eg = __builtin_amdgcn_exp2f(gl);          // e^G    <= 1
      const float ieg = __builtin_amdgcn_exp2f(-gl);        // e^-G   <  e^80
      en8[e] = row_bcast<15>(eg);                           // e^G_15 of this channel
      const float kf = (float)kv[s][e] * lv;
      const float qf = (float)qv[s][e] * (scale * lv);
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
    __builtin_nontemporal_store(f16x8{(f16)qh[0], (f16)qh[1], (f16)qh[2], (f16)qh[3],
                                      (f16)qh[4], (f16)qh[5], (f16)qh[6], (f16)qh[7]},
                                (f16x8*)(R + rec::kQh + s * 1024 + lane * 16));
    // Channel-major blocks 2s (channels 32 s + 8 g + 0..3) and 2s+1 (+ 4..7).
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const f16x4 kh4 = {(f16)kh[4 * hb], (f16)kh[4 * hb + 1], (f16)kh[4 * hb + 2],
                         (f16)kh[4 * hb + 3]};
      const f16x4 kb4 = {(f16)kb[4 * hb], (f16)kb[4 * hb + 1], (f16)kb[4 * hb + 2],
                         (f16)kb[4 * hb + 3]};
      khT[2 * s + hb] = to_h4(mma16h(kh4, ident, zero4()));
      __builtin_nontemporal_store(to_h4(mma16h(kb4, ident, zero4())),
                                  (f16x4*)(R + rec::kKb + (2 * s + hb) * 512 + lane * 8));
    }
    if (t == 15) {
      f32x4* ep = (f32x4*)(R + rec::kEn + (32 * s + 8 * lg) * 4);
      __builtin_nontemporal_store(f32x4{en8[0], en8[1], en8[2], en8[3]}, ep);
      __builtin_nontemporal_store(f32x4{en8[4], en8[5], en8[6], en8[7]}, ep + 1);
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
  __builtin_nontemporal_store(aq, (f16x4*)(R + rec::kAqk + lane * 8));
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
  const f16x4 tb = {(f16)(y[0] * bj[0]), (f16)(y[1] * bj[1]), (f16)(y[2] * bj[2]),
                    (f16)(y[3] * bj[3])};  // lane (i, g): T[i][4 g + e]
  __builtin_nontemporal_store(tb, (f16x4*)(R + rec::kT + lane * 8));

  // W^T block b = Kh^T_b T^T: lane (i, g) receives W[i][chan(b, 4 g + r)].
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const f32x4 w0 = mma16h(khT[2 * s], tb, zero4());
    const f32x4 w1 = mma16h(khT[2 * s + 1], tb, zero4());
    __builtin_nontemporal_store(cat8(to_h4(-w0), to_h4(-w1)),
                                (f16x8*)(R + rec::kW + s * 1024 + lane * 16));
  }
}

}  // namespace

hipError_t launch_chunk_tiles(const ChunkArgs& a, unsigned char* recs, int64_t x0,
                              int64_t nseg) {
  const int64_t BH = a.B * a.H;
  const int64_t nblk = (BH * nseg + kWaves - 1) / kWaves;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kda_tile_kernel, dim3((unsigned)nblk), dim3(64 * kWaves), 0,
                     (hipStream_t)a.stream, (const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.beta,
                     recs, a.T, a.H, BH, x0, nseg, a.scale);
  return hipGetLastError();
}

}  // namespace kda
