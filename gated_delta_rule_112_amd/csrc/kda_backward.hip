// Backward of the KDA token recurrence (gfx950), dk = dv = 128.
//
// The forward is the recurrence of "Kimi K3 Architecture Explained ...",
// section "Token mixing": S_t = (I - beta k k^T) Diag(a) S_{t-1} + beta k v^T
// with a = exp(g), o_t = scale S_t^T q_t.  The pages give no backward pass;
// these are the plain gradients of a loss given dO for every token and dS_T
// for the final state.  Reverse mode, per token, with Sd = Diag(a) S_{t-1},
// p = Sd^T k, u = beta (v - p) and dS the adjoint of S_t:
//   dS += scale q dO^T
//   dq  = scale (Sd dO + k (u . dO))
//   du  = dS^T k,  dp = -beta du,  dv = beta du,  dbeta = du . (v - p)
//   dk  = dS u + Sd dp
//   dSd = dS + k dp^T,  dg = a * rowsum(dSd * S_{t-1}),  dS <- Diag(a) dSd
//
// One 256-thread workgroup per (b, h) keeps S and dS as float4 strips of 16
// rows in registers (the layout of the decode step).  A forward pass stores
// the state every kBwdPiece tokens in the workspace; the reverse sweep then
// takes the pieces last to first, recomputes each piece's pre-token states
// from its checkpoint into the workspace and walks the piece backwards.  Every
// workspace strip is read back only by the thread that wrote it.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int D = 128, NT = 256, CG = D / 4, RG = NT / CG, RPT = D / RG;
constexpr int64_t DD = (int64_t)D * D;

struct BwdSmem {
  float k[D], q[D], v[D], a[D], dO[D];
  float u[D], vmp[D], dp[D];
  float part[RG][D];
  float red[2][2];
  float beta;
};

template <typename IO>
__device__ __forceinline__ void load_tok(BwdSmem& sm, const IO* q, const IO* k, const IO* v,
                                         const float* g, const float* beta, const IO* dO,
                                         int64_t row, bool grads) {
  const int tid = threadIdx.x;
  if (tid < D) {
    sm.k[tid] = ld_f32(k + row * D + tid);
    sm.a[tid] = __expf(g[row * D + tid]);
    sm.v[tid] = ld_f32(v + row * D + tid);
    if (grads) {
      sm.q[tid] = ld_f32(q + row * D + tid);
      sm.dO[tid] = ld_f32(dO + row * D + tid);
    }
  }
  if (tid == 0) sm.beta = beta[row];
}

__device__ __forceinline__ void ld_strip(f32x4 (&s)[RPT], const float* src) {
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = *(const f32x4*)(src + (rg + m * RG) * D + 4 * cg);
}

__device__ __forceinline__ void st_strip(float* dst, const f32x4 (&s)[RPT]) {
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
#pragma unroll
  for (int m = 0; m < RPT; ++m) *(f32x4*)(dst + (rg + m * RG) * D + 4 * cg) = s[m];
}

// Sum of x over the 32 column groups of a half-wave (the lanes of one row group).
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// p_j = sum_i a_i k_i S_ij into sm.part (per row group), then u_j, v_j - p_j
// for column j = tid.  The token's inputs are in sm (synchronised).
__device__ __forceinline__ void form_u(BwdSmem& sm, const f32x4 (&s)[RPT]) {
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    p += (sm.a[i] * sm.k[i]) * s[m];
  }
  *(f32x4*)&sm.part[rg][4 * cg] = p;
  __syncthreads();
  if (tid < D) {
    float pj = 0.f;
#pragma unroll
    for (int x = 0; x < RG; ++x) pj += sm.part[x][tid];
    const float vmp = sm.v[tid] - pj;
    sm.vmp[tid] = vmp;
    sm.u[tid] = sm.beta * vmp;
  }
  __syncthreads();
}

__device__ __forceinline__ void fwd_step(BwdSmem& sm, f32x4 (&s)[RPT]) {
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  form_u(sm, s);
  const f32x4 u4 = *(const f32x4*)&sm.u[4 * cg];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    s[m] = sm.a[i] * s[m] + sm.k[i] * u4;
  }
  __syncthreads();  // the token's shared inputs are replaced next
}

template <typename IO>
__device__ __forceinline__ void bwd_step(BwdSmem& sm, const f32x4 (&sp)[RPT], f32x4 (&dS)[RPT],
                                         float scale, int64_t row, IO* dq, IO* dk, IO* dv,
                                         float* dg, float* dbeta) {
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  form_u(sm, sp);
  // u . dO over the 128 columns (waves 0 and 1 hold them)
  if (tid < D) {
    float x = sm.u[tid] * sm.dO[tid];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (tid % 64 == 0) sm.red[0][tid / 64] = x;
  }
  // the output's term, then du_j = sum_i dS_ij k_i
  const f32x4 dO4 = *(const f32x4*)&sm.dO[4 * cg];
  f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    dS[m] += (scale * sm.q[i]) * dO4;
    du += sm.k[i] * dS[m];
  }
  *(f32x4*)&sm.part[rg][4 * cg] = du;
  __syncthreads();
  if (tid < D) {
    float duj = 0.f;
#pragma unroll
    for (int x = 0; x < RG; ++x) duj += sm.part[x][tid];
    st_f32(dv + row * D + tid, sm.beta * duj);
    sm.dp[tid] = -sm.beta * duj;
    float x = duj * sm.vmp[tid];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (tid % 64 == 0) sm.red[1][tid / 64] = x;
  }
  __syncthreads();
  if (tid == 0) dbeta[row] = sm.red[1][0] + sm.red[1][1];
  const float udo = sm.red[0][0] + sm.red[0][1];
  const f32x4 u4 = *(const f32x4*)&sm.u[4 * cg];
  const f32x4 dp4 = *(const f32x4*)&sm.dp[4 * cg];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    const float ai = sm.a[i], ki = sm.k[i];
    const f32x4 sd = ai * sp[m];
    const f32x4 dsd = dS[m] + ki * dp4;
    const f32x4 xq = sd * dO4, xk = dS[m] * u4 + sd * dp4, xg = dsd * sp[m];
    const float rq = row_sum(xq[0] + xq[1] + xq[2] + xq[3]);
    const float rk = row_sum(xk[0] + xk[1] + xk[2] + xk[3]);
    const float rgs = row_sum(xg[0] + xg[1] + xg[2] + xg[3]);
    if (cg == 0) {
      st_f32(dq + row * D + i, scale * (rq + ki * udo));
      st_f32(dk + row * D + i, rk);
      dg[row * D + i] = ai * rgs;
    }
    dS[m] = ai * dsd;
  }
  __syncthreads();  // the token's shared inputs are replaced next
}

template <typename IO>
__global__ void __launch_bounds__(NT, 1)
kda_bwd_kernel(const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
               const float* __restrict__ g, const float* __restrict__ beta,
               const float* __restrict__ s0, const IO* __restrict__ dO,
               const float* __restrict__ ds_final, IO* __restrict__ dq, IO* __restrict__ dk,
               IO* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta,
               float* __restrict__ ds0, int64_t T, int64_t H, float scale,
               float* __restrict__ ws) {
  __shared__ BwdSmem sm;
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H;
  const int64_t npc = (T + kBwdPiece - 1) / kBwdPiece;
  float* ck = ws + bh * (npc + kBwdPiece) * DD;  // checkpoints, then one piece's states
  float* pre = ck + npc * DD;
  auto row = [&](int64_t t) { return (b * T + t) * H + h; };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // forward: the state at the start of every piece
  f32x4 s[RPT];
  if (s0 != nullptr) {
    ld_strip(s, s0 + bh * DD);
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = zero;
  }
  for (int64_t t = 0; t < (npc - 1) * kBwdPiece; ++t) {
    if (t % kBwdPiece == 0) st_strip(ck + (t / kBwdPiece) * DD, s);
    load_tok(sm, q, k, v, g, beta, dO, row(t), false);
    __syncthreads();
    fwd_step(sm, s);
  }
  st_strip(ck + (npc - 1) * DD, s);

  // reverse sweep, piece by piece
  f32x4 dS[RPT];
  if (ds_final != nullptr) {
    ld_strip(dS, ds_final + bh * DD);
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) dS[m] = zero;
  }
  for (int64_t c = npc - 1; c >= 0; --c) {
    const int64_t t0 = c * kBwdPiece, t1 = (t0 + kBwdPiece < T) ? t0 + kBwdPiece : T;
    ld_strip(s, ck + c * DD);
    for (int64_t t = t0; t < t1; ++t) {
      st_strip(pre + (t - t0) * DD, s);
      if (t + 1 < t1) {
        load_tok(sm, q, k, v, g, beta, dO, row(t), false);
        __syncthreads();
        fwd_step(sm, s);
      }
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      ld_strip(s, pre + (t - t0) * DD);
      load_tok(sm, q, k, v, g, beta, dO, row(t), true);
      __syncthreads();
      bwd_step(sm, s, dS, scale, row(t), dq, dk, dv, dg, dbeta);
    }
  }
  if (ds0 != nullptr) st_strip(ds0 + bh * DD, dS);
}

}  // namespace

int64_t bwd_workspace_floats(int64_t B, int64_t T, int64_t H) {
  const int64_t npc = (T + kBwdPiece - 1) / kBwdPiece;
  return B * H * (npc + kBwdPiece) * DD;
}

hipError_t launch_recurrent_bwd(const BwdArgs& a) {
  const int64_t BH = a.B * a.H;
  if (BH <= 0 || a.T <= 0 || BH > 0x7fffffffLL) return hipErrorInvalidValue;
#define KDA_BWD(IO)                                                                          \
  hipLaunchKernelGGL((kda_bwd_kernel<IO>), dim3((unsigned)BH), dim3(NT), 0,                   \
                     (hipStream_t)a.stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g, \
                     a.beta, a.s0, (const IO*)a.dout, a.ds_final, (IO*)a.dq, (IO*)a.dk,        \
                     (IO*)a.dv, a.dg, a.dbeta, a.ds0, a.T, a.H, a.scale, a.workspace)
  if (a.io_bf16)
    KDA_BWD(bf16_t);
  else
    KDA_BWD(float);
#undef KDA_BWD
  return hipGetLastError();
}

}  // namespace kda
