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
// kBwdSplit 256-thread workgroups per (b, h) each keep 128 / kBwdSplit value
// columns of S and dS as float4 strips in registers.  A forward pass stores
// the state every kBwdPiece tokens in the workspace; the reverse sweep then
// takes the pieces last to first, recomputes each piece's pre-token states
// from its checkpoint into the workspace and walks the piece backwards.  Every
// workspace strip is read back only by the thread that wrote it.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int D = 128, NT = 256;
constexpr int64_t DD = (int64_t)D * D;

// NS workgroups share one (b, h): each holds CW = D / NS value columns of S
// and dS, as float4 strips of RPT rows per thread (CG column groups of four,
// RG row groups).  Every cross-column quantity of the adjoint step (dq, dk,
// dg, dbeta and u . dO) is a sum over columns, so with NS > 1 each workgroup
// writes its part and a second kernel adds the NS parts.
template <int NS>
struct Lay {
  static constexpr int CW = D / NS, CG = CW / 4, RG = NT / CG, RPT = D / RG;
  static constexpr int NW = CW >= 64 ? CW / 64 : 1;  // waves that hold the columns
};

template <int NS>
struct BwdSmem {
  float k[D], q[D], v[D], a[D], dO[D];
  float u[D], vmp[D], dp[D];
  float part[Lay<NS>::RG][Lay<NS>::CW];
  float red[2][2];
  float beta;
};

template <int NS, typename IO>
__device__ __forceinline__ void load_tok(BwdSmem<NS>& sm, const IO* q, const IO* k, const IO* v,
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

template <int NS>
__device__ __forceinline__ void ld_strip(f32x4 (&s)[Lay<NS>::RPT], const float* src, int col0) {
  using L = Lay<NS>;
  const int cg = threadIdx.x % L::CG, rg = threadIdx.x / L::CG;
#pragma unroll
  for (int m = 0; m < L::RPT; ++m)
    s[m] = *(const f32x4*)(src + (rg + m * L::RG) * D + col0 + 4 * cg);
}

template <int NS>
__device__ __forceinline__ void st_strip(float* dst, const f32x4 (&s)[Lay<NS>::RPT], int col0) {
  using L = Lay<NS>;
  const int cg = threadIdx.x % L::CG, rg = threadIdx.x / L::CG;
#pragma unroll
  for (int m = 0; m < L::RPT; ++m)
    *(f32x4*)(dst + (rg + m * L::RG) * D + col0 + 4 * cg) = s[m];
}

// Sum of x over the CG column groups of one row group (CG consecutive lanes).
template <int NS>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = Lay<NS>::CG / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Sum over the workgroup's CW columns of x (given by thread tid < CW; others
// pass 0), into sm.red[w][*]: call from every thread, read after a barrier.
template <int NS>
__device__ __forceinline__ void col_total(BwdSmem<NS>& sm, int w, float x) {
  const int tid = threadIdx.x;
  if (tid < 64 * Lay<NS>::NW) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (tid % 64 == 0) sm.red[w][tid / 64] = x;
  }
}

template <int NS>
__device__ __forceinline__ float red_sum(const BwdSmem<NS>& sm, int w) {
  return Lay<NS>::NW == 2 ? sm.red[w][0] + sm.red[w][1] : sm.red[w][0];
}

// p_j = sum_i a_i k_i S_ij for the workgroup's columns, then u_j and v_j - p_j.
template <int NS>
__device__ __forceinline__ void form_u(BwdSmem<NS>& sm, const f32x4 (&s)[Lay<NS>::RPT],
                                       int col0) {
  using L = Lay<NS>;
  const int tid = threadIdx.x, cg = tid % L::CG, rg = tid / L::CG;
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < L::RPT; ++m) {
    const int i = rg + m * L::RG;
    p += (sm.a[i] * sm.k[i]) * s[m];
  }
  *(f32x4*)&sm.part[rg][4 * cg] = p;
  __syncthreads();
  if (tid < L::CW) {
    float pj = 0.f;
#pragma unroll
    for (int x = 0; x < L::RG; ++x) pj += sm.part[x][tid];
    const int j = col0 + tid;
    const float vmp = sm.v[j] - pj;
    sm.vmp[j] = vmp;
    sm.u[j] = sm.beta * vmp;
  }
  __syncthreads();
}

template <int NS>
__device__ __forceinline__ void fwd_step(BwdSmem<NS>& sm, f32x4 (&s)[Lay<NS>::RPT], int col0) {
  using L = Lay<NS>;
  const int cg = threadIdx.x % L::CG, rg = threadIdx.x / L::CG;
  form_u(sm, s, col0);
  const f32x4 u4 = *(const f32x4*)&sm.u[col0 + 4 * cg];
#pragma unroll
  for (int m = 0; m < L::RPT; ++m) {
    const int i = rg + m * L::RG;
    s[m] = sm.a[i] * s[m] + sm.k[i] * u4;
  }
  __syncthreads();  // the token's shared inputs are replaced next
}

// Row outputs of one token: with NS = 1 the gradients themselves, else this
// workgroup's parts (pq, pk, pg [NS][rows][D], pb [NS][rows]).
template <typename IO>
struct RowOut {
  IO* dq;
  IO* dk;
  float* dg;
  float* dbeta;
  float* pq;
  float* pk;
  float* pg;
  float* pb;
};

template <int NS, typename IO>
__device__ __forceinline__ void bwd_step(BwdSmem<NS>& sm, const f32x4 (&sp)[Lay<NS>::RPT],
                                         f32x4 (&dS)[Lay<NS>::RPT], float scale, int64_t row,
                                         int64_t rows, int col0, int split, IO* dv,
                                         const RowOut<IO>& ro) {
  using L = Lay<NS>;
  const int tid = threadIdx.x, cg = tid % L::CG, rg = tid / L::CG;
  form_u(sm, sp, col0);
  col_total(sm, 0, tid < L::CW ? sm.u[col0 + tid] * sm.dO[col0 + tid] : 0.f);
  // the output's term, then du_j = sum_i dS_ij k_i
  const f32x4 dO4 = *(const f32x4*)&sm.dO[col0 + 4 * cg];
  f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < L::RPT; ++m) {
    const int i = rg + m * L::RG;
    dS[m] += (scale * sm.q[i]) * dO4;
    du += sm.k[i] * dS[m];
  }
  *(f32x4*)&sm.part[rg][4 * cg] = du;
  __syncthreads();
  float xb = 0.f;
  if (tid < L::CW) {
    const int j = col0 + tid;
    float duj = 0.f;
#pragma unroll
    for (int x = 0; x < L::RG; ++x) duj += sm.part[x][tid];
    st_f32(dv + row * D + j, sm.beta * duj);
    sm.dp[j] = -sm.beta * duj;
    xb = duj * sm.vmp[j];
  }
  col_total(sm, 1, xb);
  __syncthreads();
  if (tid == 0) {
    if constexpr (NS == 1)
      ro.dbeta[row] = red_sum(sm, 1);
    else
      ro.pb[split * rows + row] = red_sum(sm, 1);
  }
  const float udo = red_sum(sm, 0);
  const f32x4 u4 = *(const f32x4*)&sm.u[col0 + 4 * cg];
  const f32x4 dp4 = *(const f32x4*)&sm.dp[col0 + 4 * cg];
#pragma unroll
  for (int m = 0; m < L::RPT; ++m) {
    const int i = rg + m * L::RG;
    const float ai = sm.a[i], ki = sm.k[i];
    const f32x4 sd = ai * sp[m];
    const f32x4 dsd = dS[m] + ki * dp4;
    const f32x4 xq = sd * dO4, xk = dS[m] * u4 + sd * dp4, xg = dsd * sp[m];
    const float rq = row_sum<NS>(xq[0] + xq[1] + xq[2] + xq[3]);
    const float rk = row_sum<NS>(xk[0] + xk[1] + xk[2] + xk[3]);
    const float rgs = row_sum<NS>(xg[0] + xg[1] + xg[2] + xg[3]);
    if (cg == 0) {
      const float vq = scale * (rq + ki * udo), vg = ai * rgs;
      if constexpr (NS == 1) {
        st_f32(ro.dq + row * D + i, vq);
        st_f32(ro.dk + row * D + i, rk);
        ro.dg[row * D + i] = vg;
      } else {
        const int64_t at = (split * rows + row) * D + i;
        ro.pq[at] = vq;
        ro.pk[at] = rk;
        ro.pg[at] = vg;
      }
    }
    dS[m] = ai * dsd;
  }
  __syncthreads();  // the token's shared inputs are replaced next
}

template <int NS, typename IO>
__global__ void __launch_bounds__(NT, 1)
kda_bwd_kernel(const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
               const float* __restrict__ g, const float* __restrict__ beta,
               const float* __restrict__ s0, const IO* __restrict__ dO,
               const float* __restrict__ ds_final, IO* __restrict__ dv,
               float* __restrict__ ds0, int64_t B, int64_t T, int64_t H, float scale,
               float* __restrict__ ws, RowOut<IO> ro) {
  using L = Lay<NS>;
  __shared__ BwdSmem<NS> sm;
  const int64_t bh = blockIdx.x / NS, b = bh / H, h = bh % H;
  const int split = (int)(blockIdx.x % NS), col0 = split * L::CW;
  const int64_t npc = (T + kBwdPiece - 1) / kBwdPiece, rows = B * T * H;
  float* ck = ws + bh * (npc + kBwdPiece) * DD;  // checkpoints, then one piece's states
  float* pre = ck + npc * DD;
  auto row = [&](int64_t t) { return (b * T + t) * H + h; };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // forward: the state at the start of every piece
  f32x4 s[L::RPT];
  if (s0 != nullptr) {
    ld_strip<NS>(s, s0 + bh * DD, col0);
  } else {
#pragma unroll
    for (int m = 0; m < L::RPT; ++m) s[m] = zero;
  }
  for (int64_t t = 0; t < (npc - 1) * kBwdPiece; ++t) {
    if (t % kBwdPiece == 0) st_strip<NS>(ck + (t / kBwdPiece) * DD, s, col0);
    load_tok(sm, q, k, v, g, beta, dO, row(t), false);
    __syncthreads();
    fwd_step(sm, s, col0);
  }
  st_strip<NS>(ck + (npc - 1) * DD, s, col0);

  // reverse sweep, piece by piece
  f32x4 dS[L::RPT];
  if (ds_final != nullptr) {
    ld_strip<NS>(dS, ds_final + bh * DD, col0);
  } else {
#pragma unroll
    for (int m = 0; m < L::RPT; ++m) dS[m] = zero;
  }
  for (int64_t c = npc - 1; c >= 0; --c) {
    const int64_t t0 = c * kBwdPiece, t1 = (t0 + kBwdPiece < T) ? t0 + kBwdPiece : T;
    ld_strip<NS>(s, ck + c * DD, col0);
    for (int64_t t = t0; t < t1; ++t) {
      st_strip<NS>(pre + (t - t0) * DD, s, col0);
      if (t + 1 < t1) {
        load_tok(sm, q, k, v, g, beta, dO, row(t), false);
        __syncthreads();
        fwd_step(sm, s, col0);
      }
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      ld_strip<NS>(s, pre + (t - t0) * DD, col0);
      load_tok(sm, q, k, v, g, beta, dO, row(t), true);
      __syncthreads();
      bwd_step(sm, s, dS, scale, row(t), rows, col0, split, dv, ro);
    }
  }
  if (ds0 != nullptr) st_strip<NS>(ds0 + bh * DD, dS, col0);
}

// The NS parts of the row outputs added up.
template <int NS, typename IO>
__global__ void __launch_bounds__(256)
kda_bwd_combine(RowOut<IO> ro, int64_t rows) {
  const int64_t n = rows * D;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    float aq = 0.f, ak = 0.f, ag = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      aq += ro.pq[s * n + e];
      ak += ro.pk[s * n + e];
      ag += ro.pg[s * n + e];
    }
    st_f32(ro.dq + e, aq);
    st_f32(ro.dk + e, ak);
    ro.dg[e] = ag;
    if (e % D == 0) {
      const int64_t r = e / D;
      float ab = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) ab += ro.pb[s * rows + r];
      ro.dbeta[r] = ab;
    }
  }
}

template <int NS, typename IO>
hipError_t launch_bwd(const BwdArgs& a) {
  const int64_t BH = a.B * a.H, rows = a.B * a.T * a.H;
  const int64_t npc = (a.T + kBwdPiece - 1) / kBwdPiece;
  RowOut<IO> ro{(IO*)a.dq, (IO*)a.dk, a.dg, a.dbeta, nullptr, nullptr, nullptr, nullptr};
  if (NS > 1) {  // the parts follow the states in the workspace
    float* parts = a.workspace + BH * (npc + kBwdPiece) * DD;
    ro.pq = parts;
    ro.pk = ro.pq + NS * rows * D;
    ro.pg = ro.pk + NS * rows * D;
    ro.pb = ro.pg + NS * rows * D;
  }
  hipLaunchKernelGGL((kda_bwd_kernel<NS, IO>), dim3((unsigned)(BH * NS)), dim3(NT), 0,
                     (hipStream_t)a.stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g,
                     a.beta, a.s0, (const IO*)a.dout, a.ds_final, (IO*)a.dv, a.ds0, a.B, a.T,
                     a.H, a.scale, a.workspace, ro);
  if (NS > 1) {
    int64_t nb = (rows * D + 255) / 256;
    if (nb > 4096) nb = 4096;
    hipLaunchKernelGGL((kda_bwd_combine<NS, IO>), dim3((unsigned)nb), dim3(256), 0,
                       (hipStream_t)a.stream, ro, rows);
  }
  return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_floats(int64_t B, int64_t T, int64_t H) {
  const int64_t npc = (T + kBwdPiece - 1) / kBwdPiece, rows = B * T * H;
  return B * H * (npc + kBwdPiece) * DD + kBwdSplit * rows * (3 * D + 1);
}

hipError_t launch_recurrent_bwd(const BwdArgs& a) {
  const int64_t BH = a.B * a.H;
  if (BH <= 0 || a.T <= 0 || BH * kBwdSplit > 0x7fffffffLL) return hipErrorInvalidValue;
  return a.io_bf16 ? launch_bwd<kBwdSplit, bf16_t>(a) : launch_bwd<kBwdSplit, float>(a);
}

}  // namespace kda
