// KDA single-token decode step: one pass over the resident float32 state.
//
// Per (b, h), with a = exp(g) (per key channel):
//   p_j = sum_i a_i k_i S_ij        (what the decayed state predicts for k)
//   r_j = sum_i a_i q_i S_ij        (decayed state read by q)
//   u_j = beta (v_j - p_j)
//   o_j = scale (r_j + (q . k) u_j)                  = scale * S_new^T q
//   S_ij <- a_i S_ij + k_i u_j                       (in place)
// "Kimi K3 Architecture Explained ...", section "Token mixing": constant
// per-token decode cost against a fixed-size state.
//
// The kernel is bound by HBM: every state element is read once and written
// once (8 bytes per element per step).  One workgroup owns one (b, h) state;
// each thread holds a float4 column strip of RPT rows in registers for the
// whole step, so the write never re-reads memory.  A wavefront's float4 loads
// for one row index cover whole 512-byte rows, and all RPT loads of a thread
// are issued before the first use.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int DK, int DV>
struct DecodeShape {
  static constexpr int CG = DV / 4;                                   // float4 column groups
  static constexpr int RG = (DK < 256 / CG) ? DK : 256 / CG;          // row groups
  static constexpr int RPT = DK / RG;                                 // rows per thread
  static constexpr int NT = CG * RG;                                  // threads per block
  static_assert(NT <= 256 && NT % 64 == 0, "decode block must be whole wavefronts");
  static_assert(RPT * RG == DK, "rows must split evenly");
};

template <int DK, int DV, typename IO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
kda_decode_kernel(const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
                  const float* __restrict__ g, const float* __restrict__ beta,
                  float* __restrict__ state, IO* __restrict__ o,
                  const IO* __restrict__ gate, const float* __restrict__ norm_w,
                  float eps, float scale) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT;

  __shared__ float s_a[DK];         // a_i = exp(g_i)
  __shared__ float s_k[DK];         // k_i
  __shared__ float s_ak[DK];        // a_i * k_i
  __shared__ float s_aq[DK];        // a_i * q_i
  __shared__ float s_part[2][RG][DV];
  __shared__ float s_u[DV];
  __shared__ float s_qk;
  __shared__ float s_red[DV];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  float* Sp = state + bh * (int64_t)(DK * DV);

  // Issue every state load first: RPT independent float4 loads per thread.
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    s[m] = __builtin_nontemporal_load((const f32x4*)(Sp + i * DV + 4 * cg));
  }

  // Per-channel factors.
  if (tid < DK) {
    const float a = expf(g[bh * DK + tid]);
    const float kk = ld_f32(k + bh * DK + tid);
    const float qq = ld_f32(q + bh * DK + tid);
    s_a[tid] = a;
    s_k[tid] = kk;
    s_ak[tid] = a * kk;
    s_aq[tid] = a * qq;
  }
  // q . k over the undecayed vectors (one wavefront reduction).
  if (tid < 64) {
    float acc = 0.f;
    for (int i = tid; i < DK; i += 64) acc += ld_f32(q + bh * DK + i) * ld_f32(k + bh * DK + i);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (tid == 0) s_qk = acc;
  }
  __syncthreads();

  // Partial column sums over this thread's rows.
  f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    p += s_ak[i] * s[m];
    r += s_aq[i] * s[m];
  }
  *(f32x4*)&s_part[0][rg][4 * cg] = p;
  *(f32x4*)&s_part[1][rg][4 * cg] = r;
  __syncthreads();

  // Column j: finish the reductions, form u_j and o_j.
  const float bt = beta[bh];
  float oj = 0.f;
  if (tid < DV) {
    float pj = 0.f, rj = 0.f;
#pragma unroll 8
    for (int x = 0; x < RG; ++x) {
      pj += s_part[0][x][tid];
      rj += s_part[1][x][tid];
    }
    const float uj = bt * (ld_f32(v + bh * DV + tid) - pj);
    s_u[tid] = uj;
    oj = scale * (rj + s_qk * uj);
  }
  __syncthreads();

  // State update in place: S_ij <- a_i S_ij + k_i u_j.
  {
    const f32x4 u4 = *(const f32x4*)&s_u[4 * cg];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = rg + m * RG;
      const f32x4 nv = s_a[i] * s[m] + s_k[i] * u4;
      __builtin_nontemporal_store(nv, (f32x4*)(Sp + i * DV + 4 * cg));
    }
  }

  // Output, optionally through the head-wise RMSNorm x sigmoid(gate) epilogue.
  if (gate == nullptr) {
    if (tid < DV) st_f32(o + bh * DV + tid, oj);
    return;
  }
  if (tid < DV) s_red[tid] = oj * oj;
  __syncthreads();
  if (tid < 64) {
    float acc = 0.f;
    for (int j = tid; j < DV; j += 64) acc += s_red[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (tid == 0) s_qk = acc;  // reuse: sum of squares
  }
  __syncthreads();
  if (tid < DV) {
    const float inv = rsqrtf(s_qk / (float)DV + eps);
    const float w = norm_w ? norm_w[tid] : 1.f;
    const float gt = ld_f32(gate + bh * DV + tid);
    st_f32(o + bh * DV + tid, oj * inv * w * sigmoidf_(gt));
  }
}

template <int DK, int DV, typename IO>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  using Sh = DecodeShape<DK, DV>;
  const int64_t nblk = a.B * a.H;
  hipLaunchKernelGGL((kda_decode_kernel<DK, DV, IO>), dim3((unsigned)nblk), dim3(Sh::NT), 0,
                     (hipStream_t)a.stream, (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g,
                     a.beta, a.state, (IO*)a.o, (const IO*)a.gate, a.norm_w, a.eps, a.scale);
  return hipGetLastError();
}

template <typename IO>
static hipError_t dispatch_dims(const DecodeArgs& a) {
#define KDA_CASE(DKV, DVV) \
  if (a.dk == DKV && a.dv == DVV) return launch_decode_t<DKV, DVV, IO>(a);
#define KDA_ROW(DKV) KDA_CASE(DKV, 16) KDA_CASE(DKV, 32) KDA_CASE(DKV, 64) KDA_CASE(DKV, 128)
  KDA_ROW(16) KDA_ROW(32) KDA_ROW(64) KDA_ROW(128)
#undef KDA_ROW
#undef KDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.io_bf16 ? dispatch_dims<bf16_t>(a) : dispatch_dims<float>(a);
}

}  // namespace kda
