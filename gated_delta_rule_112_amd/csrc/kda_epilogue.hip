// Standalone output epilogue: head-wise RMSNorm followed by a sigmoid gate.
//
// "Kimi K3 Architecture Explained ...", section "Token mixing": the output gate
// is applied after a head-wise RMSNorm.  Per row r (one head's dv vector):
//   y[r] = x[r] * rsqrt(mean(x[r]^2) + eps) * w * sigmoid(gate[r])
// The prefill and decode kernels fuse the same arithmetic into their output
// write; this kernel is the unfused form.  It streams x and gate once and
// writes y once (bound by HBM); y may be x (in place: each lane reads its
// elements before writing the same ones).  dv/4 lanes own one row, a float4 (or four
// bfloat16) each, and reduce the sum of squares with lane shuffles.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kNormThreads = 256;

template <int DV, typename IO>
__global__ void __launch_bounds__(kNormThreads)
kda_gate_rmsnorm_kernel(const IO* x, const IO* __restrict__ gate,
                        const float* __restrict__ norm_w, IO* y, int64_t rows, float eps) {
  constexpr int LPR = DV / 4;                       // lanes per row
  constexpr int RPB = kNormThreads / LPR;           // rows per block
  const int lane = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const bool live = row < rows;
  f32x4 xv = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    xv = ld4(x + row * DV + 4 * lane);
    gv = ld4(gate + row * DV + 4 * lane);
  }
  float ss = xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3];
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (!live) return;
  const float inv = rsqrtf(ss / (float)DV + eps);
  f32x4 w = {1.f, 1.f, 1.f, 1.f};
  if (norm_w) w = *(const f32x4*)(norm_w + 4 * lane);
  f32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = xv[e] * inv * w[e] * sigmoidf_(gv[e]);
  st4(y + row * DV + 4 * lane, out);
}

template <int DV, typename IO>
static hipError_t launch_norm_t(const NormArgs& a) {
  constexpr int RPB = kNormThreads / (DV / 4);
  const int64_t nblk = (a.rows + RPB - 1) / RPB;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kda_gate_rmsnorm_kernel<DV, IO>), dim3((unsigned)nblk), dim3(kNormThreads),
                     0, (hipStream_t)a.stream, (const IO*)a.x, (const IO*)a.gate, a.norm_w,
                     (IO*)a.y, a.rows, a.eps);
  return hipGetLastError();
}

template <typename IO>
static hipError_t dispatch_norm(const NormArgs& a) {
  switch (a.dv) {
    case 16: return launch_norm_t<16, IO>(a);
    case 32: return launch_norm_t<32, IO>(a);
    case 64: return launch_norm_t<64, IO>(a);
    case 128: return launch_norm_t<128, IO>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gate_rmsnorm(const NormArgs& a) {
  return a.io_bf16 ? dispatch_norm<bf16_t>(a) : dispatch_norm<float>(a);
}

}  // namespace kda
