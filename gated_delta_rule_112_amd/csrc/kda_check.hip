// Input-check mode (KDA_CHECK_INPUTS=1): before a call launches its kernels,
// its floating-point inputs are scanned on the device for values outside what
// the method takes, and the call returns KDA_ERR_INPUT_RANGE instead of
// running on them.
//
// What is checked ("Kimi K3: Engineering a 2.8 Trillion Parameter Frontier",
// section "Dimension 1": the log-decay is bounded below by -5 through a scaled
// sigmoid, which keeps exp(-sum of g) over a 16-token tile finite):
//   finite      every element of a float32 or bfloat16 tensor is finite
//   range       every float32 element lies in [lo, hi] (NaN fails)
//   row norm    every row of d bfloat16 elements has an L2 norm in [lo, hi],
//               or is all zero (the raw q and k of the normalising entry
//               points on the matrix-core path)
// Each item of a call sets its own bit of a flag word when it finds a bad
// element; the host reads the word back and waits for it.  Flag words live in
// a small array in device memory (module scope), one word per call in flight:
// the host hands out the words round robin, so up to kSlots checked calls may
// overlap.
#include <atomic>

#include "kda_check.h"
#include "kda_device.h"

namespace kda {
namespace {

constexpr int kSlots = 64;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned int check_flags[kSlots];

__global__ void clear_flag_kernel(unsigned int* flag) { *flag = 0u; }

__device__ __forceinline__ bool bf16_finite(unsigned short b) { return (b & 0x7f80u) != 0x7f80u; }

__global__ void __launch_bounds__(256)
check_kernel(const void* __restrict__ p, int64_t n, int kind, int d, float lo, float hi,
             unsigned int bit, unsigned int* flag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    switch (kind) {
      case kCheckFiniteF32: {
        const float x = ((const float*)p)[i];
        bad |= !isfinite(x);
        break;
      }
      case kCheckFiniteBF16:
        bad |= !bf16_finite(((const unsigned short*)p)[i]);
        break;
      case kCheckRangeF32: {
        const float x = ((const float*)p)[i];
        bad |= !(x >= lo && x <= hi);
        break;
      }
      case kCheckRowNormBF16: {  // element i is row i of d elements
        const unsigned short* r = (const unsigned short*)p + i * d;
        float ss = 0.f;
        bool fin = true;
        for (int j = 0; j < d; ++j) {
          fin &= bf16_finite(r[j]);
          const float x = __builtin_bit_cast(float, (unsigned)r[j] << 16);
          ss = fmaf(x, x, ss);
        }
        bad |= !fin || !(ss == 0.f || (ss >= lo * lo && ss <= hi * hi));
        break;
      }
      default:
        bad = true;
    }
  }
  if (__any(bad) && threadIdx.x % 64 == 0) atomicOr(flag, bit);
}

// Device address of this device's check_flags, looked up once per device.
unsigned int* flags_on_current_device(hipError_t* err) {
  static std::atomic<unsigned int*> ptr[kMaxDevices];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  unsigned int* p = ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* a = nullptr;
    *err = hipGetSymbolAddress(&a, HIP_SYMBOL(check_flags));
    if (*err != hipSuccess) return nullptr;
    p = (unsigned int*)a;
    ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

bool check_mode_on() {
  const char* e = getenv("KDA_CHECK_INPUTS");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

hipError_t check_inputs(const CheckItem* items, int n, void* stream, bool* bad) {
  static std::atomic<unsigned int> next_slot{0};
  *bad = false;
  hipError_t err;
  unsigned int* flags = flags_on_current_device(&err);
  if (flags == nullptr) return err;
  unsigned int* flag = flags + next_slot.fetch_add(1, std::memory_order_relaxed) % kSlots;
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s, flag);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  for (int i = 0; i < n && i < 32; ++i) {
    const CheckItem& it = items[i];
    if (it.p == nullptr || it.n <= 0) continue;
    int64_t blocks = (it.n + 255) / 256;
    blocks = blocks < 4096 ? blocks : 4096;
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, it.p, it.n,
                       it.kind, it.d, it.lo, it.hi, 1u << i, flag);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  unsigned int host = 0;
  if ((err = hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return err;
  if ((err = hipStreamSynchronize(s)) != hipSuccess) return err;
  *bad = host != 0u;
  return hipSuccess;
}

}  // namespace kda
