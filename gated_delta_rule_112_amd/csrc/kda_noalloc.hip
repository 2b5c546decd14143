// kda_chunk_fwd_noalloc: the prefill for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It is kda_chunk_fwd with the workspace replaced by a
// fixed scratch array in device memory that the library declares at module
// scope: kScratchBytes per GPU, held until the process ends.
//
// The array's name is a host-side stand-in, not a device address.  The first
// call on a device (that device current) looks up its address there with
// hipGetSymbolAddress and keeps it per device; only that address is handed to
// the kernels.  The matrix-core path fits its segments of per-pair records to
// the array (shorter segments, so more launches than with the default
// workspace); every record and the carried state are written before they are
// read within one call, so nothing needs clearing between calls.  Every call
// on a GPU shares that GPU's array: calls that overlap in time on one GPU
// (concurrent streams or host threads) race and must be serialised by the
// caller.
#include <atomic>

#include "kda.h"
#include "kda_launch.h"

namespace kda {

kda_status chunk_fwd_fixed_scratch(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* s0, void* o, float* s_out,
                                   const void* gate, const float* norm_w, float eps, int64_t B,
                                   int64_t T, int64_t H, int dk, int dv, float scale,
                                   kda_dtype io, void* scratch, size_t scratch_bytes,
                                   void* stream);

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// This device's address of `scratch` (looked up on the first call per device).
void* scratch_on_current_device() {
  static std::atomic<void*> ptr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace kda

extern "C" {

size_t kda_chunk_fwd_noalloc_scratch_bytes(void) { return kda::kScratchBytes; }

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* s0, void* o, float* s_out,
                                 const void* gate, const float* norm_w, float eps, int64_t B,
                                 int64_t T, int64_t H, int dk, int dv, float scale, kda_dtype io,
                                 void* stream) {
  void* ws = kda::scratch_on_current_device();
  if (ws == nullptr) return KDA_ERR_LAUNCH;
  return kda::chunk_fwd_fixed_scratch(q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps, B, T, H,
                                      dk, dv, scale, io, ws, kda::kScratchBytes, stream);
}

}  // extern "C"
