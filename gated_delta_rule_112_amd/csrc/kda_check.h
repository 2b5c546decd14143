// Input-check mode (KDA_CHECK_INPUTS=1): interface between the C ABI and the
// check kernels of kda_check.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace kda {

enum CheckKind {
  kCheckFiniteF32 = 0,    // every float32 element finite
  kCheckFiniteBF16 = 1,   // every bfloat16 element finite
  kCheckRangeF32 = 2,     // every float32 element in [lo, hi]
  kCheckRowNormBF16 = 3,  // every row of d bfloat16 elements: norm in [lo, hi] or zero
};

struct CheckItem {
  const void* p;  // device tensor, or NULL to skip
  int64_t n;      // elements (rows for kCheckRowNormBF16)
  int kind;
  int d;          // row length (kCheckRowNormBF16)
  float lo, hi;
};

// True when the environment asks for the check (KDA_CHECK_INPUTS=1).
bool check_mode_on();

// Runs the checks of items[0 .. n) (at most 32) on `stream`, waits for them and
// sets *bad when any failed.  Returns the first runtime error, if any.
hipError_t check_inputs(const CheckItem* items, int n, void* stream, bool* bad);

}  // namespace kda
