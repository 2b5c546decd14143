// Placeholder: the matrix-core prefill kernel is not built yet.
#include "kda_launch.h"
namespace kda {
bool chunk_mfma_supports(int, int, bool) { return false; }
hipError_t launch_chunk_mfma(const ChunkArgs&) { return hipErrorNotSupported; }
}  // namespace kda
