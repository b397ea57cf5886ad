// kda_bwd.hip -- chunked backward (placeholder until the kernels land).
#include "kda_chunk.cuh"
#include "kda_internal.h"

namespace kda {
hipError_t launch_bwd(const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
