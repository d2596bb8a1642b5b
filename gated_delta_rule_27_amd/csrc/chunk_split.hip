// chunk_split.hip — two-kernel chunk path (per-channel gate).  Placeholder
// until the kernels land: reports the configuration as unsupported.
#include "launch.h"

namespace linattn {

bool chunk_split_supported(const ChunkProblem&) { return false; }
size_t chunk_split_workspace_bytes(const ChunkProblem&) { return 0; }
hipError_t launch_chunk_split(const ChunkProblem&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace linattn
