// chunk_mfma.hip -- chunked gated delta rule on bf16 matrix cores (placeholder until the kernels land).
#include "common.h"
#include "launch.h"

namespace gdn {

bool chunk_mfma_supported(int, int, gdn_dtype) { return false; }
size_t chunk_mfma_workspace_size(int, int, int, int, int, int) { return 0; }
hipError_t launch_chunk_mfma(const ChunkArgs&) { return hipErrorNotSupported; }

}  // namespace gdn
