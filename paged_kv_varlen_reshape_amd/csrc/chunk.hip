// chunk_mfma: causal attention of multi-row (prefill chunk) sequences on bf16 MFMA.
// Not built yet: every row takes the row-wise kernel.
#include "internal.h"

namespace pa {
bool chunk_supported(int, int, int) { return false; }
int chunk_tile_rows(int) { return 32; }
hipError_t launch_chunk(const AttnArgs&, const Workspace&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pa
