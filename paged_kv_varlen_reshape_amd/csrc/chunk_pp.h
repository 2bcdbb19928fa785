// The eight-wavefront chunk kernel (chunk_pp.hip): the launcher and the host
// rule that picks it over the four-wavefront kernel of chunk.hip.
#pragma once

#include "internal.h"

namespace pa {

// Query rows (tokens x heads of one kv head) of one chunk_pp work item.
constexpr int kPPRows = 256;

// Head sizes and group sizes chunk_pp is built for.
bool chunk_pp_supported(int head_dim, int group, int bf16);
// Tokens per chunk_pp tile (the plan's tile_rows when it runs).
int chunk_pp_tile_rows(int group);
// Whether a planned step takes chunk_pp (PA_OPT_CHUNK_KERNEL = 2; never by default).
bool chunk_pp_selected(int head_dim, int group, int bf16, int32_t max_query_len);

hipError_t launch_chunk_pp(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);

}  // namespace pa
