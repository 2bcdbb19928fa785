// pa_validate_metadata: host-side consistency check of one step's index arrays.
//
// The device calls trust their metadata (checking it there would need a
// device->host copy per step); this routine checks host copies once, e.g. in
// tests or behind a debug flag of the caller.
#include <vector>

#include "errors.h"

extern "C" int pa_validate_metadata(const int32_t* bt, const int32_t* seq_lens, const int32_t* qsl,
                                    const int32_t* ctx, const int32_t* slots, int32_t num_seqs,
                                    int32_t num_tokens, int32_t mbps, int64_t num_blocks,
                                    int32_t block_size) {
  pa::clear_error();
  if (num_seqs < 0 || num_tokens < 0 || mbps < 0 || num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "validate: negative or zero size");
  if (!qsl || (num_seqs > 0 && (!seq_lens || !ctx || (!bt && mbps > 0))))
    return pa::fail(PA_ERR_INVALID, "validate: null array");
  if (qsl[0] != 0) return pa::fail(PA_ERR_INVALID, "validate: query_start_loc[0] = %d, not 0", qsl[0]);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t q = int64_t(qsl[i + 1]) - qsl[i];
    if (q < 0) return pa::fail(PA_ERR_INVALID, "validate: query_start_loc decreases at %d", i);
    if (ctx[i] < 0) return pa::fail(PA_ERR_INVALID, "validate: context_lens[%d] < 0", i);
    if (int64_t(seq_lens[i]) != int64_t(ctx[i]) + q)
      return pa::fail(PA_ERR_INVALID, "validate: seq_lens[%d] = %d != context %d + query %lld", i,
                      seq_lens[i], ctx[i], (long long)q);
    const int64_t nblk = (int64_t(seq_lens[i]) + block_size - 1) / block_size;
    if (nblk > mbps)
      return pa::fail(PA_ERR_INVALID, "validate: sequence %d needs %lld blocks > max_blocks_per_seq %d", i,
                      (long long)nblk, mbps);
    for (int64_t b = 0; b < nblk; ++b) {
      const int32_t id = bt[int64_t(i) * mbps + b];
      if (id < 0 || id >= num_blocks)
        return pa::fail(PA_ERR_INVALID, "validate: block_tables[%d][%lld] = %d out of [0, %lld)", i,
                        (long long)b, id, (long long)num_blocks);
    }
  }
  if (qsl[num_seqs] != num_tokens)
    return pa::fail(PA_ERR_INVALID, "validate: query_start_loc[num_seqs] = %d != num_tokens %d", qsl[num_seqs],
                    num_tokens);
  if (slots) {
    const int64_t nslots = num_blocks * block_size;
    std::vector<char> seen(size_t(nslots), 0);
    for (int32_t n = 0; n < num_tokens; ++n) {
      const int32_t s = slots[n];
      if (s < 0) continue;
      if (s >= nslots) return pa::fail(PA_ERR_INVALID, "validate: slot_mapping[%d] = %d out of range", n, s);
      if (seen[s]) return pa::fail(PA_ERR_INVALID, "validate: slot %d used twice", s);
      seen[s] = 1;
    }
  }
  return PA_OK;
}
