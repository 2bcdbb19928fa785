// Internal declarations shared by the libpa translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>

#include "errors.h"
#include "pa.h"

namespace pa {

// 16-byte lane chunk as a native vector (usable with the nontemporal builtins)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- fixed facts
constexpr int kBlock = 16;         // tokens per KV block
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kDecodeThreads = 256;  // 4 waves per decode workgroup
constexpr int kChunkRows = 32;     // query rows per MFMA chunk tile
constexpr int kPlanThreads = 1024;
constexpr int kMinSplitTokens = 256;   // smallest automatic split-K partition
constexpr int kDefaultTargetItems = 8192;

// ---------------------------------------------------------------- workspace
// Plan header words (int32) at the start of the workspace.
enum PlanHeader : int {
  H_ROWS = 0,          // rows taking the row-wise kernel
  H_SPLITS = 1,        // (row, split) items; decode work items = H_SPLITS * Hkv
  H_SPLIT_TOKENS = 2,  // split-K partition P in tokens
  H_TILES = 3,         // query tiles of the MFMA chunk kernel
  H_REDUCE = 4,        // rows with more than one split
  H_COUNTER = 8,       // dynamic work counter of the decode kernel
  H_COUNTER2 = 9,      // dynamic work counter of the chunk kernel
  H_WORDS = 64
};

// One (row, split) item of the row-wise kernel: query token row, sequence,
// keys the row sees (absolute position + 1), split index | kSingleSplit.
constexpr int kSingleSplit = 1 << 30;

struct Workspace {
  int32_t* hdr;        // [H_WORDS]
  int32_t* row_tok;    // [rows_cap]   token row of each row-wise row (plan scratch)
  int32_t* row_seq;    // [rows_cap]
  int32_t* row_len;    // [rows_cap]
  int32_t* split_base; // [rows_cap+1] prefix sums of splits per row (plan scratch)
  int4* items;         // [splits_cap] {tok, seq, len, split | kSingleSplit}
  int4* reduce;        // [rows_cap]   {tok, first item, splits, 0} for rows with >1 split
  int2* tiles;         // [tiles_cap]  {seq, first query row in the sequence}
  float* part_o;       // [splits_cap * Hq * D] unnormalised split outputs
  float2* part_ml;     // [splits_cap * Hq]     split (max, sum) in the log2 domain
  int64_t rows_cap, tiles_cap, splits_cap;
  size_t bytes;
};

struct StepShape {
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq;
};

// Carve the workspace (ws == nullptr: only compute sizes).
Workspace layout_workspace(const StepShape& s, void* ws);

// ---------------------------------------------------------------- launchers
hipError_t launch_reshape_and_cache(const void* k, const void* v, const int32_t* slots,
                                    void* kc, void* vc, int32_t ntok, int32_t hkv,
                                    int32_t row_bytes, int64_t num_blocks, hipStream_t st);

struct PlanArgs {
  const int32_t* qsl;
  const int32_t* ctx;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t max_len;        // max_blocks_per_seq * 16: rows never see more keys than this
  int32_t use_mfma;       // 1: sequences with >1 query rows go to the MFMA chunk kernel
  int32_t fixed_split;    // >0: split partition in tokens
  int32_t target_items;   // automatic split: aim at about this many (row, kv head, split) items
};
hipError_t launch_plan(const PlanArgs& a, const Workspace& w, hipStream_t st);

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int32_t* ctx;
  float* out;
  float scale_log2;  // scale * log2(e)
  int32_t num_seqs, num_tokens, hq, hkv, d, mbps;
  int64_t nb;
  int32_t bf16;
};
hipError_t launch_decode(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
hipError_t launch_reduce(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
hipError_t launch_chunk(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
bool chunk_supported(int head_dim, int group, int bf16);

int device_cus();

// Scoped HIP-event timing of one launch (active only when its kind is enabled).
class KernelTimer {
 public:
  KernelTimer(int kind, hipStream_t st);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int kind_;
  hipStream_t st_;
  hipEvent_t start_ = nullptr;
};

}  // namespace pa
