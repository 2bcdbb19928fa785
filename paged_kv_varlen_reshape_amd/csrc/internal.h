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
constexpr int kPlanThreads = 1024;
constexpr int kMaxWavesPerCU = 32;  // upper bound of resident wavefronts per CU (8 per SIMD)
// Work queues of the chunk kernel: one per XCD of the MI355X (8 XCDs of 32 CUs,
// each with its own L2).  Workgroups are dispatched to the XCDs round robin, so
// workgroup b runs on XCD b % kXcdQueues.
constexpr int kXcdQueues = 8;

// ---------------------------------------------------------------- workspace
// Plan header words at the start of the workspace: int32 words, then int64
// words from index H64 on.
enum PlanHeader : int {
  H_ROWS = 0,     // row-wise rows
  H_TILES = 1,    // query tiles of the MFMA chunk kernel
  H_RANGES = 2,   // decode ranges (one wavefront each, in stream order)
  H_FLAGS = 3,    // sticky PA_FLAG_* bits: metadata a kernel had to clamp (never cleared by a kernel)
  H_QUEUE = 8,    // kXcdQueues dynamic work counters of the chunk kernel (words 8..15)
  H64 = 16,       // int64 words follow
  H64_UNITS = 0,  // (row, kv head, page) units of all row-wise rows
  H64_PER = 1,    // units per decode range
  H_WORDS = 64
};

// Decode work is a stream of units in (row, kv head, page) order: row r owns
// units [rows_base[r], rows_base[r] + Hkv * pages_r), kv head k of it the k-th
// run of pages_r.  The stream is cut into ranges of equal length, one
// wavefront each.  A (row, kv head) that a range boundary cuts leaves partial
// results in two slots per range: slot 0 for the range's first segment, slot 1
// for its last; split_merge folds them, reading only the pair's merge record.
struct Workspace {
  int64_t* hdr64;      // hdr + H64
  int32_t* hdr;        // [H_WORDS]
  int4* rows;          // [rows_cap]   {first token row, seq, keys seen by its last row, query rows nq}:
                       //   nq consecutive rows of one sequence (nq > 1: a short query whose
                       //   rows share every K/V page, one accumulator column per row and head)
  int64_t* rows_base;  // [rows_cap]   first unit of each row
  int2* tiles;         // [tiles_cap]  {seq, first query row of the tile within the sequence},
                       //   longest first
  int4* tiles_tmp;     // [tiles_cap]  plan scratch: tiles in sequence order with their bucket
  int32_t* range_row;  // [ranges_cap] row holding each range's first unit
  int4* range_cut;     // [ranges_cap] merge record of the (row, kv head) pair first cut by this
                       //   range's start (cut_record), or x = -1
  float* part_o;       // [2 * ranges_cap * ncol * D] unnormalised partial outputs
  float2* part_ml;     // [2 * ranges_cap * ncol]     partial (max, sum), log2 domain
  int64_t rows_cap, tiles_cap, ranges_cap;
  int32_t ncol;        // columns per partial slot: G * (most query rows of one record)
  size_t bytes;
};

struct StepShape {
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq;
};

// Decode ranges the workspace must hold for this shape.
int64_t ranges_capacity(const StepShape& s);
// Most query rows one row-wise record may hold for this group size (option, else 16 / group).
int verify_rows(int group);

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
  int32_t fixed_units;    // >0: units per decode range
  int32_t num_ranges;     // automatic: spread the units over this many ranges
  int32_t tile_rows;      // query rows per chunk-kernel tile
  int32_t verify_rows;    // >1: sequences with 2..verify_rows query rows become one row-wise
                          //   record (their rows share the K/V pages); 1: one record per row
  int32_t all_chunk;      // 1: every sequence with query rows goes to the chunk kernel (the step
                          //   launches no row-wise kernel)
};
hipError_t launch_plan(const PlanArgs& a, const Workspace& w, hipStream_t st);

// PA_FLAG_ROWS if the rows of one sequence (query_start_loc r0..r1, cached
// context ctx) are not consistent with the step, i.e. if the plans clamp them:
// rows outside [0, num_tokens), a negative count or context, or more keys than
// the block-table row holds.
__device__ __forceinline__ int rows_flag(int64_t r0, int64_t r1, int64_t ctx, int64_t num_tokens, int64_t max_len) {
  return (r1 < r0 || r0 < 0 || r1 > num_tokens || ctx < 0 || ctx + (r1 - r0) > max_len) ? PA_FLAG_ROWS : 0;
}

// Units (pages of 16 keys) of the rows whose key counts are 1..n:
// sum over p = 1..n of ceil(p / 16).
__device__ __forceinline__ int64_t pages_upto(int64_t n) {
  const int64_t a = n / kBlock, b = n - a * kBlock;
  return kBlock * a * (a + 1) / 2 + b * (a + 1);
}

// Merge record of the (row, kv head) pair whose units are [f, f + pages) when
// the range starting at g * per is the first boundary strictly inside it
// (0 < g * per - f <= per): {first token row of the record, kv head | query
// rows << 16, first range g0 of the pair, parts << 1 | slot of g0's part}.
// The pair's parts are the segments of ranges g0 .. (f + pages - 1) / per;
// g0's part is its last segment (slot 1) unless the pair starts g0 (slot 0).
__device__ __forceinline__ int4 cut_record(int64_t f, int64_t pages, int64_t per, int tok, int kvh, int nq) {
  const int64_t g0 = f / per, g1 = (f + pages - 1) / per;
  return make_int4(tok, kvh | (nq << 16), int(g0), int(2 * (g1 - g0 + 1)) | (f != g0 * per ? 1 : 0));
}

// Most rows (and sequences) of a step that the MFMA decode kernel plans by
// itself, without the plan kernel; also the most sequences of a step the chunk
// kernel plans by itself.
constexpr int kSelfPlanRows = 512;
// Most query tokens of a step the chunk kernel plans by itself in any case.
constexpr int kChunkSelfPlanTokens = 2048;
// A self-planned step whose tiles the chunk kernel can also put longest first
// (it ranks every tile against every sequence in LDS): at most this many
// sequences, tiles (an upper bound: tokens / tile rows + sequences) and
// tile-sequence pairs.  Such a step self-plans at any size when every sequence
// goes to the chunk kernel.
constexpr int kChunkSortSeqs = 64;
constexpr int kChunkSortTiles = 1024;
constexpr int kChunkSortPairs = 16384;

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
  // The chunk kernel takes row maxima of raw scores and multiplies them by a
  // positive factor, chunk_scale_log2 = |scale| * log2(e) (1 for a zero scale);
  // the rest of the scale goes into its Q operand, each dword ANDed with q_and
  // and XORed with q_xor: a negative scale flips every bf16 sign bit (exact:
  // every score changes sign and nothing else), a zero scale zeroes Q (every
  // score exactly 0, as scale * <q, K> is).  Identity: q_and = ~0, q_xor = 0.
  float chunk_scale_log2;
  uint32_t q_and, q_xor;
  int32_t num_seqs, num_tokens, hq, hkv, d, mbps;
  int64_t nb;
  int32_t bf16;
  int32_t merge_rows;  // most query rows of one row-wise record this step (the plan's verify_rows)
  int32_t self_plan;   // 1: the MFMA decode kernel plans the step's row-wise rows by itself (no plan kernel)
  int32_t self_skip_chunks;  // with self_plan: sequences with more than one query row belong to the chunk kernel
  int32_t chunk_self_plan;   // the chunk kernel plans the step by itself (no plan kernel): 1 tiles in
                             //   sequence order, 2 longest first
  int32_t all_chunk;         // 1: every sequence with query rows goes to the chunk kernel (the plan's all_chunk)
  int32_t fixed_units, num_ranges, max_len;  // the plan's range parameters, for self_plan
};
hipError_t launch_decode(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
// Resident decode wavefronts on the current device for this kernel instance.
int decode_waves(int bf16, int head_dim, int group);
// Page buffers per decode wavefront (option, else by group size).
int decode_buffers(int group);
// The bf16 MFMA decode kernel (decode_mfma.hip).
hipError_t launch_decode_mfma(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
int decode_mfma_waves(int head_dim, int group);
// Row-wise decode runs on the MFMA kernel (option, else bf16).
bool decode_uses_mfma(int bf16);
// max_ranges: an upper bound on the plan's range count (sizes the grid)
hipError_t launch_merge(const AttnArgs& a, const Workspace& w, int group, int64_t max_ranges, hipStream_t st);
hipError_t launch_chunk(const AttnArgs& a, const Workspace& w, int group, hipStream_t st);
bool chunk_supported(int head_dim, int group, int bf16);
int chunk_tile_rows(int group);

int device_cus();
// The current device's static workspace of pa_attention_noalloc (nullptr, with the
// error set, if it cannot be found).
void* noalloc_scratch(const char* who);

// pa_attention's argument checks (PA_OK, or the error it reports for `who`) and
// its launch sequence on an already checked call with a workspace of at least
// layout_workspace(...).bytes at a 256-byte-aligned device address.
int check_attention_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens,
                         float scale, float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t dtype, const char* who);
int run_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                  float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                  int32_t dtype, void* workspace, void* stream, const char* who);

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
