// C-ABI entry points of libpa: argument checks, workspace layout and the
// launch sequence of one step (scatter; plan -> chunk -> row-wise split-K -> split merge).
#include <atomic>
#include <cfloat>
#include <cmath>
#include <mutex>
#include <vector>

#include "internal.h"
#include "chunk_pp.h"

namespace pa {

int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (dev >= int(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {

// ---------------------------------------------------------------- kernel timing
std::mutex g_prof_mu;
std::atomic<int32_t> g_prof_mask{0};
struct Timed {
  int kind;
  hipEvent_t start, stop;
};
std::vector<Timed> g_pending;
std::vector<hipEvent_t> g_spare;

hipEvent_t take_event() {
  hipEvent_t e = nullptr;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_spare.empty()) {
      e = g_spare.back();
      g_spare.pop_back();
    }
  }
  if (!e && hipEventCreate(&e) != hipSuccess) e = nullptr;
  return e;
}

}  // namespace

KernelTimer::KernelTimer(int kind, hipStream_t st) : kind_(kind), st_(st) {
  if (!(g_prof_mask.load() & (1 << kind))) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, st_) != hipSuccess) start_ = nullptr;
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, st_) != hipSuccess) return;
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_pending.push_back({kind_, start_, stop});
}

namespace {

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int check_dims(int32_t hkv, int32_t d, int32_t bs, int32_t dtype, int64_t nb, const char* who) {
  if (hkv <= 0 || hkv >= (1 << 15)) return fail(PA_ERR_INVALID, "%s: num_kv_heads %d out of range", who, hkv);
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, dtype);
  if (bs != kBlock) return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is built)", who, bs);
  if (d != 64 && d != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 are built)", who, d);
  if (nb <= 0 || nb * kBlock >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID, "%s: num_blocks %lld out of range", who, (long long)nb);
  return PA_OK;
}

}  // namespace

int64_t ranges_capacity(const StepShape& s) {
  int64_t cap = int64_t(device_cus()) * kMaxWavesPerCU;
  const int64_t want = option(PA_OPT_TARGET_ITEMS);
  if (want > cap) cap = want;
  const int64_t fixed = option(PA_OPT_SPLIT_TOKENS) / kBlock;
  if (fixed > 0) {
    const int64_t units = int64_t(s.num_tokens) * s.num_kv_heads * s.max_blocks_per_seq;
    int64_t n = (units + fixed - 1) / fixed;
    if (n > (int64_t(1) << 20)) n = int64_t(1) << 20;  // the plan lengthens ranges beyond this
    if (n > cap) cap = n;
  }
  return cap;
}

int verify_rows(int group) {
  const int cap = 16 / (group > 0 && group <= 16 ? group : 16);  // one 16-wide accumulator
  const int64_t v = option(PA_OPT_VERIFY_ROWS);
  // automatic: one row per record in the workspace layout.  run_attention
  // still takes records of up to `cap` rows on steps the decode kernel plans
  // by itself, in the same partial arrays (fewer, longer ranges); on planned
  // steps the chunk kernel measured faster on short queries (64 sequences x
  // 2..4 rows over contexts of 512-2048: 86-89 us against 92-99 us)
  if (v >= 1) return v < cap ? int(v) : cap;
  return 1;
}

Workspace layout_workspace(const StepShape& s, void* ws) {
  Workspace w{};
  const int64_t T = s.num_tokens > 0 ? s.num_tokens : 1;
  const int64_t G = s.num_kv_heads > 0 ? s.num_q_heads / s.num_kv_heads : 1;
  w.rows_cap = T;
  w.tiles_cap = T;
  w.ranges_cap = ranges_capacity(s);
  w.ncol = int32_t(G * verify_rows(int(G)));
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align_up(bytes);
    return r;
  };
  w.hdr = reinterpret_cast<int32_t*>(take(H_WORDS * sizeof(int32_t)));
  w.hdr64 = reinterpret_cast<int64_t*>(w.hdr ? w.hdr + H64 : nullptr);
  w.rows = reinterpret_cast<int4*>(take(w.rows_cap * sizeof(int4)));
  w.rows_base = reinterpret_cast<int64_t*>(take(w.rows_cap * sizeof(int64_t)));
  w.tiles = reinterpret_cast<int2*>(take(w.tiles_cap * sizeof(int2)));
  w.tiles_tmp = reinterpret_cast<int4*>(take(w.tiles_cap * sizeof(int4)));
  w.range_row = reinterpret_cast<int32_t*>(take(w.ranges_cap * sizeof(int32_t)));
  w.range_cut = reinterpret_cast<int4*>(take(w.ranges_cap * sizeof(int4)));
  w.part_o = reinterpret_cast<float*>(take(size_t(2 * w.ranges_cap * w.ncol) * s.head_dim * sizeof(float)));
  w.part_ml = reinterpret_cast<float2*>(take(size_t(2 * w.ranges_cap * w.ncol) * sizeof(float2)));
  w.bytes = off;
  return w;
}

}  // namespace pa

using namespace pa;

extern "C" int pa_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping, void* k_cache,
                                    void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream) {
  clear_error();
  if (int rc = check_dims(num_kv_heads, head_dim, block_size, dtype, num_blocks, "pa_reshape_and_cache")) return rc;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_reshape_and_cache: num_tokens < 0");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: null pointer");
  const int32_t row_bytes = head_dim * (dtype == PA_BF16 ? 2 : 4);
  if (int64_t(num_tokens) * num_kv_heads * (row_bytes / 16) >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: num_tokens * num_kv_heads too large for one call");
  hipError_t e;
  {
    KernelTimer t(PA_K_RESHAPE, static_cast<hipStream_t>(stream));
    e = launch_reshape_and_cache(k, v, slot_mapping, k_cache, v_cache, num_tokens, num_kv_heads, row_bytes,
                                 num_blocks, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_reshape_and_cache: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq < 0)
    return 0;
  StepShape s{num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq};
  return layout_workspace(s, nullptr).bytes;
}

namespace pa {

int check_attention_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens,
                         float scale, float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t dtype, const char* who) {
  if (int rc = check_dims(num_kv_heads, head_dim, block_size, dtype, num_blocks, who)) return rc;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who, num_q_heads,
                num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "%s: query heads per kv head = %d (1, 2, 4 or 8 are built)", who, group);
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0) return fail(PA_ERR_INVALID, "%s: negative size", who);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale is not finite", who);
  if (num_tokens == 0 || num_seqs == 0) return PA_OK;
  if (max_blocks_per_seq == 0) return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq is 0 with query rows", who);
  if (int64_t(max_blocks_per_seq) * kBlock >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq too large", who);
  if (int64_t(num_kv_heads) * max_blocks_per_seq >= (int64_t(1) << 31))  // one row's pages over all kv heads
    return fail(PA_ERR_INVALID, "%s: num_kv_heads * max_blocks_per_seq too large", who);
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc || !context_lens || !out)
    return fail(PA_ERR_INVALID, "%s: null pointer", who);
  return PA_OK;
}

int run_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                  float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                  int32_t dtype, void* workspace, void* stream, const char* who) {
  const int group = num_q_heads / num_kv_heads;
  StepShape shape{num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq};

  Workspace w = layout_workspace(shape, workspace);
  const bool bf16 = dtype == PA_BF16;
  // short queries share their pages in one record: only the MFMA decode kernel
  // has the per-column causal limits (and the debug route keeps one row per record)
  const bool vr_auto = option(PA_OPT_VERIFY_ROWS) == 0;
  int vrows = bf16 && max_query_len > 1 && decode_uses_mfma(1) && !option(PA_OPT_FORCE_ROWWISE)
                  ? (vr_auto ? 16 / group : verify_rows(group))
                  : 1;
  // a small step whose sequences all fit one record each (by the hint): the
  // decode kernel plans it by itself, as records, and no chunk kernel runs (a
  // sequence longer than the hint says becomes several records)
  const bool self_records =
      vrows >= 2 && max_query_len <= vrows && num_tokens <= kSelfPlanRows && num_seqs <= kSelfPlanRows;
  if (vr_auto) {
    if (!self_records) {
      vrows = 1;  // automatic: records only where the decode kernel plans them itself
    } else {
      // the workspace was laid out for one-row records (G columns per partial
      // slot); the same partial arrays hold fewer ranges of G * vrows columns
      // (a self-planned step lengthens its ranges to fit)
      w.ranges_cap = w.ranges_cap * w.ncol / (int64_t(group) * vrows);
      w.ncol = group * vrows;
    }
  }
  // a decode-only step (every query of length <= 1) has no chunk tiles
  const bool use_mfma = !option(PA_OPT_FORCE_ROWWISE) && max_query_len > 1 && !self_records &&
                        chunk_supported(head_dim, group, bf16);
  hipStream_t st = static_cast<hipStream_t>(stream);

  PlanArgs pa_args{};
  pa_args.qsl = query_start_loc;
  pa_args.ctx = context_lens;
  pa_args.num_seqs = num_seqs;
  pa_args.num_tokens = num_tokens;
  pa_args.num_kv_heads = num_kv_heads;
  pa_args.max_len = max_blocks_per_seq * kBlock;
  pa_args.use_mfma = use_mfma ? 1 : 0;
  pa_args.fixed_units = int32_t(option(PA_OPT_SPLIT_TOKENS) / kBlock);
  {
    const int64_t want = option(PA_OPT_TARGET_ITEMS);
    int64_t n = want > 0 ? want : decode_waves(bf16 ? 1 : 0, head_dim, group);
    if (n > w.ranges_cap) n = w.ranges_cap;
    pa_args.num_ranges = int32_t(n < 1 ? 1 : n);
  }
  pa_args.tile_rows = use_mfma ? chunk_tile_rows(group) : 1;
  pa_args.verify_rows = vrows;
  // T = S * max_query_len: with a true hint every sequence has max_query_len rows, too many
  // for a row-wise record, so no row-wise row exists and the decode and merge kernels are not
  // launched.  The plan then sends every sequence to the chunk kernel, so a wrong hint (some
  // sequences shorter, others longer) still gets every row computed.
  const bool all_chunk = use_mfma && num_seqs > 0 && max_query_len > pa_args.verify_rows &&
                         int64_t(num_seqs) * max_query_len == num_tokens;
  pa_args.all_chunk = all_chunk ? 1 : 0;

  AttnArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.bt = block_tables;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.ctx = context_lens;
  a.out = out;
  a.scale_log2 = scale * 1.4426950408889634f;
  {
    const float mag = std::fabs(scale) * 1.4426950408889634f;
    if (mag < FLT_MIN) {  // zero (or below the normal range: every weight equal to fp32 precision)
      a.chunk_scale_log2 = 1.f;
      a.q_and = 0u;
      a.q_xor = 0u;
    } else {
      a.chunk_scale_log2 = mag;
      a.q_and = ~0u;
      a.q_xor = scale < 0.f ? 0x80008000u : 0u;
    }
  }
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.d = head_dim;
  a.mbps = max_blocks_per_seq;
  a.nb = num_blocks;
  a.bf16 = bf16 ? 1 : 0;
  a.merge_rows = pa_args.verify_rows;
  // a small decode-only step on the MFMA decode kernel skips the plan kernel:
  // every decode workgroup plans the (few) rows itself; so does a small step
  // of short-query records
  a.self_plan = (max_query_len <= 1 && bf16 && decode_uses_mfma(1) && num_tokens <= kSelfPlanRows &&
                 num_seqs <= kSelfPlanRows) ||
                self_records;
  // a small step with chunks skips it too: the chunk kernel plans its tiles and
  // the MFMA decode kernel the single-row sequences (short-query records need
  // the plan kernel)
  a.all_chunk = all_chunk ? 1 : 0;
  {
    const int64_t tiles_bound = use_mfma ? int64_t(num_tokens) / chunk_tile_rows(group) + num_seqs : 0;
    const bool sortable = num_seqs <= kChunkSortSeqs && tiles_bound <= kChunkSortTiles &&
                          tiles_bound * num_seqs <= kChunkSortPairs;
    const bool can = use_mfma && pa_args.verify_rows == 1 && decode_uses_mfma(1) && num_seqs <= kSelfPlanRows &&
                     option(PA_OPT_CHUNK_KERNEL) != 2;
    a.chunk_self_plan = can && (num_tokens <= kChunkSelfPlanTokens || (all_chunk && sortable)) ? (sortable ? 2 : 1) : 0;
  }
  if (a.chunk_self_plan && !all_chunk) {
    a.self_plan = 1;
    a.self_skip_chunks = 1;
  }
  // on request, the eight-wavefront chunk kernel (its tiles are twice as long)
  const bool chunk_pp = use_mfma && !a.chunk_self_plan && chunk_pp_selected(head_dim, group, bf16 ? 1 : 0, max_query_len);
  if (chunk_pp) pa_args.tile_rows = chunk_pp_tile_rows(group);
  a.fixed_units = pa_args.fixed_units;
  a.num_ranges = pa_args.num_ranges;
  a.max_len = pa_args.max_len;

  hipError_t e = hipSuccess;
  if (!a.self_plan && !a.chunk_self_plan) {
    KernelTimer t(PA_K_PLAN, st);
    e = launch_plan(pa_args, w, st);
  }
  if (e == hipSuccess && use_mfma) {
    KernelTimer t(PA_K_CHUNK, st);
    e = chunk_pp ? launch_chunk_pp(a, w, group, st) : launch_chunk(a, w, group, st);
  }
  if (e == hipSuccess && !all_chunk) {
    KernelTimer t(PA_K_DECODE, st);
    e = launch_decode(a, w, group, st);
  }
  if (e == hipSuccess && !all_chunk) {
    KernelTimer t(PA_K_MERGE, st);
    // automatic ranges number at most num_ranges; fixed-length ones up to the capacity
    e = launch_merge(a, w, group, pa_args.fixed_units > 0 ? w.ranges_cap : pa_args.num_ranges, st);
  }
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

extern "C" int pa_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* seq_lens, const int32_t* query_start_loc, const int32_t* context_lens,
                            float scale, float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_query_len, int32_t dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  clear_error();
  static const char* who = "pa_attention";
  if (int rc = check_attention_args(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale,
                                    out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                                    num_blocks, max_blocks_per_seq, dtype, who))
    return rc;
  if (num_tokens == 0 || num_seqs == 0) return PA_OK;
  StepShape shape{num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq};
  const size_t need = layout_workspace(shape, nullptr).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "pa_attention: workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_ERR_WORKSPACE, "pa_attention: workspace must be 256-byte aligned");
  return run_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out,
                       num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                       max_query_len, dtype, workspace, stream, who);
}

extern "C" int pa_attention_flags(const void* workspace, int32_t* flags, int32_t clear, void* stream) {
  clear_error();
  static const char* who = "pa_attention_flags";
  const void* ws = workspace ? workspace : noalloc_scratch(who);
  if (!ws) return PA_ERR_HIP;
  int32_t* word = static_cast<int32_t*>(const_cast<void*>(ws)) + H_FLAGS;  // the header opens the workspace
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (flags) {
    int32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: read-back failed: %s", who, hipGetErrorString(e));
    *flags = v;
  }
  if (clear) {
    const hipError_t e = hipMemsetAsync(word, 0, sizeof(int32_t), st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: clear failed: %s", who, hipGetErrorString(e));
  }
  return PA_OK;
}

extern "C" int pa_profile_enable(int32_t mask) {
  clear_error();
  if (mask < 0 || mask >= (1 << PA_K_COUNT)) return fail(PA_ERR_INVALID, "pa_profile_enable: bad mask %d", mask);
  g_prof_mask = mask;
  return PA_OK;
}

extern "C" int pa_profile_read(int64_t* counts, double* total_ms) {
  clear_error();
  std::vector<Timed> pend;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    pend.swap(g_pending);
  }
  int64_t c[PA_K_COUNT] = {0};
  double ms[PA_K_COUNT] = {0};
  int rc = PA_OK;
  for (const Timed& t : pend) {
    float x = 0.f;
    if (hipEventSynchronize(t.stop) == hipSuccess && hipEventElapsedTime(&x, t.start, t.stop) == hipSuccess) {
      c[t.kind] += 1;
      ms[t.kind] += x;
    } else {
      rc = fail(PA_ERR_HIP, "pa_profile_read: event query failed");
    }
  }
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (const Timed& t : pend) {
      g_spare.push_back(t.start);
      g_spare.push_back(t.stop);
    }
  }
  for (int k = 0; k < PA_K_COUNT; ++k) {
    if (counts) counts[k] = c[k];
    if (total_ms) total_ms[k] = ms[k];
  }
  return rc;
}
