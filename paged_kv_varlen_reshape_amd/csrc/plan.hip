// plan: turns the step's per-sequence metadata into device work lists, with no
// host synchronisation.
//
// The step is one flattened super-sequence (Inside vLLM summary, techfeed.io,
// section "PagedAttentionの仕組み") that mixes prefill chunks and single-token
// decodes (section "エンジンの中核：スケジューラとKVキャッシュ管理").  Each
// sequence's query rows go either to the MFMA chunk kernel (bf16 sequences
// with more than one query row, in tiles of kChunkRows rows) or to the
// row-wise split-K kernel (decodes, and every row when MFMA is off).  A
// row-wise row at absolute position p sees p+1 keys; it is cut into splits of
// P tokens, P chosen so that the whole step makes about `target_items`
// (row, kv head, split) items, never below kMinSplitTokens.
//
// One workgroup of 1024 threads walks the sequences, then the rows, in chunks
// of 1024 with block-wide scans.  It also clears the work counters the later
// kernels of the step use.
#include "internal.h"

namespace pa {
namespace {

constexpr int kWavesPerPlan = kPlanThreads / kWave;

// Exclusive scan over the workgroup; returns this thread's prefix, total in *total.
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* total, int64_t* sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int64_t inc = x;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == kWave - 1) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < kWavesPerPlan ? sh[lane] : 0;
#pragma unroll
    for (int d = 1; d < kWavesPerPlan; d <<= 1) {
      const int64_t y = __shfl_up(w, d);
      if (lane >= d) w += y;
    }
    if (lane < kWavesPerPlan) sh[kWavesPerPlan + lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  const int64_t before = wave ? sh[kWavesPerPlan + wave - 1] : 0;
  *total = sh[2 * kWavesPerPlan - 1];
  __syncthreads();
  return before + inc - x;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(PlanArgs a, Workspace w) {
  __shared__ int64_t sh[2 * kWavesPerPlan];
  const int tid = threadIdx.x;
  int64_t rows = 0, tiles = 0, keys = 0;

  // pass 1: rows and tiles of every sequence
  for (int base = 0; base < a.num_seqs; base += kPlanThreads) {
    const int i = base + tid;
    int64_t nrow = 0, ntile = 0, nkey = 0;
    int32_t q = 0, c = 0, r0 = 0;
    if (i < a.num_seqs) {
      r0 = a.qsl[i];
      q = a.qsl[i + 1] - r0;
      c = a.ctx[i];
      // metadata is trusted, but nothing below may index outside the arrays
      if (q < 0) q = 0;
      if (r0 < 0 || r0 >= a.num_tokens) q = 0;
      if (q > a.num_tokens - r0) q = a.num_tokens - r0;
      if (c < 0) c = 0;
      if (int64_t(c) + q > a.max_len) q = c >= a.max_len ? 0 : a.max_len - c;
      if (q > 1 && a.use_mfma) {
        ntile = (q + kChunkRows - 1) / kChunkRows;
      } else if (q > 0) {
        nrow = q;
        nkey = int64_t(q) * c + int64_t(q) * (q + 1) / 2;
      }
    }
    int64_t tot_r, tot_t, tot_k;
    const int64_t off_r = rows + block_exclusive_scan(nrow, &tot_r, sh);
    const int64_t off_t = tiles + block_exclusive_scan(ntile, &tot_t, sh);
    block_exclusive_scan(nkey, &tot_k, sh);
    for (int64_t j = 0; j < nrow && off_r + j < w.rows_cap; ++j) {
      w.row_tok[off_r + j] = r0 + int32_t(j);
      w.row_seq[off_r + j] = i;
      w.row_len[off_r + j] = c + int32_t(j) + 1;
    }
    for (int64_t t = 0; t < ntile && off_t + t < w.tiles_cap; ++t)
      w.tiles[off_t + t] = make_int2(i, int32_t(t) * kChunkRows);
    rows += tot_r;
    tiles += tot_t;
    keys += tot_k;
  }

  // split partition
  int64_t P;
  if (a.fixed_split > 0) {
    P = a.fixed_split;
  } else {
    const int64_t want = (keys * a.num_kv_heads + a.target_items - 1) / a.target_items;
    P = (want + kBlock - 1) / kBlock * kBlock;
    if (P < kMinSplitTokens) P = kMinSplitTokens;
    if (P > (int64_t(1) << 30)) P = int64_t(1) << 30;
  }
  if (rows > w.rows_cap) rows = w.rows_cap;
  if (tiles > w.tiles_cap) tiles = w.tiles_cap;
  __syncthreads();  // row_* written above are read by other threads below

  // pass 2: splits per row, item records, reduce list
  int64_t splits = 0, nred = 0;
  for (int base = 0; base < rows; base += kPlanThreads) {
    const int64_t r = base + tid;
    int64_t ns = 0;
    int32_t tok = 0, seq = 0, len = 0;
    if (r < rows) {
      tok = w.row_tok[r];
      seq = w.row_seq[r];
      len = w.row_len[r];
      ns = (len + P - 1) / P;
    }
    int64_t tot_s, tot_red;
    const int64_t u0 = splits + block_exclusive_scan(ns, &tot_s, sh);
    const int64_t red = nred + block_exclusive_scan(ns > 1 ? 1 : 0, &tot_red, sh);
    for (int64_t s = 0; s < ns && u0 + s < w.splits_cap; ++s)
      w.items[u0 + s] = make_int4(tok, seq, len, int32_t(s) | (ns == 1 ? kSingleSplit : 0));
    if (ns > 1 && u0 + ns <= w.splits_cap) w.reduce[red] = make_int4(tok, int32_t(u0), int32_t(ns), 0);
    splits += tot_s;
    nred += tot_red;
  }

  if (splits > w.splits_cap) splits = w.splits_cap;  // only with inconsistent metadata
  if (nred > w.rows_cap) nred = w.rows_cap;
  if (tid == 0) {
    w.hdr[H_ROWS] = int32_t(rows);
    w.hdr[H_SPLITS] = int32_t(splits);
    w.hdr[H_SPLIT_TOKENS] = int32_t(P);
    w.hdr[H_TILES] = int32_t(tiles);
    w.hdr[H_REDUCE] = int32_t(nred);
    w.hdr[H_COUNTER] = 0;
    w.hdr[H_COUNTER2] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, const Workspace& w, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a, w);
  return hipGetLastError();
}

}  // namespace pa
