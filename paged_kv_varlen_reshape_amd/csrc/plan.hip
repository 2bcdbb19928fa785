// plan: turns the step's per-sequence metadata into device work lists, with no
// host synchronisation.
//
// The step is one flattened super-sequence (Inside vLLM summary, techfeed.io,
// section "PagedAttentionの仕組み") that mixes prefill chunks and single-token
// decodes (section "エンジンの中核：スケジューラとKVキャッシュ管理").  Each
// sequence's query rows go either to the MFMA chunk kernel (bf16 sequences
// with more than one query row, in tiles of `tile_rows` rows) or to the
// row-wise decode kernel (decodes, and every row when MFMA is off).  A short
// query (2..verify_rows rows, as in speculative-decoding verification) is one
// row-wise record whose rows share every page of its last row.  A
// row-wise row at absolute position p sees p+1 keys, i.e. ceil((p+1)/16)
// pages per kv head; all those (row, kv head, page) units form one stream
// that is cut into equal ranges, one per decode wavefront.
//
// One workgroup of 1024 threads.  Pass 1 gives each thread a contiguous run of
// sequences and places every tile record, row record and row's first unit
// with one block scan; the tiles are then sorted longest first; pass 2 marks,
// for every range, the row holding its first unit and the (row, kv head) it
// cuts.  It also clears the work counters the chunk kernel uses.
#include "internal.h"

namespace pa {
namespace {

constexpr int kWavesPerPlan = kPlanThreads / kWave;
constexpr int kSortBuckets = kPlanThreads;  // key-count buckets of the tile sort, one per thread
constexpr int kSortBucketKeys = 64;         // keys per bucket (one chunk-kernel key tile)
constexpr int kSeqBatch = 4;                // sequences whose metadata loads are issued together
constexpr int kLdsRows = 8192;              // rows whose first units the range search keeps in LDS

// Exclusive scans of two non-negative int64 at once (one set of barriers).
__device__ void block_exclusive_scan2(int64_t x, int64_t y, int64_t* ox, int64_t* oy, int64_t* tx, int64_t* ty,
                                      int64_t* sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int64_t ix = x, iy = y;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t a = __shfl_up(ix, d), b = __shfl_up(iy, d);
    if (lane >= d) {
      ix += a;
      iy += b;
    }
  }
  if (lane == kWave - 1) {
    sh[wave] = ix;
    sh[kWavesPerPlan + wave] = iy;
  }
  __syncthreads();
  int64_t bx = 0, by = 0, sx = 0, sy = 0;
#pragma unroll
  for (int ww = 0; ww < kWavesPerPlan; ++ww) {
    const int64_t vx = sh[ww], vy = sh[kWavesPerPlan + ww];
    bx += ww < wave ? vx : 0;
    by += ww < wave ? vy : 0;
    sx += vx;
    sy += vy;
  }
  *ox = bx + ix - x;
  *oy = by + iy - y;
  *tx = sx;
  *ty = sy;
  __syncthreads();
}


struct SeqInfo {
  int32_t r0, q, c;
  bool chunk;   // query rows go to the chunk kernel in tiles
  bool group;   // query rows form one row-wise record (a short query)
};

// Sequence i's rows, clamped so that nothing below indexes outside the
// arrays (metadata is trusted).  Branch-free: an index past the last
// sequence (valid == false) loads sequence 0 and yields no rows, so a batch of
// calls issues all its loads at once.
__device__ __forceinline__ SeqInfo seq_info(const PlanArgs& a, int64_t i, bool valid) {
  const int j = valid ? int(i) : 0;
  const int32_t r0 = a.qsl[j];
  int32_t q = a.qsl[j + 1] - r0;
  int32_t c = a.ctx[j];
  q = int32_t(min(int64_t(max(q, 0)), int64_t(a.num_tokens) - r0));
  if (!valid || r0 < 0 || r0 >= a.num_tokens) q = 0;
  c = max(c, 0);
  if (int64_t(c) + q > a.max_len) q = c >= a.max_len ? 0 : a.max_len - c;
  const bool group = !a.all_chunk && q > 1 && q <= a.verify_rows;
  return SeqInfo{r0, q, c, !group && q > (a.all_chunk ? 0 : 1) && a.use_mfma, group};
}

__device__ __forceinline__ void seq_counts(const SeqInfo& s, int tile_rows, int64_t hkv, int64_t& ntile,
                                           int64_t& nrow, int64_t& nunit) {
  if (s.chunk) {
    ntile += (s.q + tile_rows - 1) / tile_rows;
  } else if (s.group) {
    nrow += 1;
    nunit += hkv * ((int64_t(s.c) + s.q + kBlock - 1) / kBlock);  // the pages of its last row
  } else if (s.q > 0) {
    nrow += s.q;
    nunit += hkv * (pages_upto(int64_t(s.c) + s.q) - pages_upto(s.c));
  }
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(PlanArgs a, Workspace w) {
  __shared__ int64_t sh[2 * kWavesPerPlan];
  __shared__ int s_hist[kSortBuckets];
  __shared__ int64_t s_base[kLdsRows];   // first unit of each row
  __shared__ int32_t s_pages[kLdsRows];  // pages of each row (per kv head)
  __shared__ int32_t s_tok[kLdsRows];    // first token row of each record
  __shared__ int8_t s_nq[kLdsRows];      // query rows of each record
  const int tid = threadIdx.x;
  const int64_t hkv = a.num_kv_heads;

  // pass 1: thread t owns the contiguous sequences [i0, i1); one scan of the
  // per-thread counts places its tile records, row records and units
  const int64_t m = (int64_t(a.num_seqs) + kPlanThreads - 1) / kPlanThreads;
  const int64_t i0 = min(int64_t(tid) * m, int64_t(a.num_seqs)), i1 = min(i0 + m, int64_t(a.num_seqs));
  int64_t ntile = 0, nrow = 0, nunit = 0;
  int flags = 0;
  for (int64_t ib = i0; ib < i1; ib += kSeqBatch) {
#pragma unroll
    for (int c = 0; c < kSeqBatch; ++c)
      seq_counts(seq_info(a, ib + c, ib + c < i1), a.tile_rows, hkv, ntile, nrow, nunit);
  }
  for (int64_t i = i0; i < i1; ++i)  // metadata the rows above were clamped against (sticky flag)
    flags |= rows_flag(a.qsl[i], a.qsl[i + 1], a.ctx[i], a.num_tokens, a.max_len);
  if (flags) atomicOr(&w.hdr[H_FLAGS], flags);
  int64_t off_tr, off_u, tot_tr, tot_u;
  block_exclusive_scan2((ntile << 32) | nrow, nunit, &off_tr, &off_u, &tot_tr, &tot_u, sh);
  int64_t tiles = tot_tr >> 32, rows = tot_tr & 0xFFFFFFFFll;
  const int64_t units = tot_u;
  {
    int64_t t = off_tr >> 32, r = off_tr & 0xFFFFFFFFll, u = off_u;
    for (int64_t ib = i0; ib < i1; ib += kSeqBatch) {
#pragma unroll
      for (int c = 0; c < kSeqBatch; ++c) {
        const SeqInfo s = seq_info(a, ib + c, ib + c < i1);
        if (s.chunk) {
          // tile records with their key count (bucketed in kSortBucketKeys) for the sort below
          for (int32_t first = 0; first < s.q && t < w.tiles_cap; first += a.tile_rows, ++t) {
            const int32_t nt = min(a.tile_rows, s.q - first);
            const int64_t bucket = (int64_t(s.c) + first + nt) / kSortBucketKeys;
            w.tiles_tmp[t] = make_int4(int(ib + c), first, int32_t(bucket < kSortBuckets ? bucket : kSortBuckets - 1), 0);
          }
        } else {
          // one record per row, or one for all rows of a short query
          const int32_t nrec = s.group ? 1 : s.q, nq = s.group ? s.q : 1;
          for (int32_t j = 0; j < nrec && r < w.rows_cap; ++j, ++r) {
            const int32_t len = s.c + j + nq;  // keys seen by the record's last row
            const int32_t pages = (len + kBlock - 1) / kBlock;
            w.rows[r] = make_int4(s.r0 + j, int(ib + c), len, nq);
            w.rows_base[r] = u;
            if (r < kLdsRows) {
              s_base[r] = u;
              s_pages[r] = pages;
              s_tok[r] = s.r0 + j;
              s_nq[r] = int8_t(nq);
            }
            u += hkv * pages;
          }
        }
      }
    }
  }
  if (tiles > w.tiles_cap) tiles = w.tiles_cap;  // only with inconsistent metadata
  if (rows > w.rows_cap) rows = w.rows_cap;
  __syncthreads();  // tile and row records written above are read by other threads below

  // chunk tiles longest first (counting sort on key count, descending), so
  // the tiles that see the most keys start first and the tail stays short;
  // the order inside a bucket does not matter
  if (tiles > 0) {
    int* hist = s_hist;
    hist[tid] = 0;  // one bucket per thread
    __syncthreads();
    for (int64_t t = tid; t < tiles; t += kPlanThreads)
      atomicAdd(&hist[kSortBuckets - 1 - w.tiles_tmp[t].z], 1);
    __syncthreads();
    int64_t off, dummy, tot, tot2;
    block_exclusive_scan2(hist[tid], 0, &off, &dummy, &tot, &tot2, sh);
    hist[tid] = int(off);
    __syncthreads();
    for (int64_t t = tid; t < tiles; t += kPlanThreads) {
      const int4 rec = w.tiles_tmp[t];
      const int at = atomicAdd(&hist[kSortBuckets - 1 - rec.z], 1);
      w.tiles[at] = make_int2(rec.x, rec.y);
    }
  }

  // the unit stream is cut into ranges of `per` units
  int64_t per = a.fixed_units > 0 ? a.fixed_units : (units + a.num_ranges - 1) / a.num_ranges;
  if (per < 1) per = 1;
  int64_t nranges = (units + per - 1) / per;
  if (nranges > w.ranges_cap) {  // a fixed range length too short for the workspace
    per = (units + w.ranges_cap - 1) / w.ranges_cap;
    nranges = (units + per - 1) / per;
  }

  // pass 2: every range start names the row holding it and, if it is the
  // first boundary strictly inside a (row, kv head) pair, the pair's merge
  // record.  A start `off` units into its pair is that boundary iff
  // 0 < off <= per.
  if (rows <= kLdsRows) {
    // one thread per range: binary search of the rows' first units in LDS
    for (int64_t g = tid; g < nranges; g += kPlanThreads) {
      const int64_t start = g * per;
      int lo = 0, hi = int(rows);  // s_base[lo] <= start < s_base[hi] (hi == rows: end of stream)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_base[mid] <= start) lo = mid;
        else hi = mid;
      }
      const uint32_t rel = uint32_t(start - s_base[lo]), pages = uint32_t(s_pages[lo]);
      const uint32_t k = rel / pages, off = rel - k * pages;
      w.range_row[g] = lo;
      w.range_cut[g] = off > 0 && off <= per
                           ? cut_record(start - off, pages, per, s_tok[lo], int(k), s_nq[lo])
                           : make_int4(-1, -1, -1, -1);
    }
  } else {
    // one thread per row: the range starts inside each of its pairs
    const double inv_per = 1.0 / double(per);
    for (int64_t r = tid; r < rows; r += kPlanThreads) {
      const int4 rec = w.rows[r];
      const int64_t pages = (rec.z + kBlock - 1) / kBlock;
      for (int k = 0; k < hkv; ++k) {
        const int64_t start = w.rows_base[r] + k * pages;
        int64_t g = int64_t(double(start) * inv_per);  // first range starting at or after start
        while (g * per < start) ++g;
        while (g > 0 && (g - 1) * per >= start) --g;
        for (; g * per < start + pages && g < nranges; ++g) {
          const int64_t off = g * per - start;
          w.range_row[g] = int32_t(r);
          w.range_cut[g] = off > 0 && off <= per ? cut_record(start, pages, per, rec.x, k, rec.w)
                                                 : make_int4(-1, -1, -1, -1);
        }
      }
    }
  }

  if (tid == 0) {
    w.hdr[H_ROWS] = int32_t(rows);
    w.hdr[H_TILES] = int32_t(tiles);
    w.hdr[H_RANGES] = int32_t(nranges);
    for (int x = 0; x < kXcdQueues; ++x) w.hdr[H_QUEUE + x] = 0;
    w.hdr64[H64_UNITS] = units;
    w.hdr64[H64_PER] = per;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, const Workspace& w, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a, w);
  return hipGetLastError();
}

}  // namespace pa
