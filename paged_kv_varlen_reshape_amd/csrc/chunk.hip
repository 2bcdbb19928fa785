// chunk_mfma: causal attention of multi-row (prefill chunk) sequences on bf16 MFMA.
//
// Prefill processes every prompt token of a request at once and is bound by
// compute (Inside vLLM summary, techfeed.io, section "エンジンの中核：スケジューラ
// とKVキャッシュ管理"); long prompts arrive as chunks on top of tokens already
// cached (section "高度な機能群", chunked prefill), and each chunk row attends
// only to its own sequence's keys up to its own position (section
// "PagedAttentionの仕組み": flattened super-sequence with positions and mask).
// Row j of a chunk with c cached tokens sits at position p = c + j and sees
// keys 0..p, read through the block table.
//
// Tile: 128 query rows = (128/G tokens) x (the G query heads of one kv head),
// so one K/V tile in LDS serves the whole GQA group.  Wavefront w owns rows
// 32w..32w+31 (row rho = head_in_group * TQ + token).  Keys come in tiles of 64
// (four 16-token pages).  Both products run transposed on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   S^T[key][row] = sum_d K[key][d] Q[row][d]        (A = K from LDS, B = Q in registers)
//   O^T[d][row]  += sum_key V^T[d][key] P^T[key][row] (A = V^T from LDS, B = P in registers)
// In the 32x32 accumulator layout lane l holds column l%32 (one query row) and
// 16 rows (keys), so a query row's max and sum need only one exchange between
// lanes l and l^32, and the bf16 weights P feed the PV product straight from
// the S^T accumulator: the PV operand slots are matched to the keys the lane
// holds, and V^T is read in the same key order.
//
// Staging is DMA: wavefront w copies page w of the tile (16 rows of K and of
// V) from the pool into LDS with buffer_load_dwordx4 ... lds (one wave-uniform
// block id, each instruction fills 1 KiB of LDS in lane order), so K and V
// never pass through registers.  K is read back as the MFMA A operand with
// ds_read_b128; V stays row-major and ds_read_b64_tr_b16 returns it
// transposed: within 16 lanes, lane i receives the (i%4)-th element of the 8
// bytes addressed by lane 4k + i/4 for k = 0..3, so if lane s addresses
// V[key0 + s/4][d0 + 4*(s%4)], lane i gets V[key0 + 0..3][d0 + i], a V^T
// operand quarter.  Both tiles are XOR-swizzled by 16-byte chunk (K by the row
// within its page, V by a table over row % 4) so the operand loads touch
// distinct banks; the DMA chooses, per lane, the global chunk that belongs in
// its LDS slot.  LDS holds two tiles: the DMA of tile kt+1 is issued before
// tile kt is multiplied, and one barrier per tile closes both.
//
// Online softmax in the log2 domain on the VALU; P is rounded to bf16 for the
// PV product and the row sum l adds the rounded values, so the output is an
// exact convex combination of V rows with the rounded weights.  Row maxima are
// taken on raw scores and then multiplied by the scale, which is therefore
// kept positive: the host folds a negative scale's sign into Q (a bf16 sign
// flip, exact) and turns a zero scale into a zeroed Q, so masked keys (-inf)
// always end as weight 0 and never meet a factor of 0.  The reference
// maximum moves lazily (the O accumulators are rescaled only when a row's
// maximum grows by more than 2^8).  Keys past a row's position get -inf by
// select; V rows of keys past the tile's last position are zeroed in LDS after
// the DMA (pages past the sequence are not read at all), so nothing outside
// the sequence reaches the PV product (NaN-safe).  Tiles are taken from work
// counters, longest first: one queue per XCD when the kv heads split evenly
// over the XCDs (the tiles of one sequence and kv head then share an L2).
#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;

constexpr int kTileRows = 128;  // query rows per workgroup tile
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 256;
constexpr int kHandoverTiles = 4;  // the next item is claimed this many key tiles before the end

typedef const __attribute__((address_space(4))) int32_t const_i32;  // read with scalar loads
constexpr int KLOOK = 3;  // k-steps of K operand reads in flight ahead of the Q.K products
constexpr int VLOOK = 4;  // V^T operand reads in flight ahead of the P.V products

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lanes l and l ^ 32 (v_permlane32_swap of x with itself: a VALU exchange of
// the two lane halves; in every lane one result holds x of lane l, the other
// x of lane l ^ 32)
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, uint32_t(sw[0]));
  b = __builtin_bit_cast(float, uint32_t(sw[1]));
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  lane_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  lane_pair(x, a, b);
  return a + b;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Raw buffer descriptor over one page (bytes [0, bytes) from base; word 3 =
// 32-bit data format, the gfx9-family value for untyped byte-offset access).
// The tile copies go through MUBUF loads into LDS rather than the FLAT-encoded
// global form: a FLAT load that may write LDS makes the compiler wait for
// every LDS read with lgkmcnt(0), so no operand read could stay in flight
// past the one a product needs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}

// two floats -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

constexpr bf16x2_t kOnes = {__bf16(1.0f), __bf16(1.0f)};

// XOR swizzle of V's 16-byte chunks by row % 4 (a table found to make the
// transposed operand loads touch distinct banks in 16- and 32-lane groups)
__device__ __forceinline__ int v_swz(int row) { return (0xEA40 >> ((row & 3) * 4)) & 15; }  // {0, 4, 10, 14}

template <int D>
struct ChunkCfg {
  static constexpr int RB = D * 2;                  // bytes per K/V row
  static constexpr int CH = RB / 16;                // 16-byte chunks per row: 16 or 8
  static constexpr int RPI = kWave / CH;            // rows per DMA instruction: 4 or 8
  static constexpr int IPG = kBlock / RPI;          // DMA instructions per page and tensor
  static constexpr int KSTEPS = D / 16;             // MFMA k-steps of Q.K (16 dims each)
  static constexpr int DBLK = D / 32;               // 32-dim blocks of O^T
  static constexpr int TILE_BYTES = kBN * RB;       // one K or V tile
};

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2)
chunk_mfma_kernel(AttnArgs a, Workspace w) {
  using C = ChunkCfg<D>;
  constexpr int RB = C::RB, CH = C::CH, RPI = C::RPI, IPG = C::IPG, KSTEPS = C::KSTEPS, DBLK = C::DBLK;
  constexpr int TQ = kTileRows / G;  // tokens per tile

  // two buffers of each: tile kt+1 lands while tile kt is multiplied.  Four
  // separate arrays, each step naming its buffers at compile time, so the
  // compiler can see that the DMA in flight does not write what is being read
  // (it would otherwise wait for the DMA before every LDS read)
  __shared__ __attribute__((aligned(16))) char s_k0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_k1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_v0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_v1[C::TILE_BYTES];
  __shared__ int s_item;
  __shared__ int s_tbase[kSelfPlanRows + 1];  // self-planned steps: first tile of each sequence,
  __shared__ int s_qsl[kSelfPlanRows + 1];    //   its query_start_loc entries
  __shared__ int s_ctx[kSelfPlanRows];        //   and its context_lens entry,
  __shared__ int s_q[kSelfPlanRows];          //   its chunk rows (clamped; 0 if none)
  __shared__ int s_order[kChunkSortTiles];    //   and, longest first, the tiles in sequence order

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 31;  // accumulator column = query row within the wavefront
  const int lg = lane >> 5;   // lane half

  // K operand (ds_read_b128): row mb*32 + col, chunk (2kk + lg) ^ (col % CH) = 2kk ^ kx
  const int kx = lg ^ (col & (CH - 1));
  // V operand (ds_read_b64_tr_b16): source lane s addresses row 4*lg + s/4 (+ 16t + 8e)
  // and dims 32db + 16*(col/16) + 4*(s%4) (chunk c, half s&1), swizzled by row % 4 = s/4
  int vaddr[DBLK];
  {
    const int s = lane & 15, q = s >> 2, h16 = col >> 4;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int c = 4 * db + 2 * h16 + ((s >> 1) & 1);
      vaddr[db] = (4 * lg + q) * RB + 16 * ((c ^ v_swz(q)) & (CH - 1)) + 8 * (s & 1);
    }
  }
  // DMA: in instruction j of a page, lane -> row j*RPI + lane/CH of the page,
  // LDS chunk lane%CH, which holds global chunk (lane%CH) ^ swizzle(row)
  const int dma_row = lane / CH, dma_chunk = lane % CH;
  // so each copy instruction is a scalar page base plus these per-lane byte
  // offsets (fixed size: an array sized by a template parameter and captured
  // by the lambdas below is not instantiated in the host pass)
  static_assert(IPG <= 4, "copy instructions per page");
  uint32_t off_k[4], off_v[4];
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int row = j * RPI + dma_row;  // token within the page
    off_k[j] = uint32_t(row * RB + 16 * (dma_chunk ^ (row & (CH - 1))));
    off_v[j] = uint32_t(row * RB + 16 * (dma_chunk ^ (v_swz(row) & (CH - 1))));
  }

  // A small step may be planned here instead of by the plan kernel: every
  // workgroup counts the tiles of each sequence (the same routing and clamping
  // as the plan) and keeps their prefix sum in LDS.  With chunk_self_plan = 2
  // it also ranks the tiles longest first (below); every workgroup then takes
  // its queue positions in fixed rounds, so nothing depends on counters or a
  // list in the workspace.
  int n_items;
  bool sorted = false;
  if (a.chunk_self_plan) {
    constexpr int SPT = kSelfPlanRows / kThreads;  // sequences per thread
    int cnt[SPT], tot = 0;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid * SPT + k;
      int q = 0;
      if (i < a.num_seqs) {
        const int r0 = a.qsl[i], r1 = a.qsl[i + 1], cr = a.ctx[i];
        s_qsl[i] = r0;  // kept for the items' metadata (meta_stage2)
        s_ctx[i] = cr;
        if (i == a.num_seqs - 1) s_qsl[i + 1] = r1;
        q = int(min(int64_t(max(r1 - r0, 0)), int64_t(a.num_tokens) - r0));
        if (r0 < 0 || r0 >= a.num_tokens) q = 0;
        const int c = max(cr, 0);
        if (int64_t(c) + q > a.max_len) q = c >= a.max_len ? 0 : a.max_len - c;
        if (blockIdx.x == 0) {  // metadata clamped above: sticky flag (once, not per workgroup)
          const int f = rows_flag(r0, r1, cr, a.num_tokens, a.max_len);
          if (f) atomicOr(&w.hdr[H_FLAGS], f);
        }
      }
      cnt[k] = q > (a.all_chunk ? 0 : 1) ? (q + TQ - 1) / TQ : 0;  // a chunk sequence's tiles
      if (i < a.num_seqs) s_q[i] = cnt[k] > 0 ? q : 0;
      tot += cnt[k];
    }
    // exclusive scan of the per-thread tile counts over the workgroup
    int incl = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int x = __shfl_up(incl, d);
      if (lane >= d) incl += x;
    }
    if (lane == kWave - 1) s_tbase[kSelfPlanRows - kThreads / kWave + wave] = incl;  // wave totals, scratch
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int ww = 0; ww < kThreads / kWave; ++ww) {
      const int t = s_tbase[kSelfPlanRows - kThreads / kWave + ww];
      base += ww < wave ? t : 0;
      total += t;
    }
    __syncthreads();  // the wave totals are read before the table overwrites them
    int run = base + incl - tot;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      s_tbase[tid * SPT + k] = run;
      run += cnt[k];
    }
    if (tid == 0) s_tbase[kSelfPlanRows] = total;
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(total);
    n_items = total * a.hkv;

    // Longest first, without a sort: a tile's rank is the number of tiles that
    // see more keys (its last row's), or as many with a lower index.  Within a
    // sequence (c cached tokens, q chunk rows) tile t sees c + min(q, TQ(t+1))
    // keys, strictly increasing in t, so each other sequence's count is a
    // closed form.  Every workgroup computes the same ranks.
    // (only when the items take more than one round of the grid: in one round
    // every workgroup takes one item and the order changes nothing)
    sorted = a.chunk_self_plan == 2 && total <= kChunkSortTiles && a.num_seqs <= kChunkSortSeqs &&
             n_items > int(gridDim.x);
    if (sorted) {
      for (int i = tid; i < total; i += kThreads) {
        int lo = 0, hi = a.num_seqs;  // the last sequence whose first tile is at or before i
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_tbase[mid] <= i) lo = mid;
          else hi = mid;
        }
        const int keys = max(s_ctx[lo], 0) + min(s_q[lo], TQ * (i - s_tbase[lo] + 1));
        int rank = 0;
        for (int s2 = 0; s2 < a.num_seqs; ++s2) {
          const int first = s_tbase[s2], n2 = s_tbase[s2 + 1] - first;
          if (n2 == 0) continue;
          const int f = keys - max(s_ctx[s2], 0), q2 = s_q[s2];
          if (f < 0) {  // every tile of s2 sees more keys
            rank += n2;
            continue;
          }
          // full tiles t2 < n2 - 1 see c2 + TQ(t2+1) keys, the last c2 + q2
          rank += max(0, n2 - 1 - f / TQ) + (q2 > f ? 1 : 0);
          // an equal tile with a lower index
          const int t_eq = (f % TQ == 0 && f / TQ - 1 < n2 - 1) ? f / TQ - 1 : (q2 == f ? n2 - 1 : -1);
          if (t_eq >= 0 && first + t_eq < i) ++rank;
        }
        s_order[rank] = i;
      }
      __syncthreads();
    }
  } else {
    n_items = w.hdr[H_TILES] * a.hkv;
  }
  // Items are (tile, kv head) pairs, item = tile * hkv + kv head, tiles longest
  // first.  Tiles of one sequence and kv head re-read the same K/V prefix, so
  // when the kv heads split evenly over the XCDs each XCD gets a queue of its
  // own: queue x holds kv heads x, x + 8, ... of every tile, in tile order, and
  // is served by the workgroups b with b % 8 == x, which run on XCD x and share
  // its L2.  Every queue has gridDim.x / 8 workgroups, so every item is taken.
  const bool xcd_queues = a.hkv % kXcdQueues == 0 && gridDim.x % kXcdQueues == 0;
  const int xq = xcd_queues ? int(blockIdx.x % kXcdQueues) : 0;    // this workgroup's queue
  const int q_wgs = xcd_queues ? int(gridDim.x / kXcdQueues) : int(gridDim.x);
  const int q_len = xcd_queues ? n_items / kXcdQueues : n_items;
  const int h_per_q = a.hkv / kXcdQueues;
  // the j-th item of this workgroup's queue (n_items: the queue is empty)
  auto queue_item = [&](int j) __attribute__((always_inline)) -> int {
    if (j >= q_len) return n_items;
    if (!xcd_queues) return j;
    const int tl = j / h_per_q;
    return tl * a.hkv + xq + kXcdQueues * (j - tl * h_per_q);
  };
  const int64_t page_stride = int64_t(kBlock) * RB;
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  // Work queue: the workgroup's first item is its queue's (blockIdx.x / 8)-th
  // (blockIdx.x-th with a single queue), later ones come from the queue's
  // counter (longest items first).  The next item is claimed a few key
  // tiles before the current one ends (late enough to keep the queue's
  // longest-first balance) and everything it needs before its first DMA is
  // fetched at the following tile boundaries, one dependent scalar load per
  // boundary, so an item starts with one memory latency instead of a chain.
  const_i32* cqsl = (const_i32*)a.qsl;
  const_i32* cctx = (const_i32*)a.ctx;
  const_i32* ctiles = (const_i32*)w.tiles;  // int2 records {seq, first row}
  const_i32* cbt = (const_i32*)a.bt;
  struct Meta {
    int seq, t0, r0, qend, ctx, blk0;  // blk0: block id of this wavefront's page of tile 0
  };
  // the item's tile record (stage 1), its sequence's rows (stage 2), its first block id (stage 3)
  auto meta_stage1 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    if (it >= n_items) return;
    const int tl = __builtin_amdgcn_readfirstlane(it / a.hkv);
    if (a.chunk_self_plan) {
      const int ti = sorted ? __builtin_amdgcn_readfirstlane(s_order[tl]) : tl;  // tile in sequence order
      // the last sequence whose first tile is at or before it (sequences
      // without tiles share their successor's first tile and are passed over)
      int lo = 0, hi = a.num_seqs;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tbase[mid] <= ti) lo = mid;
        else hi = mid;
      }
      mt.seq = __builtin_amdgcn_readfirstlane(lo);
      mt.t0 = __builtin_amdgcn_readfirstlane((ti - s_tbase[lo]) * TQ);
    } else {
      mt.seq = ctiles[2 * tl];
      mt.t0 = ctiles[2 * tl + 1];
    }
  };
  auto meta_stage2 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    if (it >= n_items) return;
    if (a.chunk_self_plan) {  // kept in LDS by the self-plan
      mt.r0 = __builtin_amdgcn_readfirstlane(s_qsl[mt.seq]);
      mt.qend = __builtin_amdgcn_readfirstlane(s_qsl[mt.seq + 1]);
      mt.ctx = __builtin_amdgcn_readfirstlane(s_ctx[mt.seq]);
    } else {
      mt.r0 = cqsl[mt.seq];
      mt.qend = cqsl[mt.seq + 1];
      mt.ctx = cctx[mt.seq];
    }
  };
  // the plan clamped the rows it tiled the same way: nothing may index
  // outside q, out or the block-table row even with inconsistent metadata
  auto tile_len = [&](const Meta& mt) __attribute__((always_inline)) -> int {
    const int cx = max(mt.ctx, 0);
    const int qlen = min(min(mt.qend - mt.r0, a.num_tokens - mt.r0), a.mbps * kBlock - cx);
    return max(0, min(TQ, qlen - mt.t0));
  };
  auto meta_stage3 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    mt.blk0 = 0;
    if (it >= n_items) return;
    const int kv_end_n = max(mt.ctx, 0) + mt.t0 + tile_len(mt);
    if (wave * kBlock < kv_end_n) mt.blk0 = cbt[int64_t(mt.seq) * a.mbps + wave];
  };

  bool blk_bad = false;  // a block id outside the pool was clamped (reported at the end)
  // Self-planned steps take queue positions in rounds: round r covers
  // positions r * q_wgs .. (r + 1) * q_wgs - 1, one per workgroup of the queue,
  // in workgroup order on even rounds and, with longest-first tiles, in
  // reverse order on odd rounds (so the workgroup with the longest first item
  // gets the shortest second one).
  const int qu = int(blockIdx.x) / (xcd_queues ? kXcdQueues : 1);  // this workgroup's index in its queue
  int rnd = 0;
  auto round_pos = [&](int r) __attribute__((always_inline)) -> int {
    return r * q_wgs + ((sorted && (r & 1)) ? q_wgs - 1 - qu : qu);
  };
  int item = queue_item(round_pos(0));
  Meta cur{};
  meta_stage1(item, cur);
  meta_stage2(item, cur);
  meta_stage3(item, cur);
  while (item < n_items) {
    // the hand-over to the next item: phase 0 claims it (thread 0), phase 1
    // publishes its number in LDS, phases 2 and 3 load its tile record and
    // sequence rows; each phase runs at the start of one key tile, after the
    // barrier that ended the tile before (which also waited for the phase
    // before it), and what is left runs when the item ends
    int claimed = 0, next = n_items, phase = 0;
    Meta nxt{};
    auto handover = [&]() __attribute__((always_inline)) {
      if (phase == 0) {
        // self-planned: the next position in this workgroup's fixed stride
        if (tid == 0)
          claimed = queue_item(a.chunk_self_plan ? round_pos(rnd + 1) : q_wgs + atomicAdd(&w.hdr[H_QUEUE + xq], 1));
      } else if (phase == 1) {
        if (tid == 0) s_item = claimed;
      } else if (phase == 2) {
        next = __builtin_amdgcn_readfirstlane(s_item);
        meta_stage1(next, nxt);
      } else if (phase == 3) {
        meta_stage2(next, nxt);
      }
      ++phase;
    };

    const int kvh = item - (item / a.hkv) * a.hkv;
    const int seq = cur.seq, t0 = cur.t0;
    const int r0 = cur.r0;
    const int ctx = max(cur.ctx, 0);
    const int nt = tile_len(cur);  // valid tokens of this tile
    const int kv_end = ctx + t0 + nt;           // keys seen by the tile's last row
    const int n_kt = (kv_end + kBN - 1) / kBN;
    const int n_pages = (kv_end + kBlock - 1) / kBlock;
    const int32_t* btrow = a.bt + int64_t(seq) * a.mbps;

    // this lane's query row
    const int rho = wave * 32 + col;
    const int hh = rho / TQ, tt = rho - hh * TQ;
    const bool valid = tt < nt;
    const int pos = ctx + t0 + tt;  // keys 0..pos are visible
    const int head = kvh * G + hh;

    u32x4 qf[KSTEPS];
    {
      const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) +
                                                       ((int64_t(r0) + t0 + tt) * a.hq + head) * RB);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = valid ? qp[2 * kk + lg] : u32x4{0u, 0u, 0u, 0u};
      // a negative or zero scale: its sign (or the zero) goes into Q, so the
      // factor the scores are multiplied by below is always positive
      if (a.q_and != ~0u || a.q_xor != 0u) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = (qf[kk] & a.q_and) ^ a.q_xor;
      }
    }

    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    // block id of this wavefront's page in tile kt (raw: made wave-uniform and
    // clamped where it is used, a tile later, so its load is not waited for here
    // -- vector loads retire in order, so that wait would also wait for the DMA)
    auto page_id = [&](int kt) __attribute__((always_inline)) -> int32_t {
      const int page = kt * 4 + wave;
      return page < n_pages ? btrow[page] : 0;
    };
    // DMA of this wavefront's page of tile kt into buffer buf (nothing past the sequence)
    auto dma_tile = [&](int kt, auto bufc, int32_t raw) __attribute__((always_inline)) {
      constexpr int buf = decltype(bufc)::value;
      char* dk = buf ? s_k1 : s_k0;
      char* dv = buf ? s_v1 : s_v0;
      if (kt * 4 + wave >= n_pages) return;
      raw = __builtin_amdgcn_readfirstlane(raw);
      const int32_t blk = raw < 0 ? 0 : (raw >= a.nb ? int32_t(a.nb - 1) : raw);  // never leave the pool
      blk_bad |= blk != raw;
      const int64_t page = (int64_t(blk) * a.hkv + kvh) * page_stride;
      // one buffer descriptor per page: the per-lane offsets stay 32-bit and
      // a copy can never read past the page
      const __amdgpu_buffer_rsrc_t rk = page_rsrc(kbase + page, int(page_stride));
      const __amdgpu_buffer_rsrc_t rv = page_rsrc(vbase + page, int(page_stride));
#pragma unroll
      for (int j = 0; j < IPG; ++j) {
        const int lrow = wave * kBlock + j * RPI;  // first LDS row of this instruction
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(dk + lrow * RB), 16, off_k[j], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(dv + lrow * RB), 16, off_v[j], 0, 0, 0);
      }
    };
    // after the DMA has landed: V rows of keys at or past kv_end become zeros
    auto zero_tail = [&](int kt, auto bufc) __attribute__((always_inline)) {
      char* dv = decltype(bufc)::value ? s_v1 : s_v0;
      const int key0 = kt * kBN + wave * kBlock;  // first key of this wavefront's page
      if (key0 + kBlock <= kv_end) return;
      for (int idx = lane; idx < kBlock * CH; idx += kWave) {
        const int row = idx / CH;
        if (key0 + row >= kv_end)
          *reinterpret_cast<u32x4*>(dv + (wave * kBlock + row) * RB + (idx % CH) * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    };

    // prologue: tile 0 in buffer 0 (its block id came with the item)
    dma_tile(0, I0{}, cur.blk0);
    int32_t id_next = n_kt > 1 ? page_id(1) : 0;
    __builtin_amdgcn_s_waitcnt(0);
    zero_tail(0, I0{});
    __syncthreads();
    const int handover_from = n_kt - kHandoverTiles;  // key tile of phase 0

    // tiles below n_full are visible to every row of the tile: no mask
    const int n_full = (ctx + t0 + 1) / kBN;
    auto tile_step = [&](int kt, auto bufc, auto masked) __attribute__((always_inline)) {
      constexpr int buf = decltype(bufc)::value;
      using Other = std::integral_constant<int, buf ^ 1>;
      if (kt >= handover_from) handover();
      // the next tile's DMA flies while this one is multiplied
      if (kt + 1 < n_kt) {
        dma_tile(kt + 1, Other{}, id_next);
        if (kt + 2 < n_kt) id_next = page_id(kt + 2);
      }
      const char* ks = buf ? s_k1 : s_k0;
      const char* vs = buf ? s_v1 : s_v0;
      const int key0 = kt * kBN;

      // S^T = K Q^T: two 32-key blocks, the chains interleaved.  The K operand
      // reads run KLOOK k-steps ahead of the products; sched_barrier pins that
      // order, so each product waits only for its own reads (counted waits)
      // instead of for every read in flight.  The products run at raised wave
      // priority, so the matrix core is fed before the other wavefront's
      // softmax when both are ready to issue
      __builtin_amdgcn_s_setprio(1);
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
      {
        const char* kr = ks + col * RB;
        u32x4 ka[KSTEPS], kb[KSTEPS];
        auto kread = [&](int kk) __attribute__((always_inline)) {
          const int off = 16 * ((2 * kk) ^ kx);
          ka[kk] = *reinterpret_cast<const u32x4*>(kr + off);
          kb[kk] = *reinterpret_cast<const u32x4*>(kr + 32 * RB + off);
        };
#pragma unroll
        for (int kk = 0; kk < KLOOK; ++kk) kread(kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kk]), as_bf16x8(qf[kk]), s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[kk]), as_bf16x8(qf[kk]), s[1], 0, 0, 0);
          if (kk + KLOOK < KSTEPS) kread(kk + KLOOK);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // O^T += V^T P^T runs as NPV products, i = t*DBLK + db: 16-key step t
      // uses accumulator rows j = (t%2)*8 .. +8 of block t/2, i.e. keys
      // 16t + (i/4)*8 + lg*4 + i%4, loaded as two transposed quarters (i = 0..3:
      // rows 16t + 4lg + k, i = 4..7: rows 16t + 8 + 4lg + k).  The V^T operands
      // do not depend on P: the first VLOOK are read now, so their LDS latency
      // hides behind the softmax, and the rest run VLOOK products ahead
      constexpr int NPV = 4 * DBLK;
      u32x4 va[NPV];
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int t = i / DBLK, db = i % DBLK;
        const char* vr = vs + vaddr[db] + 16 * t * RB;
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr + 8 * RB));
        va[i] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))};
      };
#pragma unroll
      for (int i = 0; i < VLOOK; ++i) vread(i);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);

      // causal mask (also hides keys past the tile's end): key > pos -> -inf;
      // accumulator row j of block mb is key key0 + lg*4 + mb*32 + (j/4)*8 + j%4
      if constexpr (decltype(masked)::value) {
        const int lim = pos - key0 - lg * 4;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (mb * 32 + (j / 4) * 8 + (j % 4) > lim) s[mb][j] = -INFINITY;
      }
      // online softmax for this lane's row in the log2 domain.  The reference
      // maximum m only moves when a row's maximum exceeds it by more than 2^8
      // (lazy rescale): weights stay <= 2^8, exact in fp32 and bf16 range, and
      // the final division by l cancels the common factor.  The two lane halves
      // hold disjoint keys of the same row: they exchange maxima by a VALU lane
      // swap, which does not queue behind the V^T reads in flight
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(fmaxf(mx, s[0][j]), s[1][j]);
      mx = pair_max(mx) * a.chunk_scale_log2;
      // wave-uniform branch (rarely taken after the first tiles); lanes whose
      // maximum did not grow scale by 1
      const bool grow = mx > m + 8.f;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m - mx) : 1.f;  // 0 on the first tile (m = -inf)
        m = grow ? mx : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      }
      const float m_use = m == -INFINITY ? 0.f : m;

      // P^T in bf16 pairs: pk[mb][i] holds accumulator rows 2i, 2i+1 of block mb;
      // the row sum adds the rounded weights (dot with (1, 1))
      uint32_t pk[2][8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(fmaf(s[mb][2 * i], a.chunk_scale_log2, -m_use));
          const float p1 = fast_exp2(fmaf(s[mb][2 * i + 1], a.chunk_scale_log2, -m_use));
          pk[mb][i] = pack_bf16(p0, p1);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[mb][i]), kOnes, l, false);
        }
      __builtin_amdgcn_sched_barrier(0);

      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int t = i / DBLK, db = i % DBLK;
        const u32x4 pb = {pk[t / 2][(t % 2) * 4 + 0], pk[t / 2][(t % 2) * 4 + 1], pk[t / 2][(t % 2) * 4 + 2],
                          pk[t / 2][(t % 2) * 4 + 3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[i]), as_bf16x8(pb), o[db], 0, 0, 0);
        if (i + VLOOK < NPV) vread(i + VLOOK);
        __builtin_amdgcn_sched_barrier(0);
      }

      __builtin_amdgcn_s_setprio(0);
      // tile kt+1 has landed (and its tail is zeroed) before anyone reads it;
      // everyone is done with buffer buf before the DMA of tile kt+2 reuses it
      if (kt + 1 < n_kt) {
        __builtin_amdgcn_s_waitcnt(0);
        zero_tail(kt + 1, Other{});
      }
      __syncthreads();
    };
    // tile kt sits in buffer kt & 1: two tiles per iteration keep the buffer
    // choice static, so the accumulators flow through one path (no copies)
    auto run = [&](int kt, int kt_end, auto masked) __attribute__((always_inline)) {
      if ((kt & 1) && kt < kt_end) tile_step(kt++, I1{}, masked);
      for (; kt + 1 < kt_end; kt += 2) {
        tile_step(kt, I0{}, masked);
        tile_step(kt + 1, I1{}, masked);
      }
      if (kt < kt_end) tile_step(kt, I0{}, masked);
    };
    run(0, min(n_full, n_kt), std::false_type{});
    run(max(n_full, 0), n_kt, std::true_type{});

    // the two lane halves hold disjoint keys of the same row
    l = pair_sum(l);
    if (valid) {
      const float inv = 1.f / l;
      float* op = a.out + ((int64_t(r0) + t0 + tt) * a.hq + head) * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const float4 v = make_float4(o[db][jb * 4 + 0] * inv, o[db][jb * 4 + 1] * inv, o[db][jb * 4 + 2] * inv,
                                       o[db][jb * 4 + 3] * inv);
          *reinterpret_cast<float4*>(op + db * 32 + jb * 8 + lg * 4) = v;
        }
    }

    // phases a short item had no tiles for, each after a barrier
    while (phase < 4) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      handover();
    }
    __builtin_amdgcn_s_waitcnt(0);
    meta_stage3(next, nxt);
    // every wavefront is done with the LDS tiles and has read s_item
    __syncthreads();
    item = next;
    cur = nxt;
    ++rnd;
  }
  if (blk_bad && lane == 0) atomicOr(&w.hdr[H_FLAGS], PA_FLAG_BLOCK_ID);
}

template <int D, int G>
hipError_t launch_chunk_t(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chunk_mfma_kernel<D, G>, kThreads, 0) != hipSuccess || n <= 0)
      n = 1;
    per_cu = n;
  }
  int64_t grid = int64_t(device_cus()) * per_cu;
  const int64_t cap = w.tiles_cap * a.hkv;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((chunk_mfma_kernel<D, G>), dim3(unsigned(grid)), dim3(kThreads), 0, st, a, w);
  return hipGetLastError();
}

template <int D>
hipError_t launch_chunk_d(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_chunk_t<D, 1>(a, w, st);
    case 2: return launch_chunk_t<D, 2>(a, w, st);
    case 4: return launch_chunk_t<D, 4>(a, w, st);
    case 8: return launch_chunk_t<D, 8>(a, w, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool chunk_supported(int head_dim, int group, int bf16) {
  return bf16 && (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

int chunk_tile_rows(int group) { return kTileRows / group; }

hipError_t launch_chunk(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  return a.d == 64 ? launch_chunk_d<64>(a, w, group, st) : launch_chunk_d<128>(a, w, group, st);
}

}  // namespace pa
