// chunk_pp: causal attention of multi-row (prefill chunk) sequences on bf16
// MFMA, eight wavefronts per workgroup in two groups that take turns on the
// matrix core and on the VALU.
//
// The computation is the one of chunk_mfma (chunk.hip), which states the
// passages it follows: prefill is bound by compute (Inside vLLM summary,
// techfeed.io, section "エンジンの中核：スケジューラとKVキャッシュ管理"), long
// prompts come as chunks over cached tokens (section "高度な機能群"), and row j
// of a chunk over c cached tokens sees keys 0..c+j of its own sequence through
// the block table (section "PagedAttentionの仕組み").  Same operand layouts, same
// online softmax (log2 domain, lazy rescale past 2^8, P rounded to bf16 and l
// summed from the rounded weights, masked keys set to -inf by select, V rows
// past the tile's last key zeroed in LDS), same scale handling; only the
// schedule differs.
//
// Item: 256 query rows = (256/G tokens) x (the G query heads of one kv head).
// Wavefront w owns rows 32w..32w+31 (row = head_in_group * TQ + token), so for
// G >= 2 both groups (waves 0-3 and 4-7) hold every token of the item, each
// for half of the heads, and see the same keys.  Key tile j (64 keys) is
// processed in one step of two halves separated by workgroup barriers:
//   first half:  group 0 multiplies: O += P_{j-1} V_{j-1} and S_j = K_j Q^T
//                group 1 runs the softmax of S_{j-1} (P_{j-1})
//   second half: group 0 runs the softmax of S_j (P_j)
//                group 1 multiplies: O += P_{j-1} V_{j-1} and S_j = K_j Q^T
// Each SIMD holds one wavefront of each group, so in every half one of them
// feeds the matrix core while the other works on the VALU.  The K and V tiles
// in LDS serve all eight wavefronts; they sit in a ring of three buffers each
// (96 KiB at head dim 128), so copies run two steps ahead: during step j
// (which reads K_j and V_{j-1}) wavefront w copies page w % 4 of K_{j+2}
// (group 0) or of V_{j+1} (group 1) with buffer_load ... lds, and at the end
// of the step waits (a counted vmcnt) only for its copies of the step before,
// zeroes V rows past the item's keys, and the barrier that ends the step
// publishes them.  Block ids come by vector loads one step ahead, so no wait
// for them also waits for the LDS operand reads.  An item of n key tiles takes
// n + 1 steps (the last one only adds P_{n-1} V_{n-1}).
#include <type_traits>

#include "chunk_pp.h"
#include "errors.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef const __attribute__((address_space(4))) int32_t const_i32;  // read with scalar loads

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using Yes = std::true_type;
using No = std::false_type;

constexpr int kBN = 64;             // keys per K/V tile
constexpr int kThreads = 512;       // eight wavefronts
constexpr int kRing = 4;            // K and V buffers each: copies run up to three steps ahead
constexpr int kHandoverSteps = 7;   // the next item is claimed this many steps before the end
constexpr int KLOOK = 2;            // k-steps of K operand reads ahead of the Q.K products
constexpr int VLOOK = 4;            // V^T operand reads ahead of the P.V products

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lanes l and l ^ 32, by a VALU exchange of the two lane halves
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

// raw buffer descriptor over one page (bytes [0, bytes) from base)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}

// two floats -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

constexpr bf16x2_t kOnes = {__bf16(1.0f), __bf16(1.0f)};

// Workgroup barrier for LDS traffic between the wavefronts.  __syncthreads()
// waits for every load in flight, and so does a release fence on LDS alone
// (copies into LDS count as LDS writes), which would wait for the tile copies
// issued for later steps.  Here each wavefront waits for its own LDS reads and
// writes (lgkmcnt 0), the copies a barrier publishes are waited for explicitly
// (vmcnt) by the wavefront that issued them, and the empty asm statements keep
// the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of V's 16-byte chunks by row % 4: {0, 4, 10, 14}
__device__ __forceinline__ int v_swz(int row) { return (0xEA40 >> ((row & 3) * 4)) & 15; }

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 1) chunk_pp_kernel(AttnArgs a, Workspace w) {
  constexpr int RB = D * 2;            // bytes per K/V row
  constexpr int CH = RB / 16;          // 16-byte chunks per row: 16 or 8
  constexpr int RPI = kWave / CH;      // rows per copy instruction: 4 or 8
  constexpr int IPG = kBlock / RPI;    // copy instructions per page
  constexpr int KSTEPS = D / 16;       // MFMA k-steps of Q.K
  constexpr int DBLK = D / 32;         // 32-dim blocks of O^T
  constexpr int NPV = 4 * DBLK;        // P.V products per key tile (= 2 * KSTEPS)
  constexpr int TILE = kBN * RB;
  constexpr int TQ = kPPRows / G;      // tokens per item
  static_assert(NPV == 2 * KSTEPS, "the products pair up");

  // K_j and V_j sit in buffer j % 4; eight arrays named at compile time, so
  // the compiler can tell the copies in flight from the tiles being read
  __shared__ __attribute__((aligned(16))) char s_k0[TILE];
  __shared__ __attribute__((aligned(16))) char s_k1[TILE];
  __shared__ __attribute__((aligned(16))) char s_k2[TILE];
  __shared__ __attribute__((aligned(16))) char s_k3[TILE];
  __shared__ __attribute__((aligned(16))) char s_v0[TILE];
  __shared__ __attribute__((aligned(16))) char s_v1[TILE];
  __shared__ __attribute__((aligned(16))) char s_v2[TILE];
  __shared__ __attribute__((aligned(16))) char s_v3[TILE];
  static_assert(kRing == 4, "buffer names");
  auto kbuf = [&](auto bufc) __attribute__((always_inline)) -> char* {
    constexpr int b = decltype(bufc)::value;
    return b == 0 ? s_k0 : (b == 1 ? s_k1 : (b == 2 ? s_k2 : s_k3));
  };
  auto vbuf = [&](auto bufc) __attribute__((always_inline)) -> char* {
    constexpr int b = decltype(bufc)::value;
    return b == 0 ? s_v0 : (b == 1 ? s_v1 : (b == 2 ? s_v2 : s_v3));
  };
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave >> 2;  // 0: multiplies in the first half of each step, 1: in the second
  // tiles ahead of the step that the copies run: K_{j+3} (group 0), V_{j+2} (group 1)
  const int lead = kRing - 1 - grp;
  const int pg = wave & 3;    // the page of each tile this wavefront copies (K: group 0, V: group 1)
  const int col = lane & 31;  // accumulator column = query row within the wavefront
  const int lg = lane >> 5;   // lane half

  // K operand (ds_read_b128): row mb*32 + col, chunk (2kk + lg) ^ (col % CH)
  const int kx = lg ^ (col & (CH - 1));
  // V operand (ds_read_b64_tr_b16), as in chunk_mfma: source lane s addresses
  // row 4*lg + s/4 and dims 32db + 16*(col/16) + 4*(s%4), swizzled by row % 4
  int vaddr[DBLK];
  {
    const int s = lane & 15, q = s >> 2, h16 = col >> 4;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int c = 4 * db + 2 * h16 + ((s >> 1) & 1);
      vaddr[db] = (4 * lg + q) * RB + 16 * ((c ^ v_swz(q)) & (CH - 1)) + 8 * (s & 1);
    }
  }
  // copies: in instruction j of a page, lane -> row j*RPI + lane/CH of the
  // page, LDS chunk lane%CH, which holds global chunk (lane%CH) ^ swizzle(row)
  const int dma_row = lane / CH, dma_chunk = lane % CH;
  static_assert(IPG <= 4, "copy instructions per page");
  uint32_t off[4];
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int row = j * RPI + dma_row;
    const int swz = grp ? v_swz(row) : row;
    off[j] = uint32_t(row * RB + 16 * (dma_chunk ^ (swz & (CH - 1))));
  }

  // Items are (tile, kv head) pairs, item = tile * hkv + kv head, tiles longest
  // first (the plan's order).  With kv heads that split evenly over the XCDs,
  // queue x holds kv heads x, x + 8, ... of every tile and is served by the
  // workgroups b with b % 8 == x, which run on XCD x and share its L2.
  const int n_items = w.hdr[H_TILES] * a.hkv;
  const bool xcd_queues = a.hkv % kXcdQueues == 0 && gridDim.x % kXcdQueues == 0;
  const int xq = xcd_queues ? int(blockIdx.x % kXcdQueues) : 0;
  const int q_wgs = xcd_queues ? int(gridDim.x / kXcdQueues) : int(gridDim.x);
  const int q_len = xcd_queues ? n_items / kXcdQueues : n_items;
  const int h_per_q = a.hkv / kXcdQueues;
  auto queue_item = [&](int j) __attribute__((always_inline)) -> int {
    if (j >= q_len) return n_items;
    if (!xcd_queues) return j;
    const int tl = j / h_per_q;
    return tl * a.hkv + xq + kXcdQueues * (j - tl * h_per_q);
  };
  const int64_t page_stride = int64_t(kBlock) * RB;
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  const_i32* cqsl = (const_i32*)a.qsl;
  const_i32* cctx = (const_i32*)a.ctx;
  const_i32* ctiles = (const_i32*)w.tiles;  // int2 records {seq, first row}
  const_i32* cbt = (const_i32*)a.bt;
  struct Meta {
    int seq, t0, r0, qend, ctx, blk0, blk1, blk2;  // block ids of page pg of tiles 0, 1, 2
  };
  auto meta_stage1 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    if (it >= n_items) return;
    const int tl = __builtin_amdgcn_readfirstlane(it / a.hkv);
    mt.seq = __builtin_amdgcn_readfirstlane(ctiles[2 * tl]);
    mt.t0 = __builtin_amdgcn_readfirstlane(ctiles[2 * tl + 1]);
  };
  // (the metadata is wave-uniform; readfirstlane keeps every index and value
  // in scalar registers, so these are scalar loads)
  auto meta_stage2 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    if (it >= n_items) return;
    const int sq = __builtin_amdgcn_readfirstlane(mt.seq);
    mt.r0 = __builtin_amdgcn_readfirstlane(cqsl[sq]);
    mt.qend = __builtin_amdgcn_readfirstlane(cqsl[sq + 1]);
    mt.ctx = __builtin_amdgcn_readfirstlane(cctx[sq]);
  };
  // the plan clamped the rows it tiled the same way: nothing may index
  // outside q, out or the block-table row even with inconsistent metadata
  auto tile_len = [&](const Meta& mt) __attribute__((always_inline)) -> int {
    const int cx = max(mt.ctx, 0);
    const int qlen = min(min(mt.qend - mt.r0, a.num_tokens - mt.r0), a.mbps * kBlock - cx);
    return max(0, min(TQ, qlen - mt.t0));
  };
  auto meta_stage3 = [&](int it, Meta& mt) __attribute__((always_inline)) {
    mt.blk0 = mt.blk1 = mt.blk2 = 0;
    if (it >= n_items) return;
    const int kv_end_n = __builtin_amdgcn_readfirstlane(max(mt.ctx, 0) + mt.t0 + tile_len(mt));
    const_i32* row = cbt + int64_t(__builtin_amdgcn_readfirstlane(mt.seq)) * a.mbps;
    if (pg * kBlock < kv_end_n) mt.blk0 = __builtin_amdgcn_readfirstlane(row[pg]);
    if ((4 + pg) * kBlock < kv_end_n) mt.blk1 = __builtin_amdgcn_readfirstlane(row[4 + pg]);
    if ((8 + pg) * kBlock < kv_end_n) mt.blk2 = __builtin_amdgcn_readfirstlane(row[8 + pg]);
  };

  bool blk_bad = false;  // a block id outside the pool was clamped (reported at the end)
  int item = queue_item(int(blockIdx.x) / (xcd_queues ? kXcdQueues : 1));
  Meta cur{};
  meta_stage1(item, cur);
  meta_stage2(item, cur);
  meta_stage3(item, cur);
  while (item < n_items) {
    // Hand-over to the next item, one phase per step: the claim (phase 0) at
    // the start of its step, before the step's block-id load and copy, so the
    // counted wait at the end of the next step retires it; the rest in the
    // group's softmax half (no LDS operand reads there for the scalar loads to
    // hold up): publish in LDS (2), tile record (3), rows (4), first block ids (5).
    int claimed = 0, next = n_items, phase = 0;
    Meta nxt{};
    auto claim = [&]() __attribute__((always_inline)) {
      if (phase == 0 && tid == 0) claimed = atomicAdd(&w.hdr[H_QUEUE + xq], 1);
    };
    // the steps call claim() at their start and handover() later in the same
    // step; phase 0 of handover() only counts the claim made that step
    auto handover = [&]() __attribute__((always_inline)) {
      if (phase == 2) {
        if (tid == 0) s_item = queue_item(q_wgs + claimed);
      } else if (phase == 3) {
        next = __builtin_amdgcn_readfirstlane(s_item);
        meta_stage1(next, nxt);
      } else if (phase == 4) {
        meta_stage2(next, nxt);
      } else if (phase == 5) {
        meta_stage3(next, nxt);
      }
      ++phase;
    };
    constexpr int kPhases = 6;

    // the item's values are wave-uniform (scalar registers)
    item = __builtin_amdgcn_readfirstlane(item);
    const int kvh = __builtin_amdgcn_readfirstlane(item - (item / a.hkv) * a.hkv);
    const int seq = __builtin_amdgcn_readfirstlane(cur.seq), t0 = __builtin_amdgcn_readfirstlane(cur.t0);
    const int r0 = __builtin_amdgcn_readfirstlane(cur.r0);
    const int ctx = max(__builtin_amdgcn_readfirstlane(cur.ctx), 0);
    const int nt = __builtin_amdgcn_readfirstlane(tile_len(cur));  // valid tokens of this item
    const int kv_end = ctx + t0 + nt;           // keys seen by the item's last row
    const int n_kt = __builtin_amdgcn_readfirstlane((kv_end + kBN - 1) / kBN);  // key tiles
    const int n_pages = __builtin_amdgcn_readfirstlane((kv_end + kBlock - 1) / kBlock);
    const int n_full = __builtin_amdgcn_readfirstlane((ctx + t0 + 1) / kBN);  // tiles below: no mask
    const int v_last = (n_kt + kRing - 1) % kRing;  // buffer of V_{n_kt-1}, read by the last step

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
      // factor the raw scores are multiplied by below is always positive
      if (a.q_and != ~0u || a.q_xor != 0u) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = (qf[kk] & a.q_and) ^ a.q_xor;
      }
    }

    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};  // S^T of the tile between its product and its softmax
    uint32_t pk[2][8] = {};                     // P^T in bf16 pairs between the softmax and P.V

    // Block id of page pg of tile kt (a page past the sequence reads the
    // sequence's last page), as a scalar load.  Scalar loads share a counter
    // with the LDS operand reads, so they are only issued in a softmax half,
    // which reads no LDS operands, and the barrier that ends that half (it
    // waits for the counter anyway, while the other group multiplies) covers
    // their latency.
    const_i32* btrow_s = cbt + int64_t(seq) * a.mbps;
    auto load_id = [&](int kt) __attribute__((always_inline)) -> int32_t {
      return btrow_s[__builtin_amdgcn_readfirstlane(min(kt * 4 + pg, n_pages - 1))];
    };
    // Copy of page pg of block `raw` of K (group 0) or V (group 1; the tensor
    // is a compile-time choice, so the compiler sees which buffers a copy in
    // flight may write) into buffer b.  Every step but an item's last issues
    // exactly one copy, so the counted waits are constants: a step with no page
    // to copy (past the
    // item's tiles or past its last page) copies the page its block id names
    // (the sequence's last page) into the buffer the missing tile would use,
    // which nothing reads before a later copy of the same wavefront, landing
    // after it, or the V-tail zeroing overwrites it.
    auto copy_page = [&](auto tens, auto bufc, int32_t raw) __attribute__((always_inline)) {
      constexpr bool is_v = decltype(tens)::value;
      raw = __builtin_amdgcn_readfirstlane(raw);
      const int32_t blk = raw < 0 ? 0 : (raw >= a.nb ? int32_t(a.nb - 1) : raw);  // never leave the pool
      blk_bad |= blk != raw;
      const int64_t page = (int64_t(blk) * a.hkv + kvh) * page_stride;
      const int lrow0 = pg * kBlock;
      if constexpr (!is_v) {
        char* d = kbuf(bufc);
        const __amdgpu_buffer_rsrc_t r = page_rsrc(kbase + page, int(page_stride));
#pragma unroll
        for (int j = 0; j < IPG; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(d + (lrow0 + j * RPI) * RB), 16, off[j], 0, 0, 0);
      } else {
        char* d = vbuf(bufc);
        const __amdgpu_buffer_rsrc_t r = page_rsrc(vbase + page, int(page_stride));
#pragma unroll
        for (int j = 0; j < IPG; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(d + (lrow0 + j * RPI) * RB), 16, off[j], 0, 0, 0);
      }
    };
    // At the end of a step: wait until at most the copies of this step and of
    // the step before (2 * IPG vector memory operations of this wavefront;
    // they retire in order) are in flight, i.e. the copy of two steps ago,
    // which the next step reads, has landed.
    constexpr int kE = 0x7 << 4, kL = 0xF << 8;  // expcnt and lgkmcnt: not waited for
    static_assert(3 * IPG < 16, "vmcnt low bits");
    auto wait_copy = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(kE | kL | (2 * IPG)); };
    // after the copy has landed (group 1): V rows of keys at or past kv_end become zeros
    auto zero_tail = [&](int kt, auto bufc) __attribute__((always_inline)) {
      char* dv = vbuf(bufc);
      const int key0 = kt * kBN + pg * kBlock;
      if (key0 + kBlock <= kv_end) return;
      for (int idx = lane; idx < kBlock * CH; idx += kWave) {
        const int row = idx / CH;
        if (key0 + row >= kv_end)
          *reinterpret_cast<u32x4*>(dv + (pg * kBlock + row) * RB + (idx % CH) * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    };

    // The products of one half step: S = K_j Q^T from K buffer b = j % 4 and/or
    // O^T += V^T P^T of tile j-1 from V buffer (j-1) % 4, interleaved so that both
    // chains keep the matrix core busy while their operands stream from LDS.
    auto multiply = [&](auto bufc, auto dos, auto dopv) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      constexpr bool DS = decltype(dos)::value, DPV = decltype(dopv)::value;
      // the per-lane offsets are re-formed here rather than kept live across
      // the loop for every buffer (the eight tiles span more than the 64 KiB an
      // LDS read's immediate offset reaches, so each buffer would hold its own)
      int ko = col * RB, vo[DBLK];
#pragma unroll
      for (int db = 0; db < DBLK; ++db) vo[db] = vaddr[db];
      asm volatile("" : "+v"(ko));
#pragma unroll
      for (int db = 0; db < DBLK; ++db) asm volatile("" : "+v"(vo[db]));
      const char* kr = kbuf(bufc) + ko;
      // V_{j-1}: buffer (b + 3) % 4; the last step (no S) takes it at run time
      // (no copy is in flight by then), so one code path serves every parity
      using Prev = std::integral_constant<int, (b + kRing - 1) % kRing>;
      const char* vs = DS ? vbuf(Prev{})
                          : (v_last == 0 ? s_v0 : (v_last == 1 ? s_v1 : (v_last == 2 ? s_v2 : s_v3)));
      u32x4 ka[KSTEPS], kb[KSTEPS], va[NPV];
      auto kread = [&](int kk) __attribute__((always_inline)) {
        const int offk = 16 * ((2 * kk) ^ kx);
        ka[kk] = *reinterpret_cast<const u32x4*>(kr + offk);
        kb[kk] = *reinterpret_cast<const u32x4*>(kr + 32 * RB + offk);
      };
      // 16-key step t = i / DBLK of 32-dim block db = i % DBLK: accumulator rows
      // (t%2)*8 .. +8 of S block t/2, read as two transposed quarters
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int t = i / DBLK, db = i % DBLK;
        const char* vr = vs + vo[db] + 16 * t * RB;
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr + 8 * RB));
        va[i] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v0, v0, 2, 3)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 0, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_shufflevector(v1, v1, 2, 3))};
      };
      auto pv = [&](int i) __attribute__((always_inline)) {
        const int t = i / DBLK, db = i % DBLK;
        const u32x4 pb = {pk[t / 2][(t % 2) * 4 + 0], pk[t / 2][(t % 2) * 4 + 1], pk[t / 2][(t % 2) * 4 + 2],
                          pk[t / 2][(t % 2) * 4 + 3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[i]), as_bf16x8(pb), o[db], 0, 0, 0);
      };
      __builtin_amdgcn_s_setprio(1);
      if constexpr (DS) {
        s[0] = f32x16_t{};
        s[1] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < KLOOK; ++kk) kread(kk);
      }
      if constexpr (DPV) {
#pragma unroll
        for (int i = 0; i < VLOOK; ++i) vread(i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < KSTEPS; ++r) {
        if constexpr (DS) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[r]), as_bf16x8(qf[r]), s[0], 0, 0, 0);
        if constexpr (DPV) pv(2 * r);
        if constexpr (DS) s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[r]), as_bf16x8(qf[r]), s[1], 0, 0, 0);
        if constexpr (DPV) pv(2 * r + 1);
        if constexpr (DS) {
          if (r + KLOOK < KSTEPS) kread(r + KLOOK);
        }
        if constexpr (DPV) {
          if (2 * r + VLOOK < NPV) vread(2 * r + VLOOK);
          if (2 * r + 1 + VLOOK < NPV) vread(2 * r + 1 + VLOOK);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // The softmax of tile kt (S^T in s): causal mask on the tiles that reach
    // past the item's first row, row maxima, lazy rescale, weights P^T in bf16
    // pairs and the row sum of the rounded weights.
    auto softmax_any = [&](int kt) __attribute__((always_inline)) {
      if (kt >= n_full) {
        // accumulator row j of block mb is key kt*64 + lg*4 + mb*32 + (j/4)*8 + j%4
        const int lim = pos - kt * kBN - lg * 4;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (mb * 32 + (j / 4) * 8 + (j % 4) > lim) s[mb][j] = -INFINITY;
      }
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(fmaxf(mx, s[0][j]), s[1][j]);
      mx = pair_max(mx) * a.chunk_scale_log2;
      const bool grow = mx > m + 8.f;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2(m - mx) : 1.f;  // 0 on the first tile (m = -inf)
        m = grow ? mx : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      }
      const float m_use = m == -INFINITY ? 0.f : m;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(fmaf(s[mb][2 * i], a.chunk_scale_log2, -m_use));
          const float p1 = fast_exp2(fmaf(s[mb][2 * i + 1], a.chunk_scale_log2, -m_use));
          pk[mb][i] = pack_bf16(p0, p1);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[mb][i]), kOnes, l, false);
        }
    };

    const int handover_from = n_kt + 1 - kHandoverSteps;

    // Step j (buffer b = j % 4) has the products of tile j (dos: j < n_kt) and
    // of P_{j-1} (dopv: j >= 1).  Each group runs its own loop, so no value of
    // one group's order meets the other's in a join: group 0 multiplies, then
    // (after the barrier) runs the softmax of S_j; group 1 runs the softmax of
    // S_{j-1}, then multiplies.  Both pass the same two barriers per step.
    //
    // Copies: during step j a wavefront copies tile j + lead (K_{j+3} for
    // group 0, V_{j+2} for group 1) with the block id it loaded in the softmax
    // half of the step before, and in its own softmax half loads the block id
    // of the next step's copy.  Its vector memory operations per step are the
    // copy alone (IPG), so at the end of step j it waits for copy_{j-2}, the
    // tile step j+1 reads, while copy_{j-1} and copy_j stay in flight.
    int32_t id_next = 0;  // block id of the copy of the coming step (scalar)
    auto step0 = [&](int j, auto bufc, auto dos, auto dopv) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      multiply(bufc, dos, dopv);
      lds_barrier();
      // the copy (and the claim) go after the products, off their path: K
      // buffer (b + 3) % 4 was last read in step j - 1
      if (j >= handover_from) claim();
      // (the last step copies nothing: its fixed buffer index is not j % 4)
      if constexpr (decltype(dos)::value) copy_page(No{}, std::integral_constant<int, (b + 3) % kRing>{}, id_next);
      if (j >= handover_from) handover();
      id_next = load_id(j + 1 + lead);
      if constexpr (decltype(dos)::value) softmax_any(j);
      wait_copy();  // K_{j+1} has landed
      lds_barrier();
    };
    auto step1 = [&](int j, auto bufc, auto dos, auto dopv) __attribute__((always_inline)) {
      constexpr int b = decltype(bufc)::value;
      if (j >= handover_from) claim();
      // (the last step copies nothing: its fixed buffer index is not j % 4, and
      // a copy into V buffer 2 could overwrite V_{n_kt-1}, which it reads)
      if constexpr (decltype(dos)::value) copy_page(Yes{}, std::integral_constant<int, (b + 2) % kRing>{}, id_next);
      if (j >= handover_from) handover();
      id_next = load_id(j + 1 + lead);
      if constexpr (decltype(dopv)::value) softmax_any(j - 1);
      lds_barrier();
      multiply(bufc, dos, dopv);
      wait_copy();  // V_j has landed
      if (j < n_kt) zero_tail(j, bufc);
      lds_barrier();
    };
    // steps 0 .. n_kt: the first has no P.V, the last no S
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    auto run = [&](auto stepf) __attribute__((always_inline)) {
      stepf(0, I0{}, Yes{}, No{});
      for (int j = 1; j < n_kt; j += 4) {
        stepf(j, I1{}, Yes{}, Yes{});
        if (j + 1 < n_kt) stepf(j + 1, I2{}, Yes{}, Yes{});
        if (j + 2 < n_kt) stepf(j + 2, I3{}, Yes{}, Yes{});
        if (j + 3 < n_kt) stepf(j + 3, I0{}, Yes{}, Yes{});
      }
      // reads V buffer v_last and copies nothing (every later copy of this
      // wavefront lands after the earlier ones, so the counts of the next
      // item's prologue still retire them)
      stepf(n_kt, I0{}, No{}, Yes{});
    };

    if (n_kt > 0) {
      // Prologue: the copies of tiles 0 .. lead-1 and the block id of step 0's
      // copy; group 0 then waits for K_0 (K_1 and K_2 stay in flight).
      if (grp == 0) {
        copy_page(No{}, I0{}, cur.blk0);
        copy_page(No{}, I1{}, n_kt > 1 ? cur.blk1 : cur.blk0);
        copy_page(No{}, I2{}, n_kt > 2 ? cur.blk2 : cur.blk0);
        id_next = load_id(3);
        wait_copy();
      } else {
        copy_page(Yes{}, I0{}, cur.blk0);
        copy_page(Yes{}, I1{}, n_kt > 1 ? cur.blk1 : cur.blk0);
        id_next = load_id(2);
      }
      lds_barrier();
      if (grp == 0) run(step0);
      else run(step1);
    }

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

    // phases a short item had no steps for, each after a barrier (the output
    // stores stay in flight; the next item's counted waits retire them)
    while (phase < kPhases) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the claim has arrived (short items only)
      lds_barrier();
      claim();  // (phase 0 only)
      handover();
    }
    // every wavefront is done with the LDS tiles and has read s_item
    lds_barrier();
    item = next;
    cur = nxt;
  }
  if (blk_bad && lane == 0) atomicOr(&w.hdr[H_FLAGS], PA_FLAG_BLOCK_ID);
  __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS still in flight when the workgroup ends
}

template <int D, int G>
hipError_t launch_t(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chunk_pp_kernel<D, G>, kThreads, 0) != hipSuccess || n <= 0)
      n = 1;
    per_cu = n;
  }
  int64_t grid = int64_t(device_cus()) * per_cu;
  const int64_t cap = w.tiles_cap * a.hkv;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((chunk_pp_kernel<D, G>), dim3(unsigned(grid)), dim3(kThreads), 0, st, a, w);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_t<D, 1>(a, w, st);
    case 2: return launch_t<D, 2>(a, w, st);
    case 4: return launch_t<D, 4>(a, w, st);
    case 8: return launch_t<D, 8>(a, w, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool chunk_pp_supported(int head_dim, int group, int bf16) {
  return bf16 && (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

int chunk_pp_tile_rows(int group) { return kPPRows / group; }

bool chunk_pp_selected(int head_dim, int group, int bf16, int32_t max_query_len) {
  (void)max_query_len;
  // only on request: measured no faster than the four-wavefront kernel on the
  // chunked-prefill step and slower on the mixed one (its items are twice as
  // long, so a step with few of them ends on its longest)
  return chunk_pp_supported(head_dim, group, bf16) && option(PA_OPT_CHUNK_KERNEL) == 2;
}

hipError_t launch_chunk_pp(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  return a.d == 64 ? launch_d<64>(a, w, group, st) : launch_d<128>(a, w, group, st);
}

}  // namespace pa
