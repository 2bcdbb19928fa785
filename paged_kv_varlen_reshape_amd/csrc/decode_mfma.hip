// decode_mfma: row-wise attention over the paged cache on bf16 MFMA.
//
// Same work as the row-wise VALU kernel (decode rows, and every row of a
// chunk when the chunk kernel is off): a row at absolute position p sees keys
// 0..p of its own sequence, read through 16-token blocks (Inside vLLM summary,
// techfeed.io, section "PagedAttentionの仕組み"); decoding is bound by memory
// bandwidth (section "エンジンの中核：スケジューラとKVキャッシュ管理").  The
// work decomposition is the same stream-K walk: every resident wavefront
// streams an equal range of (row, kv head, page) units, writing the
// normalised output for whole (row, kv head) segments and (o, max, sum)
// partials for segments a range boundary cuts (split_merge folds them).
//
// A record is one decode row, or the nq <= 16 / G rows of a short query
// (speculative-decoding verification): its rows share every K/V page and
// accumulator column c is row c / G, head c % G, with that row's causal limit.
//
// Per 16-token page of one kv head, with the GQA group's G query heads:
//   S^T[key][head] = K Q^T  on v_mfma_f32_16x16x32_bf16 (A = K straight from
//     the pool into registers: lane l holds key l%16, dims 8*(l/16) + 32kk;
//     B = Q: lane l holds head l%16 -- zeros past G -- same dims);
//   in the 16x16 accumulator lane l holds head l%16 and keys 4*(l/16) + 0..3,
//   so a head's page maximum needs two cross-lane steps, and the bf16 weights
//   are already the B operand of
//   O^T[dim][head] += V^T P^T on v_mfma_f32_16x16x16_bf16 (A = V^T: each
//     wavefront DMAs its V page into its own LDS buffer with
//     global_load_lds_dwordx4 and reads it back transposed with
//     ds_read_b64_tr_b16; within 16 lanes, lane i receives the (i%4)-th
//     element of the 8 bytes lane 4k + i/4 addresses, so source lane s
//     addresses V[4g + s/4][16dblk + 4*(s%4)] and lane i gets
//     V[4g + 0..3][16dblk + i] for its lane group g).
// The page's 16-byte chunks are XOR-swizzled by row (2*(row%4) + 8*(row/4%2))
// so the transposed loads touch distinct banks; the DMA picks, per lane, the
// global chunk that belongs in its LDS slot.  NBUF LDS page buffers per
// wavefront (separate arrays, named at compile time) let the next NBUF - 1
// pages' K loads and V DMA fly while the current page is multiplied, with no
// barrier.
//
// Softmax in fp32 in the log2 domain; P is rounded to bf16 for the PV product
// and l sums the rounded weights, so each output is an exact convex
// combination of V rows with the rounded weights.  The reference maximum
// moves lazily (rescale only when a head's maximum grows by more than 2^8).
// Keys past the row get -inf by select and their V rows are zeroed in LDS
// after the DMA, so nothing outside the sequence reaches the products.
#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

template <int B>
using Buf = std::integral_constant<int, B>;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

template <int D>
struct DecM {
  static constexpr int RB = D * 2;          // bytes per K/V row
  static constexpr int CH = RB / 16;        // 16-byte chunks per row: 16 or 8
  static constexpr int RPI = kWave / CH;    // rows per DMA instruction: 4 or 8
  static constexpr int IPG = kBlock / RPI;  // DMA instructions per page
  static constexpr int KS = D / 32;         // QK k-steps (32 dims each)
  static constexpr int DB = D / 16;         // 16-dim blocks of O^T
  static constexpr int PAGE = kBlock * RB;  // bytes of one (block, kv head) page
};

// chunk swizzle of V page row `row` (a bijection of the row's chunks)
template <int CH>
__device__ __forceinline__ int v_swz(int row) {
  return (2 * (row & 3) + 8 * ((row >> 2) & 1)) & (CH - 1);
}

__device__ __forceinline__ void store_f4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store_f2(float2* p, float a, float b) { *p = make_float2(a, b); }

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// pairs per self-planned range whose Q is loaded at the range's start
constexpr int kQSlots = 4;

template <int D, int G, int NBUF, bool SELF>
__global__ void __launch_bounds__(kThreads, 2)
decode_mfma_kernel(AttnArgs a, Workspace w) {
  using C = DecM<D>;
  constexpr int RB = C::RB, CH = C::CH, RPI = C::RPI, IPG = C::IPG, KS = C::KS, DB = C::DB, PAGE = C::PAGE;
  static_assert(G <= 16, "one 16-wide accumulator column per head");
  static_assert(NBUF >= 2 && NBUF <= 4, "page buffers per wavefront");
  constexpr int PER_PAGE = IPG + KS;  // vector memory operations issued per page

  // NBUF page buffers per wavefront (page j in buffer j % NBUF), separate
  // arrays so that the compiler sees the DMA in flight does not write what is
  // being read
  __shared__ __attribute__((aligned(16))) char s_v0[kWaves][PAGE];
  __shared__ __attribute__((aligned(16))) char s_v1[kWaves][PAGE];
  __shared__ __attribute__((aligned(16))) char s_v2[NBUF > 2 ? kWaves : 1][NBUF > 2 ? PAGE : 16];
  __shared__ __attribute__((aligned(16))) char s_v3[NBUF > 3 ? kWaves : 1][NBUF > 3 ? PAGE : 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gwave = blockIdx.x * kWaves + wave;
  auto vbuf = [&](auto bufc) __attribute__((always_inline)) -> char* {
    constexpr int B = decltype(bufc)::value;
    return B == 0 ? s_v0[wave] : B == 1 ? s_v1[wave] : B == 2 ? s_v2[wave] : s_v3[wave];
  };
  const int nwaves = gridDim.x * kWaves;
  // accumulator column: query row hq / G of the record, head hq % G of the group
  // (a decode record has one row; a short query's record has up to 16 / G)
  const int hq = lane & 15;
  const int grp = lane >> 4;  // lane group: keys 4grp..4grp+3 of a page in S
  const int jrow = hq / G, hh = hq - (hq / G) * G;

  // V^T operand addresses of this lane (transposed reads, see the header)
  int vaddr[DB];
  {
    const int s = lane & 15;
    const int row = 4 * grp + (s >> 2);
    const int F = v_swz<CH>(row);
#pragma unroll
    for (int db = 0; db < DB; ++db) vaddr[db] = row * RB + 16 * (((2 * db) + ((s >> 1) & 1)) ^ F) + 8 * (s & 1);
  }
  // DMA: in instruction j of a page, lane -> row j*RPI + lane/CH, LDS chunk lane%CH
  const int dma_row = lane / CH, dma_chunk = lane % CH;

  int nranges = SELF ? 0 : w.hdr[H_RANGES];
  int64_t units = SELF ? 0 : w.hdr64[H64_UNITS];
  int64_t per = SELF ? 1 : w.hdr64[H64_PER];
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  // A small step's row-wise rows (every row of a decode-only step; the
  // single-row sequences of a mixed one, whose chunks the chunk kernel plans
  // for itself) are planned here, by every workgroup for itself,
  // instead of by the plan kernel: the row records and their first units go
  // to LDS (workgroup 0 also stores them, and the step's header, for the
  // merge), and each range finds its first row by binary search.  Same
  // records, units and ranges as the plan kernel's (records of up to
  // merge_rows rows on a short-query step; a sequence with more rows than
  // that, which the plan would give the chunk kernel, becomes several records
  // here).
  __shared__ int4 s_rec[SELF ? kSelfPlanRows : 1];
  __shared__ int64_t s_base[SELF ? kSelfPlanRows : 1];
  __shared__ int64_t s_tot[2 * kWaves];
  int nrec = 0;
  if constexpr (SELF) {
    const int tid = threadIdx.x;
    const int64_t hkv = a.hkv;
    const int vr = a.merge_rows;  // most query rows of one record (1: one record per row)
    constexpr int SPT = kSelfPlanRows / kThreads;  // sequences per thread
    int32_t r0s[SPT], qs[SPT], cs[SPT];
    int64_t nr = 0, nu = 0;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid * SPT + k;
      int32_t r0 = 0, q = 0, c = 0;
      if (i < a.num_seqs) {  // clamped as the plan clamps them
        r0 = a.qsl[i];
        q = int32_t(min(int64_t(max(a.qsl[i + 1] - r0, 0)), int64_t(a.num_tokens) - r0));
        if (r0 < 0 || r0 >= a.num_tokens) q = 0;
        c = max(a.ctx[i], 0);
        if (int64_t(c) + q > a.max_len) q = c >= a.max_len ? 0 : a.max_len - c;
        if (a.self_skip_chunks && q > 1) q = 0;  // a chunk: the chunk kernel's rows
        if (blockIdx.x == 0) {  // metadata clamped above: sticky flag (once, not per workgroup)
          const int f = rows_flag(r0, a.qsl[i + 1], a.ctx[i], a.num_tokens, a.max_len);
          if (f) atomicOr(&w.hdr[H_FLAGS], f);
        }
      }
      r0s[k] = r0;
      qs[k] = q;
      cs[k] = c;
      if (vr <= 1) {  // one record per row: rows c+1 .. c+q keys
        nr += q;
        nu += hkv * (pages_upto(int64_t(c) + q) - pages_upto(c));
      } else {  // records of up to vr consecutive rows, each over its last row's keys
        for (int32_t j = 0; j < q; j += vr) {
          ++nr;
          nu += hkv * ((int64_t(c) + min(q, j + vr) + kBlock - 1) / kBlock);
        }
      }
    }
    // exclusive scans of (rows, units) over the workgroup
    int64_t ir = nr, iu = nu;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int64_t xr = __shfl_up(ir, d), xu = __shfl_up(iu, d);
      if (lane >= d) {
        ir += xr;
        iu += xu;
      }
    }
    if (lane == kWave - 1) {
      s_tot[wave] = ir;
      s_tot[kWaves + wave] = iu;
    }
    __syncthreads();
    int64_t br = 0, bu = 0, tr = 0, tu = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      br += ww < wave ? s_tot[ww] : 0;
      bu += ww < wave ? s_tot[kWaves + ww] : 0;
      tr += s_tot[ww];
      tu += s_tot[kWaves + ww];
    }
    int64_t r = br + ir - nr, u = bu + iu - nu;
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int step = vr > 1 ? vr : 1;
      for (int32_t j = 0; j < qs[k] && r < kSelfPlanRows; j += step, ++r) {
        const int32_t nq = min(step, qs[k] - j);  // the record's rows j .. j + nq - 1
        const int32_t len = cs[k] + j + nq;       // keys its last row sees
        s_rec[r] = make_int4(r0s[k] + j, tid * SPT + k, len, nq);
        s_base[r] = u;
        u += hkv * ((len + kBlock - 1) / kBlock);
      }
    }
    __syncthreads();
    nrec = int(min(tr, int64_t(kSelfPlanRows)));
    units = tu;
    per = a.fixed_units > 0 ? a.fixed_units : (units + a.num_ranges - 1) / a.num_ranges;
    if (per < 1) per = 1;
    int64_t n_r = (units + per - 1) / per;
    if (n_r > w.ranges_cap) {
      per = (units + w.ranges_cap - 1) / w.ranges_cap;
      n_r = (units + per - 1) / per;
    }
    nranges = int(n_r);
    if (blockIdx.x == 0) {
      for (int rr = tid; rr < nrec; rr += kThreads) {
        w.rows[rr] = s_rec[rr];
        w.rows_base[rr] = s_base[rr];
      }
      if (tid == 0) {
        w.hdr[H_ROWS] = nrec;
        w.hdr[H_TILES] = 0;
        w.hdr[H_RANGES] = nranges;
        w.hdr64[H64_UNITS] = units;
        w.hdr64[H64_PER] = per;
      }
    }
  }
  bool blk_bad = false;  // a block id outside the pool was clamped (reported at the end)
  auto rec_at = [&](int r) __attribute__((always_inline)) -> int4 { return SELF ? s_rec[r] : w.rows[r]; };
  auto base_at = [&](int r) __attribute__((always_inline)) -> int64_t { return SELF ? s_base[r] : w.rows_base[r]; };

  // O^T += V^T P^T for one page.  Keys at or past `nvalid` (the last, partly
  // filled page of a row) may hold anything, so their V elements are zeroed
  // in the operand registers: element j of a lane's transposed read is key
  // 4grp + j of the page.
  auto pv_page = [&](f32x4_t (&o)[DB], bf16x4_t pw, const char* vs, int nvalid) __attribute__((always_inline)) {
    uint32_t m01 = ~0u, m23 = ~0u;
    if (nvalid < kBlock) {
      const int k0 = 4 * grp;
      m01 = (k0 < nvalid ? 0xFFFFu : 0u) | (k0 + 1 < nvalid ? 0xFFFF0000u : 0u);
      m23 = (k0 + 2 < nvalid ? 0xFFFFu : 0u) | (k0 + 3 < nvalid ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs + vaddr[db]));
      uint2 u = __builtin_bit_cast(uint2, v);
      u.x &= m01;
      u.y &= m23;
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, u), pw, o[db], 0, 0, 0);
    }
  };

  // A self-planned range streams its pages as one sequence across the (row,
  // kv head) pairs it covers, with no memory round trip at a pair boundary:
  // at the range's start one load per lane fetches the block id (and notes
  // the kv head) of each of its first 64 pages, and the Q of its first
  // kQSlots pairs comes into registers; the next pair's first page is then
  // issued while the current pair's last page is multiplied.  Inside the
  // loop only the page copies are loads in flight and LDS is touched only by
  // the copies and the V operand reads, so the compiler's own waits stay
  // per page.  (The records are in LDS; a decode record has one query row, a
  // short query's up to 16 / G.)
  auto flat_range = [&](int g, int64_t x, int64_t x_end, int r, int kvh, int p0) __attribute__((always_inline)) {
    if constexpr (SELF) {
      const int hkv = a.hkv;
      const int total = int(x_end - x);
      // (record fields are wave-uniform: read them into scalars)
      auto pages_of = [&](int rr) __attribute__((always_inline)) {
        return __builtin_amdgcn_readfirstlane((s_rec[rr].z + kBlock - 1) / kBlock);
      };
      auto next_pair = [&](int& rr, int& kh) __attribute__((always_inline)) {
        if (++kh == hkv) {
          kh = 0;
          ++rr;
        }
      };
      // Q of pair (rr, kh) as the B operand: lane holds row jrow, head hh of the
      // record (zeros past its rows), dims 8grp + 32kk
      auto load_q = [&](int rr, int kh, u32x4 (&qq)[KS]) __attribute__((always_inline)) {
        const bool ok = jrow < __builtin_amdgcn_readfirstlane(s_rec[rr].w);
        const int tok = __builtin_amdgcn_readfirstlane(s_rec[rr].x) + (ok ? jrow : 0);
        const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) +
                                                         (int64_t(tok) * a.hq + int64_t(kh) * G + hh) * RB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qq[kk] = ok ? qp[grp + 4 * kk] : u32x4{0u, 0u, 0u, 0u};
      };

      // page table of the stream, 64 pages at a time: lane j holds the block id
      // and kv head of stream page f0 + j; (tr, tkh, tp) is the batch's first page
      int tr = r, tkh = kvh, tp = p0;
      int32_t ids = 0, khs = 0;
      auto table = [&](int f0) __attribute__((always_inline)) {
        int rr = tr, kh = tkh, p = tp + lane, pg = pages_of(rr);
        const bool mine = f0 + lane < total;
        while (mine && p >= pg) {
          p -= pg;
          next_pair(rr, kh);
          pg = pages_of(rr);
        }
        ids = mine ? a.bt[int64_t(s_rec[rr].y) * a.mbps + p] : 0;
        khs = kh;
        if (f0 + kWave < total) {  // the next batch's first page
          tp += kWave;
          while (tp >= pages_of(tr)) {
            tp -= pages_of(tr);
            next_pair(tr, tkh);
          }
        }
      };
      table(0);
      // Q of the range's first kQSlots pairs (a later pair's is loaded when it starts)
      u32x4 qall[kQSlots][KS];
      {
        int rr = r, kh = kvh, left = total - (pages_of(r) - p0);
#pragma unroll
        for (int k = 0; k < kQSlots; ++k) {
          if (k == 0 || left > 0) {
            if (k > 0) {
              next_pair(rr, kh);
              left -= pages_of(rr);
            }
            load_q(rr, kh, qall[k]);
          }
        }
      }
      // the block ids are needed for the first page anyway; with the Q loads
      // done too, the page loop starts with nothing else in flight
      wait_vmcnt<0>();

      // V pages come into registers (the same 1 KB runs per instruction as the
      // LDS copy would read) and are written to the page's LDS buffer when it
      // is multiplied: on short ranges (tens of pages) this measured faster
      // than copying them with global_load_lds
      u32x4 vreg[NBUF][IPG];
      auto issue = [&](int f, u32x4 (&kf)[KS], auto bufc) __attribute__((always_inline)) {
        if (f > 0 && (f & (kWave - 1)) == 0) table(f);
        const int32_t braw = __builtin_amdgcn_readlane(ids, f & (kWave - 1));
        const int kh = __builtin_amdgcn_readlane(khs, f & (kWave - 1));
        const int32_t b = braw < 0 ? 0 : (braw >= a.nb ? int32_t(a.nb - 1) : braw);  // never leave the pool
        blk_bad |= b != braw;
        const int64_t pb = (int64_t(b) * hkv + kh) * PAGE;
#pragma unroll
        for (int ii = 0; ii < IPG; ++ii) {
          const int row = ii * RPI + dma_row;
          const int64_t gv = pb + int64_t(row) * RB + 16 * (dma_chunk ^ v_swz<CH>(row));
          vreg[decltype(bufc)::value][ii] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + gv));
        }
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + pb + int64_t(hq) * RB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kf[kk] = __builtin_nontemporal_load(kp + grp + 4 * kk);
      };

      // compute side: pair (cr, ckh) (the range's pair number cn), page cp; this range's part of it began at cp0
      int cr = r, ckh = kvh, cn = 0, cp = p0, cp0 = p0, cleft = total, cpages = pages_of(r);
      int clen = __builtin_amdgcn_readfirstlane(s_rec[r].z);  // keys the record's last row sees
      int cnq = __builtin_amdgcn_readfirstlane(s_rec[r].w);   // the record's rows
      u32x4 qf[KS];
      f32x4_t o[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x4_t{};
      float m = -INFINITY, l = 0.f;
      auto compute = [&](const u32x4 (&kf)[KS], auto bufc) __attribute__((always_inline)) {
        if (cp == cp0) {
          if (cn < kQSlots) {
#pragma unroll
            for (int k = 0; k < kQSlots; ++k)
              if (__builtin_amdgcn_readfirstlane(cn) == k) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) qf[kk] = qall[k][kk];
              }
          } else {
            load_q(cr, ckh, qf);
            wait_vmcnt<0>();  // rare (a range over many short pairs): keep the loop's waits per page
          }
        }
        char* vs = vbuf(bufc);
#pragma unroll
        for (int ii = 0; ii < IPG; ++ii)
          *reinterpret_cast<u32x4*>(vs + ii * RPI * RB + 16 * lane) = vreg[decltype(bufc)::value][ii];
        const int pos0 = cp * kBlock;  // first key of the page
        f32x4_t sc = f32x4_t{};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]),
                                                      __builtin_bit_cast(bf16x8_t, qf[kk]), sc, 0, 0, 0);
        const int kfirst = pos0 + 4 * grp;   // key of accumulator row 0 of this lane
        const int lim = clen - cnq + 1 + jrow;  // keys this column's row sees
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = kfirst + i < lim ? sc[i] * a.scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m + 8.f) {  // lazy rescale: weights stay <= 2^8
          const float alpha = fast_exp2(m - mx);
          m = mx;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
        const float m_use = m == -INFINITY ? 0.f : m;
        const uint32_t p01 = pack_bf16(fast_exp2(sc[0] - m_use), fast_exp2(sc[1] - m_use));
        const uint32_t p23 = pack_bf16(fast_exp2(sc[2] - m_use), fast_exp2(sc[3] - m_use));
        l += __uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xFFFF0000u) + __uint_as_float(p23 << 16) +
             __uint_as_float(p23 & 0xFFFF0000u);
        const bf16x4_t pv = __builtin_bit_cast(bf16x4_t, make_uint2(p01, p23));
        pv_page(o, pv, vs, clen - pos0);
        --cleft;
        if (++cp == cpages || cleft == 0) {
          // this range's part of the pair is done: the four lane groups hold disjoint keys
          float lt = l + __shfl_xor(l, 16);
          lt += __shfl_xor(lt, 32);
          const bool whole = cp0 == 0 && cp == cpages;
          const int64_t slot = int64_t(g) * 2 + (cn == 0 ? 0 : 1);
          if (jrow < cnq) {
            if (whole) {
              const float inv = 1.f / lt;
              float* op = a.out + (int64_t(s_rec[cr].x + jrow) * a.hq + int64_t(ckh) * G + hh) * D + 4 * grp;
#pragma unroll
              for (int db = 0; db < DB; ++db)
                store_f4(op + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
            } else {
              float* po = w.part_o + (slot * w.ncol + hq) * D + 4 * grp;
#pragma unroll
              for (int db = 0; db < DB; ++db)
                store_f4(po + 16 * db, o[db][0], o[db][1], o[db][2], o[db][3]);
              if (grp == 0) store_f2(w.part_ml + slot * w.ncol + hq, m, lt);
            }
          }
          if (cleft > 0) {  // the next pair
            next_pair(cr, ckh);
            ++cn;
            cp = 0;
            cp0 = 0;
            cpages = pages_of(cr);
            clen = __builtin_amdgcn_readfirstlane(s_rec[cr].z);
            cnq = __builtin_amdgcn_readfirstlane(s_rec[cr].w);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = f32x4_t{};
            m = -INFINITY;
            l = 0.f;
          }
        }
      };

      // stream page f uses LDS buffer and K register set f % NBUF; pages
      // f + 1 .. f + NBUF - 1 fly while page f (landed) is multiplied
      u32x4 kset[NBUF][KS];
      issue(0, kset[0], Buf<0>{});
      if constexpr (NBUF > 2) {
        if (1 < total) issue(1, kset[1], Buf<1>{});
      }
      if constexpr (NBUF > 3) {
        if (2 < total) issue(2, kset[2], Buf<2>{});
      }
      // a full step: the page NBUF - 1 ahead exists
      auto step = [&](int f, auto bufc) __attribute__((always_inline)) {
        constexpr int B = decltype(bufc)::value;
        constexpr int BN = (B + NBUF - 1) % NBUF;
        issue(f + NBUF - 1, kset[BN], Buf<BN>{});
        wait_vmcnt<(NBUF - 1) * PER_PAGE>();
        compute(kset[B], bufc);
      };
      // a step near the end of the stream: `later` pages fly behind page f
      auto tail_step = [&](int f, auto bufc) __attribute__((always_inline)) {
        constexpr int B = decltype(bufc)::value;
        constexpr int BN = (B + NBUF - 1) % NBUF;
        if (f >= total) return;
        if (f + NBUF - 1 < total) issue(f + NBUF - 1, kset[BN], Buf<BN>{});
        const int later = min(NBUF - 1, total - 1 - f);
        if (later >= 3) wait_vmcnt<3 * PER_PAGE>();
        else if (later == 2) wait_vmcnt<2 * PER_PAGE>();
        else if (later == 1) wait_vmcnt<PER_PAGE>();
        else wait_vmcnt<0>();
        compute(kset[B], bufc);
      };
      // every pass of the loop runs NBUF full steps (one path through it, so
      // the compiler's own waits for the K registers stay per page)
      int f = 0;
      for (; f + 2 * NBUF - 2 < total; f += NBUF) {
        step(f, Buf<0>{});
        step(f + 1, Buf<1>{});
        if constexpr (NBUF > 2) step(f + 2, Buf<2 % NBUF>{});
        if constexpr (NBUF > 3) step(f + 3, Buf<3 % NBUF>{});
      }
      // at most 2 * NBUF - 2 pages are left
      tail_step(f, Buf<0>{});
      tail_step(f + 1, Buf<1 % NBUF>{});
      tail_step(f + 2, Buf<2 % NBUF>{});
      if constexpr (NBUF > 2) {
        tail_step(f + 3, Buf<3 % NBUF>{});
      }
      if constexpr (NBUF > 3) {
        tail_step(f + 4, Buf<4 % NBUF>{});
        tail_step(f + 5, Buf<5 % NBUF>{});
      }
    }
  };

  for (int g = gwave; g < nranges; g += nwaves) {
    int64_t x = g * per;
    const int64_t x_end = min(x + per, units);
    int r;
    if constexpr (SELF) {
      // the last row whose first unit is at or before x
      int lo = 0, hi = nrec;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_base[mid] <= x) lo = mid;
        else hi = mid;
      }
      r = lo;
      // the range's cut record for the merge: a start `off` units into its
      // (row, kv head) is the first boundary strictly inside it iff 0 < off <= per
      const int pg = (s_rec[r].z + kBlock - 1) / kBlock;
      const int64_t rel = x - s_base[r];
      const int k = int(rel / pg);
      const int64_t off = rel - int64_t(k) * pg;
      if (lane == 0) {
        const int4 c = off > 0 && off <= per ? cut_record(x - off, pg, per, s_rec[r].x, k, s_rec[r].w)
                                             : make_int4(-1, -1, -1, -1);
        w.range_cut[g] = c;
      }
      flat_range(g, x, x_end, r, k, int(off));
      continue;
    } else {
      r = w.range_row[g];
    }
    int4 rec = rec_at(r);
    int64_t base = base_at(r);
    int pages = (rec.z + kBlock - 1) / kBlock;
    int kvh = int((x - base) / pages);
    int p0 = int(x - base - int64_t(kvh) * pages);
    bool first = true;

    while (x < x_end) {
      const int tok = rec.x, seq = rec.y, len = rec.z, nq = rec.w;
      const bool col_ok = jrow < nq;
      const int lim = len - nq + 1 + jrow;  // keys this column's row sees
      const int n = int(min(int64_t(pages - p0), x_end - x));  // pages of this segment
      const int32_t* btrow = a.bt + int64_t(seq) * a.mbps + p0;

      // Q as the B operand: row jrow, head hh (zeros past the record), dims 8*grp + 32kk
      u32x4 qf[KS];
      {
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            static_cast<const char*>(a.q) + (int64_t(tok + (col_ok ? jrow : 0)) * a.hq + int64_t(kvh) * G + hh) * RB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qf[kk] = col_ok ? qp[grp + 4 * kk] : u32x4{0u, 0u, 0u, 0u};
      }

      f32x4_t o[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x4_t{};
      float m = -INFINITY, l = 0.f;

      // block ids of the segment's pages, 64 at a time: lane j holds page j of the batch
      int32_t ids = 0;
      auto load_ids = [&](int j0) {
        const int j = j0 + lane;
        const int32_t b = j < n ? btrow[j] : 0;
        ids = b < 0 ? 0 : (b >= a.nb ? int32_t(a.nb - 1) : b);  // never leave the pool
        blk_bad |= ids != b;
      };
      auto page_base = [&](int j) -> int64_t {
        const int32_t b = __builtin_amdgcn_readlane(ids, j & (kWave - 1));
        return (int64_t(b) * a.hkv + kvh) * PAGE;
      };
      // K of page j straight into the A-operand layout; V of page j by DMA into buffer B
      auto issue = [&](int j, u32x4 (&kf)[KS], auto bufc) {
        if (j > 0 && (j & (kWave - 1)) == 0) load_ids(j);
        const int64_t pb = page_base(j);
        char* dv = vbuf(bufc);
#pragma unroll
        for (int ii = 0; ii < IPG; ++ii) {
          const int row = ii * RPI + dma_row;
          const int64_t gv = pb + int64_t(row) * RB + 16 * (dma_chunk ^ v_swz<CH>(row));
          __builtin_amdgcn_global_load_lds(vbase + gv, (lds_void_t*)(dv + ii * RPI * RB), 16, 0, 0);
        }
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + pb + int64_t(hq) * RB);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kf[kk] = __builtin_nontemporal_load(kp + grp + 4 * kk);
      };
      // one page: scores, online softmax, PV
      auto compute = [&](int j, const u32x4 (&kf)[KS], auto bufc) {
        char* vs = vbuf(bufc);
        const int pos0 = (p0 + j) * kBlock;  // first key of the page
        f32x4_t s = f32x4_t{};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]),
                                                     __builtin_bit_cast(bf16x8_t, qf[kk]), s, 0, 0, 0);
        const int kfirst = pos0 + 4 * grp;  // key of accumulator row 0 of this lane
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = kfirst + i < lim ? s[i] * a.scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m + 8.f) {  // lazy rescale: weights stay <= 2^8
          const float alpha = fast_exp2(m - mx);
          m = mx;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
        const float m_use = m == -INFINITY ? 0.f : m;
        const uint32_t p01 = pack_bf16(fast_exp2(s[0] - m_use), fast_exp2(s[1] - m_use));
        const uint32_t p23 = pack_bf16(fast_exp2(s[2] - m_use), fast_exp2(s[3] - m_use));
        l += __uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xFFFF0000u) + __uint_as_float(p23 << 16) +
             __uint_as_float(p23 & 0xFFFF0000u);
        const bf16x4_t pb = __builtin_bit_cast(bf16x4_t, make_uint2(p01, p23));
        pv_page(o, pb, vs, len - pos0);
      };

      // pages j+1 .. j+NBUF-1 fly while page j is multiplied: page j uses
      // buffer j % NBUF and K register set j % NBUF (static in the unrolled loop)
      load_ids(0);
      u32x4 kset[NBUF][KS];
      issue(0, kset[0], Buf<0>{});
      if constexpr (NBUF > 2) {
        if (1 < n) issue(1, kset[1], Buf<1>{});
      }
      if constexpr (NBUF > 3) {
        if (2 < n) issue(2, kset[2], Buf<2>{});
      }
      auto step = [&](int j, auto bufc) __attribute__((always_inline)) {
        constexpr int B = decltype(bufc)::value;
        constexpr int BN = (B + NBUF - 1) % NBUF;  // buffer of page j + NBUF - 1
        if (j >= n) return;
        if (j + NBUF - 1 < n) issue(j + NBUF - 1, kset[BN], Buf<BN>{});
        // page j's V copy and K loads have landed; the pages issued after it may fly
        const int later = min(NBUF - 1, n - 1 - j);
        if (later >= 3) wait_vmcnt<3 * PER_PAGE>();
        else if (later == 2) wait_vmcnt<2 * PER_PAGE>();
        else if (later == 1) wait_vmcnt<PER_PAGE>();
        else wait_vmcnt<0>();
        compute(j, kset[B], bufc);
      };
      for (int j0 = 0; j0 < n; j0 += NBUF) {
        step(j0, Buf<0>{});
        step(j0 + 1, Buf<1>{});
        if constexpr (NBUF > 2) step(j0 + 2, Buf<2>{});
        if constexpr (NBUF > 3) step(j0 + 3, Buf<3>{});
      }

      // the four lane groups hold disjoint keys of each head
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      // accumulator row i of block db is dim 16db + 4grp + i
      const bool whole = p0 == 0 && n == pages;
      const int64_t slot = int64_t(g) * 2 + (first ? 0 : 1);
      if (col_ok) {
        if (whole) {
          const float inv = 1.f / l;
          float* op = a.out + (int64_t(tok + jrow) * a.hq + int64_t(kvh) * G + hh) * D + 4 * grp;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            store_f4(op + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
        } else {
          float* po = w.part_o + (slot * w.ncol + hq) * D + 4 * grp;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            store_f4(po + 16 * db, o[db][0], o[db][1], o[db][2], o[db][3]);
          if (grp == 0) store_f2(w.part_ml + slot * w.ncol + hq, m, l);
        }
      }

      x += n;
      first = false;
      if (x < x_end) {  // next (row, kv head)
        p0 = 0;
        if (++kvh == a.hkv) {
          kvh = 0;
          rec = rec_at(++r);
          base = base_at(r);
          pages = (rec.z + kBlock - 1) / kBlock;
        }
      }
    }
  }
  if (__any(blk_bad) && lane == 0) atomicOr(&w.hdr[H_FLAGS], PA_FLAG_BLOCK_ID);
}

template <int D, int G, int NBUF>
int resident_waves_t() {
  static int per_cu = 0;  // resident workgroups per CU, from the occupancy calculator
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<D, G, NBUF, false>, kThreads, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    per_cu = n;
  }
  const int waves = device_cus() * per_cu * kWaves;
  const int cap = device_cus() * kMaxWavesPerCU;
  return waves < cap ? waves : cap;
}

template <int D, int G, int NBUF>
hipError_t launch_t(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  int64_t waves = resident_waves_t<D, G, NBUF>();
  if (waves > w.ranges_cap) waves = w.ranges_cap;
  if (a.self_plan) {  // its ranges are at most the requested count: launch just those wavefronts
    const int64_t want = a.fixed_units > 0 ? w.ranges_cap : a.num_ranges;
    if (waves > want) waves = want;
  }
  const int64_t grid = (waves + kWaves - 1) / kWaves;
  if (a.self_plan)
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, 2, true>), dim3(unsigned(grid)), dim3(kThreads), 0, st, a, w);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, NBUF, false>), dim3(unsigned(grid)), dim3(kThreads), 0, st, a, w);
  return hipGetLastError();
}

// page buffers per wavefront: the option when it names 2..4, else 2 (three and
// four measured no faster on the decode-only and long-context steps, with
// 18 / 38 more registers)
int mfma_buffers() {
  const int64_t v = option(PA_OPT_DECODE_BUFFERS);
  return v >= 2 && v <= 4 ? int(v) : 2;
}

template <int D, int G>
int waves_g() {
  switch (mfma_buffers()) {
    case 4: return resident_waves_t<D, G, 4>();
    case 3: return resident_waves_t<D, G, 3>();
    default: return resident_waves_t<D, G, 2>();
  }
}

template <int D, int G>
hipError_t launch_g(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  switch (mfma_buffers()) {
    case 4: return launch_t<D, G, 4>(a, w, st);
    case 3: return launch_t<D, G, 3>(a, w, st);
    default: return launch_t<D, G, 2>(a, w, st);
  }
}

template <int D>
int waves_d(int group) {
  switch (group) {
    case 1: return waves_g<D, 1>();
    case 2: return waves_g<D, 2>();
    case 4: return waves_g<D, 4>();
    case 8: return waves_g<D, 8>();
    default: return 1;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_g<D, 1>(a, w, st);
    case 2: return launch_g<D, 2>(a, w, st);
    case 4: return launch_g<D, 4>(a, w, st);
    case 8: return launch_g<D, 8>(a, w, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Decode ranges of a step by default: one workgroup's wavefronts per CU.  Every
// CU then streams the same share, and fewer wavefronts per CU measured faster
// than the three workgroups that fit (configuration 2: 63 vs 70 us; range
// counts that are not a multiple of the CU count leave some CUs a second
// workgroup, whose share then sets the tail).
int decode_mfma_waves(int head_dim, int group) {
  const int resident = head_dim == 64 ? waves_d<64>(group) : waves_d<128>(group);
  const int one_per_cu = device_cus() * kWaves;
  return one_per_cu < resident ? one_per_cu : resident;
}

hipError_t launch_decode_mfma(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  return a.d == 64 ? launch_d<64>(a, w, group, st) : launch_d<128>(a, w, group, st);
}

}  // namespace pa
