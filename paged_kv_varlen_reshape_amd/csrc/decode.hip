// decode_streamk + split_merge: row-wise attention over the paged cache on the VALU.
//
// Decoding reads the whole cached context of a request for one new token, so
// it is bound by memory bandwidth (Inside vLLM summary, techfeed.io, section
// "エンジンの中核：スケジューラとKVキャッシュ管理"); the cache is held in
// 16-token blocks reached through each request's block list (same page,
// section "PagedAttentionの仕組み").  A row at absolute position p sees keys
// 0..p.  The same kernel serves decodes, float32 steps and every row of a
// chunk when the MFMA path is off.
//
// Work decomposition (stream-K).  The plan lays every (row, kv head, page)
// unit of the step in one stream and cuts it into equal ranges, one per
// resident wavefront, so every wavefront streams the same number of pages:
// no atomics, no barriers, no tail of uneven items.  A range walks one or more
// segments (a run of pages of one (row, kv head)); a segment that covers its
// whole (row, kv head) writes the normalised output, one that a range
// boundary cuts writes its unnormalised partial (o, max, sum) and split_merge
// folds the pieces.
//
// Inside a segment the wavefront keeps the block ids of up to 64 pages in one
// register (lane j holds page j) and issues each page's K/V loads while the
// previous page is scored (two register buffers).  A page of one kv head is
// one contiguous 16*D*elt run read with 16-byte lanes, so each load
// instruction is a fully coalesced 1 KiB: lane = (token row within the
// instruction, 16-byte chunk of the row).  The GQA group's G query heads share
// every K/V load.  Scores: dot products of the lane's chunk (bf16 pairs on
// v_dot2_f32_bf16, float32 by FMA), summed across the lanes of a token row with
// DPP.  Online softmax per lane row in the log2 domain; at the end of a segment
// the lane rows merge by shuffles.
//
// Algorithmic HBM traffic per unit: 2 * 16 * D * elt bytes of K/V; per
// segment G * D * elt of q and G * D * 4 of output or partial.
#include "internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPR consecutive lanes (LPR = 8, 16 or 32); every lane gets its group's sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror: pairs the two quads of each 8-lane half
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x);  // row_mirror: pairs the two halves of a row
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF16, int D, int G>
struct DecodeCfg {
  static constexpr int ELT = BF16 ? 2 : 4;
  static constexpr int VEC = 16 / ELT;     // elements per 16-byte lane chunk
  static constexpr int LPR = D / VEC;      // lanes per token row
  static constexpr int RPI = kWave / LPR;  // token rows per load instruction
  static constexpr int IPP = kBlock / RPI; // load instructions per 16-token page
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported row width");
};

// Reinterpret one dword as two bf16.  Taking the dword by value matters: this
// clang lowers __builtin_bit_cast applied directly to a vector element (v.y)
// as a read of element 0.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

template <bool BF16>
__device__ __forceinline__ float chunk_dot(const u32x4& q, const u32x4& k) {
  if constexpr (BF16) {
    float acc = 0.f;
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), acc, false);
    return acc;
  } else {
    float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4& v, float* e) {
  if constexpr (BF16) {
    e[0] = bf16lo(v.x); e[1] = bf16hi(v.x); e[2] = bf16lo(v.y); e[3] = bf16hi(v.y);
    e[4] = bf16lo(v.z); e[5] = bf16hi(v.z); e[6] = bf16lo(v.w); e[7] = bf16hi(v.w);
  } else {
    e[0] = __uint_as_float(v.x); e[1] = __uint_as_float(v.y);
    e[2] = __uint_as_float(v.z); e[3] = __uint_as_float(v.w);
  }
}

// One 16-token page of one kv head: IPP 16-byte chunks per lane for K and for V.
template <int IPP>
struct PageRegs {
  u32x4 k[IPP], v[IPP];
};

template <int IPP>
__device__ __forceinline__ void load_page(PageRegs<IPP>& r, const char* kbase, const char* vbase, int64_t off,
                                          int lane) {
  const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off);
  const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off);
#pragma unroll
  for (int i = 0; i < IPP; ++i) r.k[i] = __builtin_nontemporal_load(kp + i * kWave + lane);
#pragma unroll
  for (int i = 0; i < IPP; ++i) r.v[i] = __builtin_nontemporal_load(vp + i * kWave + lane);
}

// Scores of one page for the G heads and the online-softmax update of (m, l, o).
// tbase: position of this lane's first token row; t1: first position not seen.
template <bool BF16, int D, int G>
__device__ __forceinline__ void page_update(PageRegs<DecodeCfg<BF16, D, G>::IPP>& r, const u32x4 (&qv)[G],
                                            int tbase, int t1, bool partial, float scale_log2, float (&m)[G],
                                            float (&l)[G], float (&o)[G][DecodeCfg<BF16, D, G>::VEC]) {
  using C = DecodeCfg<BF16, D, G>;
  constexpr int VEC = C::VEC, LPR = C::LPR, RPI = C::RPI, IPP = C::IPP;
  float s[G][IPP];
#pragma unroll
  for (int i = 0; i < IPP; ++i) {
    const bool valid = tbase + i * RPI < t1;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float d = group_sum<LPR>(chunk_dot<BF16>(qv[h], r.k[i]));
      s[h][i] = valid ? d * scale_log2 : -INFINITY;
    }
  }
  if (partial) {  // last, partly filled page: masked rows must not reach PV (NaN-safe)
#pragma unroll
    for (int i = 0; i < IPP; ++i)
      if (tbase + i * RPI >= t1) r.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // rescale the running sums to the new maxima; scores become weights in place
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = s[h][0];
#pragma unroll
    for (int i = 1; i < IPP; ++i) mx = fmaxf(mx, s[h][i]);
    const float m_new = fmaxf(m[h], mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m[h] - m_use);
    float lsum = l[h] * alpha;
#pragma unroll
    for (int i = 0; i < IPP; ++i) {
      s[h][i] = fast_exp2(s[h][i] - m_use);
      lsum += s[h][i];
    }
    l[h] = lsum;
    m[h] = m_new;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
  }
  // PV, token-outer: one token row's V elements are live at a time
#pragma unroll
  for (int i = 0; i < IPP; ++i) {
    float ve[VEC];
    unpack<BF16>(r.v[i], ve);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(s[h][i], ve[e], o[h][e]);
  }
}

template <bool BF16, int D, int G, int NBUF>
__global__ void __launch_bounds__(256)
decode_streamk_kernel(AttnArgs a, Workspace w) {
  using C = DecodeCfg<BF16, D, G>;
  constexpr int VEC = C::VEC, LPR = C::LPR, IPP = C::IPP;
  constexpr int ROW_BYTES = D * C::ELT;
  constexpr int WPB = 256 / kWave;  // wavefronts per workgroup

  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane / LPR;  // token row of this lane within a load instruction
  const int lc = lane % LPR;  // 16-byte chunk of the row
  const int gwave = blockIdx.x * WPB + threadIdx.x / kWave;
  const int nwaves = gridDim.x * WPB;

  const int nranges = w.hdr[H_RANGES];
  const int64_t units = w.hdr64[H64_UNITS];
  const int64_t per = w.hdr64[H64_PER];
  const int64_t page_stride = int64_t(kBlock) * ROW_BYTES;  // bytes of one (block, kv head) page
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  bool blk_bad = false;  // a block id outside the pool was clamped (reported at the end)
  for (int g = gwave; g < nranges; g += nwaves) {
    int64_t x = g * per;
    const int64_t x_end = min(x + per, units);
    int r = w.range_row[g];
    int4 rec = w.rows[r];
    int64_t base = w.rows_base[r];
    int pages = (rec.z + kBlock - 1) / kBlock;
    int kvh = int((x - base) / pages);
    int p0 = int(x - base - int64_t(kvh) * pages);
    bool first = true;

    while (x < x_end) {
      const int tok = rec.x, seq = rec.y, len = rec.z;
      const int n = int(min(int64_t(pages - p0), x_end - x));  // pages of this segment
      const int32_t* btrow = a.bt + int64_t(seq) * a.mbps + p0;

      // query chunks of the G heads of this kv head
      u32x4 qv[G];
      {
        const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) +
                                                         (int64_t(tok) * a.hq + int64_t(kvh) * G) * ROW_BYTES);
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = qp[h * LPR + lc];
      }

      float m[G], l[G], o[G][VEC];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
      }

      // block ids of the segment's pages, 64 at a time: lane j holds page j of the batch
      int32_t ids = 0;
      auto load_ids = [&](int j0) {
        const int j = j0 + lane;
        const int32_t b = j < n ? btrow[j] : 0;
        ids = b < 0 ? 0 : (b >= a.nb ? int32_t(a.nb - 1) : b);  // never leave the pool
        blk_bad |= ids != b;
      };
      auto page_off = [&](int j) -> int64_t {
        const int32_t b = __builtin_amdgcn_readlane(ids, j & (kWave - 1));
        return (int64_t(b) * a.hkv + kvh) * page_stride;
      };
      auto pos = [&](int j) { return (p0 + j) * kBlock; };

      load_ids(0);
      if constexpr (NBUF == 2) {
        PageRegs<IPP> ra, rb;
        load_page<IPP>(ra, kbase, vbase, page_off(0), lane);
        for (int j = 0; j < n; j += 2) {
          // the next page's loads are in flight while this one is scored
          if (j + 1 < n) {
            if (((j + 1) & (kWave - 1)) == 0) load_ids(j + 1);
            load_page<IPP>(rb, kbase, vbase, page_off(j + 1), lane);
          }
          page_update<BF16, D, G>(ra, qv, pos(j) + lr, len, pos(j) + kBlock > len, a.scale_log2, m, l, o);
          if (j + 1 >= n) break;
          if (j + 2 < n) {
            if (((j + 2) & (kWave - 1)) == 0) load_ids(j + 2);
            load_page<IPP>(ra, kbase, vbase, page_off(j + 2), lane);
          }
          page_update<BF16, D, G>(rb, qv, pos(j + 1) + lr, len, pos(j + 1) + kBlock > len, a.scale_log2, m, l, o);
        }
      } else {
        for (int j = 0; j < n; ++j) {
          if (j > 0 && (j & (kWave - 1)) == 0) load_ids(j);
          PageRegs<IPP> ra;
          load_page<IPP>(ra, kbase, vbase, page_off(j), lane);
          page_update<BF16, D, G>(ra, qv, pos(j) + lr, len, pos(j) + kBlock > len, a.scale_log2, m, l, o);
        }
      }

      // merge the RPI lane rows (lanes that differ above the row width), then
      // the lanes of token row 0 hold the segment's result
      const bool whole = p0 == 0 && n == pages;
      const int64_t slot = int64_t(g) * 2 + (first ? 0 : 1);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float M = m[h];
#pragma unroll
        for (int xx = LPR; xx < kWave; xx <<= 1) M = fmaxf(M, __shfl_xor(M, xx));
        const float f = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - M);
        float lsum = l[h] * f;
#pragma unroll
        for (int xx = LPR; xx < kWave; xx <<= 1) lsum += __shfl_xor(lsum, xx);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float v = o[h][e] * f;
#pragma unroll
          for (int xx = LPR; xx < kWave; xx <<= 1) v += __shfl_xor(v, xx);
          o[h][e] = v;
        }
        if (lr == 0) {
          if (whole) {
            const float inv = 1.f / lsum;
            float* op = a.out + (int64_t(tok) * a.hq + int64_t(kvh) * G + h) * D + lc * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) op[e] = o[h][e] * inv;
          } else {
            float* po = w.part_o + (slot * w.ncol + h) * D + lc * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) po[e] = o[h][e];
            if (lc == 0) w.part_ml[slot * w.ncol + h] = make_float2(M, lsum);
          }
        }
      }

      x += n;
      first = false;
      if (x < x_end) {  // next (row, kv head)
        p0 = 0;
        if (++kvh == a.hkv) {
          kvh = 0;
          rec = w.rows[++r];
          base = w.rows_base[r];
          pages = (rec.z + kBlock - 1) / kBlock;
        }
      }
    }
  }
  if (__any(blk_bad) && lane == 0) atomicOr(&w.hdr[H_FLAGS], PA_FLAG_BLOCK_ID);
}

// split_merge: (record, kv head) pairs cut by range boundaries.  Range g's
// start first cuts the pair whose merge record (cut_record) it holds; the
// pair's parts are the last segment of the range g0 holding its first unit
// (slot 0 if g0 starts exactly there, else slot 1) and the first segment
// (slot 0) of every later range up to the one holding its last unit.  One
// wavefront per (range, query row of the record) folds the G heads of that
// row with a running maximum:
//   M = max_s m_s;  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// The record says everything the fold needs, so a wavefront makes two
// dependent round trips: the record (with the range count beside it), then
// the parts, kParts at a time.  Lane l owns E = G*D/64 consecutive elements of
// a row's G x D output (one head each), so every part is read with wide
// coalesced loads.  Slots hold w.ncol columns (row j, head h is column j*G + h).
constexpr int kParts = 4;

template <int D, int G>
__global__ void __launch_bounds__(256)
split_merge_kernel(AttnArgs a, Workspace w, int64_t max_ranges) {
  constexpr int E = G * D / kWave;  // elements per lane: 1..16
  constexpr int V4 = E >= 4 ? E / 4 : 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ncol = w.ncol;
  const int vrows = a.merge_rows;  // most query rows of one record
  const int64_t waves = int64_t(gridDim.x) * (blockDim.x / kWave);
  const int e0 = lane * E;
  const int h = e0 / D;  // head of this lane's elements
  for (int64_t gj = int64_t(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave; gj < max_ranges * vrows;
       gj += waves) {
    const int64_t g = gj / vrows;
    const int j = int(gj - g * vrows);
    const int4 cut = w.range_cut[g];
    const int nr = w.hdr[H_RANGES];
    if (g >= nr || cut.x < 0 || j >= (cut.y >> 16)) continue;
    const int kvh = cut.y & 0xFFFF;
    const int64_t g0 = cut.z;
    const int nparts = cut.w >> 1, s0 = cut.w & 1;
    const int64_t c0 = int64_t(j) * G;  // the row's first column
    float M = -INFINITY, lsum = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += kParts) {
      float2 ml[kParts];
      float v[kParts][E];
#pragma unroll
      for (int p = 0; p < kParts; ++p) {
        const bool have = p0 + p < nparts;
        const int64_t slot = have ? (g0 + p0 + p) * 2 + (p0 + p == 0 ? s0 : 0) : 0;
        const float* po = w.part_o + (slot * ncol + c0) * D + e0;
        if (have) {
          ml[p] = w.part_ml[slot * ncol + c0 + h];
          if constexpr (V4 > 0) {
#pragma unroll
            for (int c = 0; c < V4; ++c) {
              const float4 t = reinterpret_cast<const float4*>(po)[c];
              v[p][4 * c] = t.x; v[p][4 * c + 1] = t.y; v[p][4 * c + 2] = t.z; v[p][4 * c + 3] = t.w;
            }
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[p][e] = po[e];
          }
        }
      }
#pragma unroll
      for (int p = 0; p < kParts; ++p) {
        if (p0 + p < nparts) {
          const float Mn = fmaxf(M, ml[p].x);
          const float fo = fast_exp2(M - Mn), fn = fast_exp2(ml[p].x - Mn);
          lsum = lsum * fo + ml[p].y * fn;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = acc[e] * fo + v[p][e] * fn;
          M = Mn;
        }
      }
    }
    const float inv = 1.f / lsum;
    float* op = a.out + (int64_t(cut.x + j) * a.hq + int64_t(kvh) * G) * D + e0;
    if constexpr (V4 > 0) {
#pragma unroll
      for (int c = 0; c < V4; ++c)
        reinterpret_cast<float4*>(op)[c] =
            make_float4(acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv, acc[4 * c + 3] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) op[e] = acc[e] * inv;
    }
  }
}

template <bool BF16, int D, int G, int NBUF>
int resident_waves() {
  static int per_cu = 0;  // resident workgroups per CU, from the occupancy calculator
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_streamk_kernel<BF16, D, G, NBUF>, 256, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    per_cu = n;
  }
  const int waves = device_cus() * per_cu * (256 / kWave);
  const int cap = device_cus() * kMaxWavesPerCU;
  return waves < cap ? waves : cap;
}

template <bool BF16, int D, int G, int NBUF>
hipError_t launch_decode_t(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  int64_t waves = resident_waves<BF16, D, G, NBUF>();
  if (waves > w.ranges_cap) waves = w.ranges_cap;
  const int64_t grid = (waves + 3) / 4;
  hipLaunchKernelGGL((decode_streamk_kernel<BF16, D, G, NBUF>), dim3(unsigned(grid)), dim3(256), 0, st, a, w);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_merge_t(const AttnArgs& a, const Workspace& w, int64_t max_ranges, hipStream_t st) {
  // one wavefront per (range, query row of a record): each merge is two
  // dependent round trips, so they all run side by side (a range without a
  // cut exits after the first)
  if (max_ranges > w.ranges_cap) max_ranges = w.ranges_cap;
  const int64_t grid = (max_ranges * a.merge_rows + 3) / 4;
  hipLaunchKernelGGL((split_merge_kernel<D, G>), dim3(unsigned(grid)), dim3(256), 0, st, a, w, max_ranges);
  return hipGetLastError();
}

template <bool BF16, int D, int G>
int waves_g(int nbuf) {
  return nbuf == 2 ? resident_waves<BF16, D, G, 2>() : resident_waves<BF16, D, G, 1>();
}

template <bool BF16, int D>
int waves_d(int group, int nbuf) {
  switch (group) {
    case 1: return waves_g<BF16, D, 1>(nbuf);
    case 2: return waves_g<BF16, D, 2>(nbuf);
    case 4: return waves_g<BF16, D, 4>(nbuf);
    case 8: return waves_g<BF16, D, 8>(nbuf);
    default: return 1;
  }
}

template <bool BF16, int D, int G>
hipError_t launch_decode_g(const AttnArgs& a, const Workspace& w, int nbuf, hipStream_t st) {
  return nbuf == 2 ? launch_decode_t<BF16, D, G, 2>(a, w, st) : launch_decode_t<BF16, D, G, 1>(a, w, st);
}

template <bool BF16, int D>
hipError_t launch_decode_d(const AttnArgs& a, const Workspace& w, int group, int nbuf, hipStream_t st) {
  switch (group) {
    case 1: return launch_decode_g<BF16, D, 1>(a, w, nbuf, st);
    case 2: return launch_decode_g<BF16, D, 2>(a, w, nbuf, st);
    case 4: return launch_decode_g<BF16, D, 4>(a, w, nbuf, st);
    case 8: return launch_decode_g<BF16, D, 8>(a, w, nbuf, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_merge_d(const AttnArgs& a, const Workspace& w, int group, int64_t mr, hipStream_t st) {
  switch (group) {
    case 1: return launch_merge_t<D, 1>(a, w, mr, st);
    case 2: return launch_merge_t<D, 2>(a, w, mr, st);
    case 4: return launch_merge_t<D, 4>(a, w, mr, st);
    case 8: return launch_merge_t<D, 8>(a, w, mr, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_buffers(int group) {
  const int64_t v = option(PA_OPT_DECODE_BUFFERS);
  if (v == 1 || v == 2) return int(v);
  return group >= 8 ? 1 : 2;
}

bool decode_uses_mfma(int bf16) {
  const int64_t v = option(PA_OPT_DECODE_KERNEL);
  return bf16 && v != 1;
}

int decode_waves(int bf16, int head_dim, int group) {
  if (decode_uses_mfma(bf16)) return decode_mfma_waves(head_dim, group);
  const int nbuf = decode_buffers(group);
  if (bf16) return head_dim == 64 ? waves_d<true, 64>(group, nbuf) : waves_d<true, 128>(group, nbuf);
  return head_dim == 64 ? waves_d<false, 64>(group, nbuf) : waves_d<false, 128>(group, nbuf);
}

hipError_t launch_decode(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  if (decode_uses_mfma(a.bf16)) return launch_decode_mfma(a, w, group, st);
  const int nbuf = decode_buffers(group);
  if (a.bf16)
    return a.d == 64 ? launch_decode_d<true, 64>(a, w, group, nbuf, st) : launch_decode_d<true, 128>(a, w, group, nbuf, st);
  return a.d == 64 ? launch_decode_d<false, 64>(a, w, group, nbuf, st) : launch_decode_d<false, 128>(a, w, group, nbuf, st);
}

hipError_t launch_merge(const AttnArgs& a, const Workspace& w, int group, int64_t max_ranges, hipStream_t st) {
  return a.d == 64 ? launch_merge_d<64>(a, w, group, max_ranges, st) : launch_merge_d<128>(a, w, group, max_ranges, st);
}

}  // namespace pa
