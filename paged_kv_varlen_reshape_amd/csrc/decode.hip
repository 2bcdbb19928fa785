// decode_splitk + splitk_reduce: row-wise attention over the paged cache on the VALU.
//
// Decoding reads the whole cached context of a request for one new token, so
// it is bound by memory bandwidth (Inside vLLM summary, techfeed.io, section
// "エンジンの中核：スケジューラとKVキャッシュ管理"); the cache is held in
// 16-token blocks reached through each request's block list (same page,
// section "PagedAttentionの仕組み").  Each work item is one (query row, kv
// head, split of P tokens); a row at absolute position p sees keys 0..p.  The
// same kernel serves decodes, float32 steps and every row of a chunk when the
// MFMA path is off.
//
// Work item -> workgroup of 4 wavefronts.  Wave w takes pages w, w+4, ... of
// the split.  A page of one kv head is one contiguous 16*D*elt run; a wave
// reads it with 16-byte lanes, so each load instruction is a fully coalesced
// 1 KiB: lane = (token row within the instruction, 16-byte chunk of the row).
// The GQA group's G query heads share every K/V load.  Scores: dot products of
// the lane's chunk (bf16 pairs on v_dot2_f32_bf16, float32 by FMA), summed
// across the lanes of a token row with DPP.  Online softmax per lane row in the
// log2 domain; at the end the rows of a wave merge by shuffles and the four
// waves by LDS, and the item writes either the normalised output (one split)
// or its unnormalised partial (o, max, sum) for splitk_reduce.
//
// Algorithmic HBM traffic per item: 2 * split_tokens * D * elt of K/V, plus
// G * D * elt of q and G * D * 4 of output or partial.
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
  static constexpr int NW = kDecodeThreads / kWave;
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

template <bool BF16, int D, int G>
__global__ void __launch_bounds__(kDecodeThreads)
decode_splitk_kernel(AttnArgs a, Workspace w) {
  using C = DecodeCfg<BF16, D, G>;
  constexpr int VEC = C::VEC, LPR = C::LPR, RPI = C::RPI, IPP = C::IPP, NW = C::NW;
  constexpr int ROW_BYTES = D * C::ELT;

  __shared__ float s_o[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int s_next;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lr = lane / LPR;  // token row of this lane within a load instruction
  const int lc = lane % LPR;  // 16-byte chunk of the row

  const int64_t n_items = int64_t(w.hdr[H_SPLITS]) * a.hkv;
  const int P = w.hdr[H_SPLIT_TOKENS];
  const int64_t page_stride = int64_t(kBlock) * ROW_BYTES;  // bytes of one (block, kv head) page
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  for (int64_t item = blockIdx.x; item < n_items;) {
    if (threadIdx.x == 0) s_next = int(gridDim.x) + atomicAdd(&w.hdr[H_COUNTER], 1);

    const int64_t u = item / a.hkv;
    const int kvh = int(item - u * a.hkv);
    const int4 rec = w.items[u];
    const int tok = rec.x, seq = rec.y, len = rec.z;
    const int split = rec.w & (kSingleSplit - 1);
    const bool single = (rec.w & kSingleSplit) != 0;
    const int t0 = split * P;
    const int t1 = min(t0 + P, len);
    const int pg0 = t0 / kBlock, pg1 = (t1 + kBlock - 1) / kBlock;
    const int32_t* btrow = a.bt + int64_t(seq) * a.mbps;

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

    for (int pg = pg0 + wave; pg < pg1; pg += NW) {
      int64_t blk = btrow[pg];
      blk = blk < 0 ? 0 : (blk >= a.nb ? a.nb - 1 : blk);  // never leave the pool
      const int64_t poff = (blk * a.hkv + kvh) * page_stride;
      const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + poff);
      const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + poff);
      u32x4 kr[IPP], vr[IPP];
#pragma unroll
      for (int i = 0; i < IPP; ++i) kr[i] = __builtin_nontemporal_load(kp + i * kWave + lane);
#pragma unroll
      for (int i = 0; i < IPP; ++i) vr[i] = __builtin_nontemporal_load(vp + i * kWave + lane);

      const int tbase = pg * kBlock + lr;
      float s[G][IPP];
#pragma unroll
      for (int i = 0; i < IPP; ++i) {
        const bool valid = tbase + i * RPI < t1;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float d = group_sum<LPR>(chunk_dot<BF16>(qv[h], kr[i]));
          s[h][i] = valid ? d * a.scale_log2 : -INFINITY;
        }
      }
      if (pg * kBlock + kBlock > t1) {  // last, partly filled page: masked rows must not reach PV
#pragma unroll
        for (int i = 0; i < IPP; ++i)
          if (tbase + i * RPI >= t1) vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
      float ve[IPP][VEC];
#pragma unroll
      for (int i = 0; i < IPP; ++i) unpack<BF16>(vr[i], ve[i]);

#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[h][0];
#pragma unroll
        for (int i = 1; i < IPP; ++i) mx = fmaxf(mx, s[h][i]);
        const float m_new = fmaxf(m[h], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m[h] - m_use);
        float lsum = l[h] * alpha;
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = o[h][e] * alpha;
#pragma unroll
        for (int i = 0; i < IPP; ++i) {
          const float p = fast_exp2(s[h][i] - m_use);
          lsum += p;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] = fmaf(p, ve[i][e], acc[e]);
        }
        l[h] = lsum;
        m[h] = m_new;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = acc[e];
      }
    }

    // merge the RPI lane rows of this wave (lanes that differ above the row width)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float M = m[h];
#pragma unroll
      for (int x = LPR; x < kWave; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
      const float f = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - M);
      float lsum = l[h] * f;
#pragma unroll
      for (int x = LPR; x < kWave; x <<= 1) lsum += __shfl_xor(lsum, x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float v = o[h][e] * f;
#pragma unroll
        for (int x = LPR; x < kWave; x <<= 1) v += __shfl_xor(v, x);
        o[h][e] = v;
      }
      if (lr == 0) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_o[wave][h][lc * VEC + e] = o[h][e];
        if (lc == 0) {
          s_m[wave][h] = M;
          s_l[wave][h] = lsum;
        }
      }
    }
    __syncthreads();

    // merge the waves and write
    for (int e = threadIdx.x; e < G * D; e += kDecodeThreads) {
      const int h = e / D, d = e - h * D;
      float M = s_m[0][h];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_m[ww][h]);
      float acc = 0.f, lsum = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = s_m[ww][h];
        const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        acc = fmaf(f, s_o[ww][h][d], acc);
        lsum = fmaf(f, s_l[ww][h], lsum);
      }
      const int64_t head = int64_t(kvh) * G + h;
      if (single) {
        a.out[(int64_t(tok) * a.hq + head) * D + d] = acc / lsum;
      } else {
        const int64_t pi = u * a.hq + head;
        w.part_o[pi * D + d] = acc;
        if (d == 0) w.part_ml[pi] = make_float2(M, lsum);
      }
    }
    __syncthreads();
    item = s_next;
    __syncthreads();
  }
}

// Merge the splits of rows that were cut into more than one:
//   M = max_s m_s;  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
template <int D>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(AttnArgs a, Workspace w) {
  const int64_t n = int64_t(w.hdr[H_REDUCE]) * a.hkv;
  const int G = a.hq / a.hkv;
  for (int64_t job = blockIdx.x; job < n; job += gridDim.x) {
    const int64_t r = job / a.hkv;
    const int kvh = int(job - r * a.hkv);
    const int4 rec = w.reduce[r];
    const int tok = rec.x, u0 = rec.y, ns = rec.z;
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
      const int h = e / D, d = e - h * D;
      const int64_t head = int64_t(kvh) * G + h;
      float M = -INFINITY;
      for (int s = 0; s < ns; ++s) M = fmaxf(M, w.part_ml[(int64_t(u0) + s) * a.hq + head].x);
      float acc = 0.f, lsum = 0.f;
      for (int s = 0; s < ns; ++s) {
        const int64_t pi = (int64_t(u0) + s) * a.hq + head;
        const float2 ml = w.part_ml[pi];
        const float f = ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - M);
        acc = fmaf(f, w.part_o[pi * D + d], acc);
        lsum = fmaf(f, ml.y, lsum);
      }
      a.out[(int64_t(tok) * a.hq + head) * D + d] = acc / lsum;
    }
  }
}

template <bool BF16, int D, int G>
hipError_t launch_decode_t(const AttnArgs& a, const Workspace& w, hipStream_t st) {
  static int per_cu = 0;  // resident workgroups per CU, from the occupancy calculator
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_splitk_kernel<BF16, D, G>, kDecodeThreads, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    per_cu = n;
  }
  const int64_t cap = w.splits_cap * a.hkv;
  int64_t grid = int64_t(device_cus()) * per_cu;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((decode_splitk_kernel<BF16, D, G>), dim3(unsigned(grid)), dim3(kDecodeThreads), 0, st, a, w);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_decode_d(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_decode_t<BF16, D, 1>(a, w, st);
    case 2: return launch_decode_t<BF16, D, 2>(a, w, st);
    case 4: return launch_decode_t<BF16, D, 4>(a, w, st);
    case 8: return launch_decode_t<BF16, D, 8>(a, w, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, const Workspace& w, int group, hipStream_t st) {
  if (a.bf16) return a.d == 64 ? launch_decode_d<true, 64>(a, w, group, st) : launch_decode_d<true, 128>(a, w, group, st);
  return a.d == 64 ? launch_decode_d<false, 64>(a, w, group, st) : launch_decode_d<false, 128>(a, w, group, st);
}

hipError_t launch_reduce(const AttnArgs& a, const Workspace& w, int /*group*/, hipStream_t st) {
  int64_t grid = w.rows_cap * a.hkv;
  if (grid > 2048) grid = 2048;
  if (a.d == 64)
    hipLaunchKernelGGL(splitk_reduce_kernel<64>, dim3(unsigned(grid)), dim3(256), 0, st, a, w);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<128>, dim3(unsigned(grid)), dim3(256), 0, st, a, w);
  return hipGetLastError();
}

}  // namespace pa
