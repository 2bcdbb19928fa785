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
// holds, and V^T is read from LDS in the same key order.
//
// Online softmax in the log2 domain on the VALU; P is rounded to bf16 for the
// PV product and the row sum l adds the rounded values, so the output is an
// exact convex combination of V rows with the rounded weights.  Keys past a
// row's position get -inf by select; K and V of keys past the tile's last
// position are written to LDS as zeros and never read from the pool, so
// nothing outside the sequence reaches the products (NaN-safe).
//
// Staging: 256 threads load one 64-key tile of K and V (16 bytes per load, a
// fully used 256-byte row segment per 16 lanes); K goes to LDS row-major, V is
// transposed in registers (4 keys x 8 dims per thread) and written as V^T
// (bank-conflict-free layout, see the V^T layout note).  LDS holds two tiles: while tile
// kt is multiplied, tile kt+1 (loaded during tile kt-1) is staged into the
// other buffer and the loads of tile kt+2 are issued, with one barrier per
// tile.  The reference maximum of the online softmax moves lazily, so the O
// accumulators are rescaled only when a row's maximum grows by more than 2^8.
// Tiles are taken from a work counter, longest first within a sequence.
#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 128;  // query rows per workgroup tile
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kThreads = 256;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// two floats -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// LDS layout of V^T[d][key]: rows are VS elements apart and the 8-byte key
// groups of row d (four keys each) are permuted by XOR with d/16, i.e. group
// u of row d sits at element d*VS + 4*(u ^ (d>>4)).  With VS = 68 both the
// staging stores (16 lanes: rows 8 apart, one key group) and the operand loads
// (16 lanes: consecutive rows, one key group) touch 32 distinct banks.

constexpr bf16x2_t kOnes = {__bf16(1.0f), __bf16(1.0f)};

template <int D>
struct ChunkCfg {
  static constexpr int KSTEPS = D / 16;            // MFMA k-steps of Q.K (16 dims each)
  static constexpr int DBLK = D / 32;              // 32-dim blocks of O^T
  static constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
  static constexpr int KPT = kBN * CPR / kThreads; // keys staged per thread: 4 (D=128) or 2 (D=64)
  static constexpr int KS = D + 8;                 // LDS row stride of K (elements), padded
  static constexpr int VS = kBN + 4;               // LDS row stride of V^T (elements), padded
  static_assert(KPT == 2 || KPT == 4, "staging layout");
};

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2)
chunk_mfma_kernel(AttnArgs a, Workspace w) {
  using C = ChunkCfg<D>;
  constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, CPR = C::CPR, KPT = C::KPT, KS = C::KS, VS = C::VS;
  constexpr int TQ = kTileRows / G;  // tokens per tile
  constexpr int ROW_BYTES = D * 2;

  // two buffers each: the next tile is staged while this one is multiplied
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2 * D * VS];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 31;  // accumulator column = query row within the wavefront
  const int lg = lane >> 5;   // lane half
  // staging coordinates: 16-byte chunk of a row, and the first of KPT keys
  const int sc = tid % CPR;
  const int sk = (tid / CPR) * KPT;
  // this lane's V^T operand row (col) and key-group bit, see the layout note
  const int vlane = col * VS + (((lg ^ (col >> 4)) & 1) << 2);

  const int n_items = w.hdr[H_TILES] * a.hkv;
  const int64_t page_stride = int64_t(kBlock) * ROW_BYTES;
  const char* kbase = static_cast<const char*>(a.kc);
  const char* vbase = static_cast<const char*>(a.vc);

  if (tid == 0) s_item = blockIdx.x;
  __syncthreads();
  int item = s_item;
  while (item < n_items) {
    __syncthreads();  // every thread has read s_item
    if (tid == 0) s_item = int(gridDim.x) + atomicAdd(&w.hdr[H_COUNTER2], 1);

    const int tile = item / a.hkv;
    const int kvh = item - tile * a.hkv;
    const int2 trec = w.tiles[tile];
    const int seq = trec.x, t0 = trec.y;
    const int r0 = a.qsl[seq];
    const int ctx = max(a.ctx[seq], 0);
    // the plan clamped the rows it tiled the same way: nothing may index
    // outside q, out or the block-table row even with inconsistent metadata
    const int qlen = min(min(a.qsl[seq + 1] - r0, a.num_tokens - r0), a.mbps * kBlock - ctx);
    const int nt = max(0, min(TQ, qlen - t0));  // valid tokens of this tile
    const int kv_end = ctx + t0 + nt;   // keys seen by the tile's last row
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
                                                       ((int64_t(r0) + t0 + tt) * a.hq + head) * ROW_BYTES);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = valid ? qp[2 * kk + lg] : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16_t o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    // staging registers: KPT keys x one 16-byte chunk of K and of V
    u32x4 gk[KPT], gv[KPT];
    auto page_id = [&](int kt) -> int32_t {
      const int page = (kt * kBN + sk) / kBlock;
      int32_t b = page < n_pages ? btrow[page] : 0;
      return b < 0 ? 0 : (b >= a.nb ? int32_t(a.nb - 1) : b);
    };
    auto load_tile = [&](int kt, int32_t blk) {
      const int key = kt * kBN + sk;
      const int64_t off = (int64_t(blk) * a.hkv + kvh) * page_stride + int64_t(key % kBlock) * ROW_BYTES + sc * 16;
      const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off);
      const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool in = key + i < kv_end;
        gk[i] = in ? kp[i * (ROW_BYTES / 16)] : u32x4{0u, 0u, 0u, 0u};
        gv[i] = in ? vp[i * (ROW_BYTES / 16)] : u32x4{0u, 0u, 0u, 0u};
      }
    };
    // K row-major; V transposed: for each of the chunk's 8 dims, KPT consecutive keys
    auto store_tile = [&](int buf) {
      uint16_t* sk_base = s_k + buf * (kBN * KS);
      uint16_t* sv_base = s_vt + buf * (D * VS);
#pragma unroll
      for (int i = 0; i < KPT; ++i) *reinterpret_cast<u32x4*>(&sk_base[(sk + i) * KS + sc * 8]) = gk[i];
      uint32_t wv[KPT][4];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        wv[i][0] = gv[i].x; wv[i][1] = gv[i].y; wv[i][2] = gv[i].z; wv[i][3] = gv[i].w;
      }
      // rows d = sc*8 + e share d>>4 = sc>>1, so one XOR per thread
      uint16_t* vdst = sv_base + sc * 8 * VS + (((sk >> 2) ^ (sc >> 1)) << 2) + (sk & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        const bool hi = e & 1;
        uint16_t* dst = vdst + e * VS;
        const uint32_t a0 = hi ? (wv[0][dw] >> 16) | (wv[1][dw] & 0xFFFF0000u)
                               : (wv[0][dw] & 0xFFFFu) | (wv[1][dw] << 16);
        if constexpr (KPT == 4) {
          const uint32_t a1 = hi ? (wv[2][dw] >> 16) | (wv[3][dw] & 0xFFFF0000u)
                                 : (wv[2][dw] & 0xFFFFu) | (wv[3][dw] << 16);
          *reinterpret_cast<uint2*>(dst) = make_uint2(a0, a1);
        } else {
          *reinterpret_cast<uint32_t*>(dst) = a0;
        }
      }
    };

    // prologue: tile 0 in LDS buffer 0, tile 1 in flight
    int32_t id_next = page_id(0);
    load_tile(0, id_next);
    if (n_kt > 1) id_next = page_id(1);
    store_tile(0);
    if (n_kt > 1) {
      load_tile(1, id_next);
      if (n_kt > 2) id_next = page_id(2);
    }
    __syncthreads();

    // tiles below n_full are visible to every row of the tile: no mask
    const int n_full = (ctx + t0 + 1) / kBN;
    auto tile_step = [&](int kt, auto masked) {
      const int buf = kt & 1;
      const uint16_t* ks = s_k + buf * (kBN * KS);
      const uint16_t* vs = s_vt + buf * (D * VS);
      const int key0 = kt * kBN;
      // S^T = K Q^T: two 32-key blocks
      f32x16_t s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(&ks[(mb * 32 + col) * KS + kk * 16 + lg * 8]);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[kk]), s[mb], 0, 0, 0);
        }
      }
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
      // the final division by l cancels the common factor.
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, fmaxf(s[0][j], s[1][j]));
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
      if (mx > m + 8.f) {
        const float alpha = fast_exp2(m - mx);  // 0 on the first tile (m = -inf)
        m = mx;
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
          const float p0 = fast_exp2(fmaf(s[mb][2 * i], a.scale_log2, -m_use));
          const float p1 = fast_exp2(fmaf(s[mb][2 * i + 1], a.scale_log2, -m_use));
          pk[mb][i] = pack_bf16(p0, p1);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[mb][i]), kOnes, l, false);
        }

      // O^T += V^T P^T: four 16-key steps; step t uses accumulator rows
      // j = (t%2)*8 .. +8 of block t/2, i.e. keys 16t + (i/4)*8 + lg*4 + i%4
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 pb = {pk[t / 2][(t % 2) * 4 + 0], pk[t / 2][(t % 2) * 4 + 1], pk[t / 2][(t % 2) * 4 + 2],
                          pk[t / 2][(t % 2) * 4 + 3]};
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          // row d = db*32 + col: group u = 4t + lg (+2) sits at u ^ (2db + col/16);
          // the lane's bit (lg ^ col/16) is in vlane, the rest is a constant
          const uint16_t* vr = vs + vlane + db * 32 * VS;
          const uint2 v0 = *reinterpret_cast<const uint2*>(vr + (((4 * t) ^ (2 * db)) << 2));
          const uint2 v1 = *reinterpret_cast<const uint2*>(vr + (((4 * t + 2) ^ (2 * db)) << 2));
          const u32x4 va = {v0.x, v0.y, v1.x, v1.y};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o[db], 0, 0, 0);
        }
      }

      // stage tile kt+1 into the other buffer (its loads were issued a tile ago)
      // and start the loads of tile kt+2; one barrier per tile
      if (kt + 1 < n_kt) {
        store_tile(buf ^ 1);
        if (kt + 2 < n_kt) {
          load_tile(kt + 2, id_next);
          if (kt + 3 < n_kt) id_next = page_id(kt + 3);
        }
      }
      __syncthreads();
    };
    for (int kt = 0; kt < min(n_full, n_kt); ++kt) tile_step(kt, std::false_type{});
    for (int kt = max(n_full, 0); kt < n_kt; ++kt) tile_step(kt, std::true_type{});

    // the two lane halves hold disjoint keys of the same row
    l += __shfl_xor(l, 32);
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

    __syncthreads();
    item = s_item;
  }
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
