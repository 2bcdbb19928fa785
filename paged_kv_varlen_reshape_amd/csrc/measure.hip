// Ceiling kernels: streaming copy, read-only reduction and random page gather
// over HBM, and a bf16 matrix-core loop.
//
// Streaming read and copy: each wavefront takes contiguous runs of the buffer
// (16 KiB for the read, 8 KiB for the copy: 16 or 8 16-byte loads per lane, all
// in flight together) and the runs go round robin over the wavefronts of a
// grid of 16 (read) or 4 (copy) workgroups per CU.  Nontemporal loads and
// stores.  On the MI355X these layouts measured fastest among runs of 1..16
// KiB and grids of 4..16 workgroups per CU (read about 7.0 TB/s, copy about
// 5.4 TB/s counting read and write bytes), so the ceilings are not set by
// issue or latency.
#include "internal.h"
#include "pa_measure.h"

namespace pa {
namespace {

constexpr int kMeasureThreads = 256;
constexpr int kReadRun = 16;  // 1 KiB pieces per wavefront run of the read
constexpr int kCopyRun = 8;   // 1 KiB pieces per wavefront run of the copy
constexpr int kReadWgPerCu = 16;
constexpr int kCopyWgPerCu = 4;

__global__ void __launch_bounds__(kMeasureThreads)
copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = int64_t(gridDim.x) * (kMeasureThreads / kWave);
  const int64_t wave = int64_t(blockIdx.x) * (kMeasureThreads / kWave) + threadIdx.x / kWave;
  const int64_t runs = n / (int64_t(kCopyRun) * kWave);
  for (int64_t r = wave; r < runs; r += waves) {
    const int64_t o = r * kCopyRun * kWave + lane;
    u32x4 v[kCopyRun];
#pragma unroll
    for (int c = 0; c < kCopyRun; ++c) v[c] = __builtin_nontemporal_load(src + o + c * kWave);
#pragma unroll
    for (int c = 0; c < kCopyRun; ++c) __builtin_nontemporal_store(v[c], dst + o + c * kWave);
  }
  // the elements past the last whole run
  const int64_t t = int64_t(blockIdx.x) * kMeasureThreads + threadIdx.x;
  for (int64_t i = runs * kCopyRun * kWave + t; i < n; i += waves * kWave)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ void __launch_bounds__(kMeasureThreads)
read_kernel(const u32x4* __restrict__ src, int64_t n, uint32_t* __restrict__ out) {
  __shared__ uint32_t s[kMeasureThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = int64_t(gridDim.x) * (kMeasureThreads / kWave);
  const int64_t wave = int64_t(blockIdx.x) * (kMeasureThreads / kWave) + threadIdx.x / kWave;
  const int64_t runs = n / (int64_t(kReadRun) * kWave);
  uint32_t acc = 0;
  for (int64_t r = wave; r < runs; r += waves) {
    const u32x4* p = src + r * kReadRun * kWave + lane;
    u32x4 v[kReadRun];
#pragma unroll
    for (int c = 0; c < kReadRun; ++c) v[c] = __builtin_nontemporal_load(p + c * kWave);
#pragma unroll
    for (int c = 0; c < kReadRun; ++c) acc ^= v[c].x ^ v[c].y ^ v[c].z ^ v[c].w;
  }
  const int64_t t = int64_t(blockIdx.x) * kMeasureThreads + threadIdx.x;
  for (int64_t i = runs * kReadRun * kWave + t; i < n; i += waves * kWave) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) acc ^= __shfl_xor(acc, d);
  if (lane == 0) s[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int ww = 0; ww < kMeasureThreads / kWave; ++ww) x ^= s[ww];
    out[blockIdx.x] = x;
  }
}

// Random page gather: one wavefront reads kGatherPages whole pages at a time
// (page_bytes / 1024 16-byte loads per lane and page), the page numbers taken
// from `pages` in order, clamped into the buffer.
constexpr int kGatherPages = 4;

__global__ void __launch_bounds__(kMeasureThreads)
gather_kernel(const char* __restrict__ src, const int32_t* __restrict__ pages, int64_t npages, int64_t src_pages,
              int32_t page_bytes, uint32_t* __restrict__ out) {
  __shared__ uint32_t s[kMeasureThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = int64_t(gridDim.x) * (kMeasureThreads / kWave);
  const int per_lane = page_bytes / (kWave * 16);  // 16-byte loads per lane and page
  uint32_t acc = 0;
  for (int64_t p0 = (int64_t(blockIdx.x) * (kMeasureThreads / kWave) + threadIdx.x / kWave) * kGatherPages;
       p0 < npages; p0 += waves * kGatherPages) {
    const u32x4* base[kGatherPages];
#pragma unroll
    for (int k = 0; k < kGatherPages; ++k) {
      int64_t pg = p0 + k < npages ? pages[p0 + k] : 0;
      pg = pg < 0 ? 0 : (pg >= src_pages ? src_pages - 1 : pg);
      base[k] = reinterpret_cast<const u32x4*>(src + pg * page_bytes);
    }
    for (int j = 0; j < per_lane; ++j) {
      u32x4 v[kGatherPages];
#pragma unroll
      for (int k = 0; k < kGatherPages; ++k)
        v[k] = p0 + k < npages ? __builtin_nontemporal_load(base[k] + j * kWave + lane) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < kGatherPages; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) acc ^= __shfl_xor(acc, d);
  if (lane == 0) s[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int ww = 0; ww < kMeasureThreads / kWave; ++ww) t ^= s[ww];
    out[blockIdx.x] = t;
  }
}

// Matrix-core ceiling: every wavefront runs `iters` rounds of kMfmaChains
// independent v_mfma_f32_32x32x16_bf16 products on register operands (no
// memory inside the loop), two workgroups of four wavefronts per CU.
constexpr int kMfmaChains = 4;
constexpr int kMfmaWgPerCu = 2;
typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(kMeasureThreads)
mfma_kernel(int32_t iters, float* __restrict__ out) {
  // finite, thread-dependent bf16 operands (exponents near 1) so nothing folds
  const uint32_t t = (threadIdx.x + 7u * blockIdx.x) & 0x7fu;
  const uint32_t w0 = 0x3f803f80u | (t << 16) | t;
  const u32x4 av = {w0, w0 ^ 0x10001u, w0 ^ 0x20002u, w0 ^ 0x30003u};
  const u32x4 bv = {w0 ^ 0x40004u, w0 ^ 0x50005u, w0, w0 ^ 0x60006u};
  const mbf16x8_t a = __builtin_bit_cast(mbf16x8_t, av), b = __builtin_bit_cast(mbf16x8_t, bv);
  mf32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = mf32x16_t{};
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = s;
}

// The same loop on operands spread like N(0,1) data: each lane holds four
// sets of bf16 A and B operands with random sign, exponent (2^-3 .. 2^0) and
// mantissa from an integer hash of its global index, and consecutive products
// take different sets, so the multipliers' inputs change with every product as
// they do on real data (the loop above feeds the same values every time).
// iters rounds of kMfmaChains products; iters is a multiple of 4.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {  // integer finaliser (xorshift-multiply)
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  return h;
}
__device__ __forceinline__ uint32_t random_bf16_pair(uint32_t h) {
  const uint32_t lo = (h & 0x807fu) | ((0x7cu + ((h >> 7) & 3u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807fu) | ((0x7cu + ((h >> 23) & 3u)) << 7);
  return lo | (hi << 16);
}

__global__ void __launch_bounds__(kMeasureThreads)
mfma_random_kernel(int32_t iters, float* __restrict__ out) {
  uint32_t h = mix32(threadIdx.x + blockIdx.x * kMeasureThreads + 0x9e3779b9u);
  mbf16x8_t a[4], b[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4 av, bv;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h = mix32(h + 1u);
      av[k] = random_bf16_pair(h);
      h = mix32(h + 1u);
      bv[k] = random_bf16_pair(h);
    }
    a[u] = __builtin_bit_cast(mbf16x8_t, av);
    b[u] = __builtin_bit_cast(mbf16x8_t, bv);
  }
  mf32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = mf32x16_t{};
  for (int32_t i = 0; i < iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + c) & 3], b[(u + 3 * c + 1) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = s;
}

// workgroups per CU -> grid (at most 65536: the read and gather write one word per workgroup)
int measure_grid(int per_cu) {
  const int g = device_cus() * per_cu;
  return g < 65536 ? g : 65536;
}

int check(const void* a, const void* b, size_t bytes, const char* who) {
  if (!a || !b) return fail(PA_ERR_INVALID, "%s: null pointer", who);
  if (bytes == 0 || bytes % 16 != 0) return fail(PA_ERR_INVALID, "%s: bytes must be a positive multiple of 16", who);
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) % 16 != 0)
    return fail(PA_ERR_INVALID, "%s: pointers must be 16-byte aligned", who);
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int pa_measure_copy(void* dst, const void* src, size_t bytes, void* stream) {
  clear_error();
  if (int rc = check(dst, src, bytes, "pa_measure_copy")) return rc;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return fail(PA_ERR_INVALID, "pa_measure_copy: buffers overlap");
  hipLaunchKernelGGL(copy_kernel, dim3(measure_grid(kCopyWgPerCu)), dim3(kMeasureThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), int64_t(bytes / 16));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : fail(PA_ERR_HIP, "pa_measure_copy: launch failed: %s", hipGetErrorString(e));
}

extern "C" int pa_measure_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  clear_error();
  if (int rc = check(src, out, bytes, "pa_measure_read")) return rc;
  hipLaunchKernelGGL(read_kernel, dim3(measure_grid(kReadWgPerCu)), dim3(kMeasureThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), int64_t(bytes / 16), out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : fail(PA_ERR_HIP, "pa_measure_read: launch failed: %s", hipGetErrorString(e));
}

extern "C" int pa_measure_gather(const void* src, int64_t src_pages, const int32_t* pages, int64_t npages,
                                 int32_t page_bytes, uint32_t* out, void* stream) {
  clear_error();
  if (int rc = check(src, out, 16, "pa_measure_gather")) return rc;
  if (!pages || npages <= 0 || src_pages <= 0)
    return fail(PA_ERR_INVALID, "pa_measure_gather: empty page list or buffer");
  if (page_bytes <= 0 || page_bytes % (kWave * 16) != 0)
    return fail(PA_ERR_INVALID, "pa_measure_gather: page_bytes must be a positive multiple of 1024");
  hipLaunchKernelGGL(gather_kernel, dim3(measure_grid(8)), dim3(kMeasureThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(src), pages, npages, src_pages, page_bytes, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : fail(PA_ERR_HIP, "pa_measure_gather: launch failed: %s", hipGetErrorString(e));
}

extern "C" int pa_measure_mfma(int32_t iters, float* out, int64_t* flops, void* stream) {
  clear_error();
  if (!out || !flops) return fail(PA_ERR_INVALID, "pa_measure_mfma: null pointer");
  if (iters <= 0) return fail(PA_ERR_INVALID, "pa_measure_mfma: iters must be positive");
  const int grid = device_cus() * kMfmaWgPerCu;
  if (int64_t(grid) * (kMeasureThreads / kWave) > 65536)
    return fail(PA_ERR_UNSUPPORTED, "pa_measure_mfma: too many compute units for the output buffer");
  *flops = int64_t(grid) * (kMeasureThreads / kWave) * iters * kMfmaChains * (2ll * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(kMeasureThreads), 0, static_cast<hipStream_t>(stream), iters, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : fail(PA_ERR_HIP, "pa_measure_mfma: launch failed: %s", hipGetErrorString(e));
}

extern "C" int pa_measure_mfma_random(int32_t iters, float* out, int64_t* flops, void* stream) {
  clear_error();
  if (!out || !flops) return fail(PA_ERR_INVALID, "pa_measure_mfma_random: null pointer");
  if (iters <= 0 || iters % 4 != 0)
    return fail(PA_ERR_INVALID, "pa_measure_mfma_random: iters must be a positive multiple of 4");
  const int grid = device_cus() * kMfmaWgPerCu;
  if (int64_t(grid) * (kMeasureThreads / kWave) > 65536)
    return fail(PA_ERR_UNSUPPORTED, "pa_measure_mfma_random: too many compute units for the output buffer");
  *flops = int64_t(grid) * (kMeasureThreads / kWave) * iters * kMfmaChains * (2ll * 32 * 32 * 16);
  hipLaunchKernelGGL(mfma_random_kernel, dim3(grid), dim3(kMeasureThreads), 0, static_cast<hipStream_t>(stream), iters,
                     out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK
                         : fail(PA_ERR_HIP, "pa_measure_mfma_random: launch failed: %s", hipGetErrorString(e));
}
