// reshape_and_cache: the step's new K/V rows written into their paged cache slots.
//
// Before attention reads the cache, every new token's K and V rows go to the
// slot its request's block list gives it (Inside vLLM summary, techfeed.io,
// section "PagedAttentionの仕組み": blocks of 16 tokens per request and the
// flattened super-sequence of the step).
//
// HBM-bound raw copy.  One thread moves one 16-byte chunk of one (token,
// kv head) row; consecutive threads take consecutive chunks of the source, so
// reads are fully coalesced and each destination row (head_dim elements of one
// page) is written as one contiguous run.  Algorithmic traffic per token:
// 2 * Hkv * head_dim * elt read + the same written + 4 bytes of slot.
#include "internal.h"

namespace pa {
namespace {

__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                         const int32_t* __restrict__ slots, u32x4* __restrict__ kc,
                         u32x4* __restrict__ vc, int64_t total_chunks, int32_t hkv,
                         int32_t chunks_per_row, int64_t num_slots) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
    const int64_t row = c / chunks_per_row;        // token * hkv + head
    const int32_t part = int32_t(c - row * chunks_per_row);
    const int64_t tok = row / hkv;
    const int32_t head = int32_t(row - tok * hkv);
    const int32_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;  // negative: skip; past the pool: never written
    const int64_t block = slot >> 4;
    const int32_t off = slot & (kBlock - 1);
    const int64_t dst = ((block * hkv + head) * kBlock + off) * chunks_per_row + part;
    const u32x4 kk = __builtin_nontemporal_load(k + c);
    const u32x4 vv = __builtin_nontemporal_load(v + c);
    kc[dst] = kk;
    vc[dst] = vv;
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* k, const void* v, const int32_t* slots, void* kc,
                                    void* vc, int32_t ntok, int32_t hkv, int32_t row_bytes,
                                    int64_t num_blocks, hipStream_t st) {
  const int32_t cpr = row_bytes / 16;
  const int64_t total = int64_t(ntok) * hkv * cpr;
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(blocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                     static_cast<u32x4*>(kc), static_cast<u32x4*>(vc), total, hkv, cpr,
                     num_blocks * kBlock);
  return hipGetLastError();
}

}  // namespace pa
