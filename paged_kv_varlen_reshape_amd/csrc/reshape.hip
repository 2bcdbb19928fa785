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

// Thread c moves chunk c & (cpr-1) of source row c >> cpr_log2, where a source
// row is one (token, kv head) pair; cpr (16-byte chunks per row) is 8, 16 or 32.
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                         const int32_t* __restrict__ slots, u32x4* __restrict__ kc,
                         u32x4* __restrict__ vc, uint32_t total_chunks, uint32_t hkv,
                         uint32_t cpr_log2, int64_t num_slots) {
  const uint32_t stride = gridDim.x * blockDim.x;
  const uint32_t cpr_mask = (1u << cpr_log2) - 1;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
    const uint32_t row = c >> cpr_log2;  // token * hkv + head
    const uint32_t part = c & cpr_mask;
    const uint32_t tok = row / hkv;
    const uint32_t head = row - tok * hkv;
    const int32_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;  // negative: skip; past the pool: never written
    const int64_t block = slot >> 4;
    const int32_t off = slot & (kBlock - 1);
    const int64_t dst = (((block * hkv + head) * kBlock + off) << cpr_log2) + part;
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
  const uint32_t cpr = uint32_t(row_bytes / 16);
  const uint32_t cpr_log2 = uint32_t(__builtin_ctz(cpr));
  const int64_t total = int64_t(ntok) * hkv * cpr;  // < 2^31, checked by the caller
  const int64_t want = (total + 255) / 256;
  const int blocks = int(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(blocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                     static_cast<u32x4*>(kc), static_cast<u32x4*>(vc), uint32_t(total), uint32_t(hkv),
                     cpr_log2, num_blocks * kBlock);
  return hipGetLastError();
}

}  // namespace pa
