// pa_attention_noalloc: pa_attention with its workspace in a library-owned
// static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Same checks, kernels and results.
//
// The array is `scratch`, one copy per GPU the library runs on, held until the
// process ends.  In host code its name is only a host-side stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.  Every call on
// one GPU shares that GPU's copy: calls that overlap on one GPU (two streams,
// two threads) race on it.  Nothing in it needs to start at zero: the plan
// kernel (or a self-planned decode kernel) writes every header word and work
// counter the later kernels of the same call read.
#include <mutex>
#include <vector>

#include "internal.h"

namespace pa {
namespace {

static __device__ __align__(256) char scratch[PA_NOALLOC_WORKSPACE_MAX];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // device address of `scratch`, per device (nullptr: not looked up yet)

// The current device's copy of `scratch` (nullptr with the error set on failure).
void* scratch_ptr(const char* who) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(PA_ERR_HIP, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (dev >= int(g_scratch_ptr.size())) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", who, dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

void* noalloc_scratch(const char* who) { return scratch_ptr(who); }

}  // namespace pa

using namespace pa;

extern "C" int pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                                    float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_query_len, int32_t dtype,
                                    void* stream) {
  clear_error();
  static const char* who = "pa_attention_noalloc";
  if (int rc = check_attention_args(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale,
                                    out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                                    num_blocks, max_blocks_per_seq, dtype, who))
    return rc;
  if (num_tokens == 0 || num_seqs == 0) return PA_OK;
  StepShape shape{num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq};
  const size_t need = layout_workspace(shape, nullptr).bytes;
  if (need > size_t(PA_NOALLOC_WORKSPACE_MAX))
    return fail(PA_ERR_WORKSPACE, "%s: this step needs %zu bytes of workspace, the static scratch holds %zu", who,
                need, size_t(PA_NOALLOC_WORKSPACE_MAX));
  void* ws = scratch_ptr(who);
  if (!ws) return PA_ERR_HIP;
  return run_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, context_lens, scale, out,
                       num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                       max_query_len, dtype, ws, stream, who);
}
