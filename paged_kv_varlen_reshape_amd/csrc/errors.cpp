// pa_last_error / pa_set_option / pa_get_option.
#include "errors.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace pa {
namespace {
thread_local std::string g_error;
std::atomic<int64_t> g_force_rowwise{0};
std::atomic<int64_t> g_split_tokens{0};
std::atomic<int64_t> g_target_items{0};
std::atomic<int64_t> g_decode_buffers{0};
std::atomic<int64_t> g_decode_kernel{0};
std::atomic<int64_t> g_verify_rows{0};
std::atomic<int64_t> g_chunk_kernel{0};
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

int64_t option(int32_t id) {
  switch (id) {
    case PA_OPT_FORCE_ROWWISE: return g_force_rowwise.load();
    case PA_OPT_SPLIT_TOKENS: return g_split_tokens.load();
    case PA_OPT_TARGET_ITEMS: return g_target_items.load();
    case PA_OPT_DECODE_BUFFERS: return g_decode_buffers.load();
    case PA_OPT_DECODE_KERNEL: return g_decode_kernel.load();
    case PA_OPT_VERIFY_ROWS: return g_verify_rows.load();
    case PA_OPT_CHUNK_KERNEL: return g_chunk_kernel.load();
    default: return -1;
  }
}
}  // namespace pa

extern "C" const char* pa_last_error(void) { return pa::g_error.c_str(); }

extern "C" int pa_set_option(int32_t id, int64_t value) {
  switch (id) {
    case PA_OPT_FORCE_ROWWISE:
      if (value != 0 && value != 1) return pa::fail(PA_ERR_INVALID, "PA_OPT_FORCE_ROWWISE takes 0 or 1");
      pa::g_force_rowwise = value;
      return PA_OK;
    case PA_OPT_SPLIT_TOKENS:
      if (value < 0 || value % 16 != 0 || value > (1 << 24))
        return pa::fail(PA_ERR_INVALID, "PA_OPT_SPLIT_TOKENS must be 0 or a positive multiple of 16");
      pa::g_split_tokens = value;
      return PA_OK;
    case PA_OPT_TARGET_ITEMS:
      if (value < 0 || value > (1 << 24)) return pa::fail(PA_ERR_INVALID, "PA_OPT_TARGET_ITEMS out of range");
      pa::g_target_items = value;
      return PA_OK;
    case PA_OPT_DECODE_BUFFERS:
      if (value < 0 || value > 4) return pa::fail(PA_ERR_INVALID, "PA_OPT_DECODE_BUFFERS takes 0..4");
      pa::g_decode_buffers = value;
      return PA_OK;
    case PA_OPT_DECODE_KERNEL:
      if (value < 0 || value > 2) return pa::fail(PA_ERR_INVALID, "PA_OPT_DECODE_KERNEL takes 0, 1 or 2");
      pa::g_decode_kernel = value;
      return PA_OK;
    case PA_OPT_VERIFY_ROWS:
      if (value < 0 || value > 16) return pa::fail(PA_ERR_INVALID, "PA_OPT_VERIFY_ROWS takes 0..16");
      pa::g_verify_rows = value;
      return PA_OK;
    case PA_OPT_CHUNK_KERNEL:
      if (value < 0 || value > 2) return pa::fail(PA_ERR_INVALID, "PA_OPT_CHUNK_KERNEL takes 0, 1 or 2");
      pa::g_chunk_kernel = value;
      return PA_OK;
    default:
      return pa::fail(PA_ERR_INVALID, "unknown option %d", id);
  }
}

extern "C" int64_t pa_get_option(int32_t id) { return pa::option(id); }
