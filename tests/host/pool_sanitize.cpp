// Host driver for the block pool and the metadata validator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
//
// It calls every host entry point through the C ABI: the worked example of the
// allocation procedure (a 17-token prefill takes ceil(17/16) = 2 blocks, Inside
// vLLM summary, techfeed.io, section "PagedAttentionの仕組み"), all-or-nothing
// exhaustion, shared prefix blocks, the prefix index, the error paths, and
// 20000 seeded random operations, each checked against what it must do, with
// the pool's invariants (free blocks = unreferenced blocks, list entries =
// references) checked throughout.  Exit status 0 means every check held and
// the sanitizers found nothing (they abort the process otherwise).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"

namespace {

int g_checks = 0;

void check(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", line, what, pa_last_error());
    std::exit(1);
  }
}
#define CHECK(x) check((x), #x, __LINE__)

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint32_t rnd(uint32_t n) {  // xorshift64*, uniform enough for choosing operations
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return uint32_t((g_state * 0x2545f4914f6cdd1dull) >> 33) % n;
}

constexpr int kReqs = 40;

// free blocks are exactly the blocks nobody references, and every list entry
// is one reference
void check_invariants(const pa_pool* p, int64_t nb) {
  int64_t zero = 0, refs = 0, listed = 0;
  for (int32_t b = 0; b < nb; ++b) {
    const int32_t r = pa_refcount(p, b);
    CHECK(r >= 0);
    zero += r == 0;
    refs += r;
  }
  for (int64_t q = 0; q < kReqs + 8; ++q) listed += pa_num_req_blocks(p, q);
  CHECK(zero == pa_num_free(p));
  CHECK(refs == listed);
}

void worked_example_and_exhaustion() {
  std::vector<int32_t> order(16);
  for (int i = 0; i < 16; ++i) order[i] = (i * 7 + 3) % 16;  // a permutation
  pa_pool* p = pa_pool_create(16, 16, order.data());
  CHECK(p != nullptr);
  int32_t ids[16], n = -1;
  CHECK(pa_allocate_slots(p, 1, 0, 17, ids, 16, &n) == PA_OK);
  CHECK(n == 2);
  CHECK(ids[0] == order[0] && ids[1] == order[1]);  // taken from the head of the queue
  CHECK(pa_num_free(p) == 14);
  // decode steps: the 18th..32nd token fit in the second block, the 33rd needs a third
  CHECK(pa_allocate_slots(p, 1, 17, 15, ids, 16, &n) == PA_OK && n == 0);
  CHECK(pa_allocate_slots(p, 1, 32, 1, ids, 16, &n) == PA_OK && n == 1 && ids[0] == order[2]);
  // exhaustion: all or nothing, nothing changes
  CHECK(pa_allocate_slots(p, 2, 0, 14 * 16 + 1, ids, 16, &n) == PA_ERR_NO_BLOCKS && n == 0);
  CHECK(pa_num_free(p) == 13 && pa_num_req_blocks(p, 2) == 0);
  // output capacity too small: an error, nothing taken
  CHECK(pa_allocate_slots(p, 3, 0, 64, ids, 2, &n) == PA_ERR_INVALID && pa_num_free(p) == 13);
  // sharing and release: shared blocks stay until the last reference goes
  int32_t row[8];
  CHECK(pa_block_table_row(p, 1, row, 8, -1) == PA_OK);
  CHECK(pa_share_prefix(p, 4, row, 2) == PA_OK);
  CHECK(pa_refcount(p, row[0]) == 2 && pa_refcount(p, row[1]) == 2);
  CHECK(pa_free(p, 1) == PA_OK);
  CHECK(pa_refcount(p, row[0]) == 1 && pa_refcount(p, row[2]) == 0 && pa_num_free(p) == 14);
  CHECK(pa_free(p, 4) == PA_OK && pa_num_free(p) == 16);
  CHECK(pa_free(p, 99) == PA_OK);  // unknown request: no-op
  // released blocks went to the tail, in release order: the queue hands out
  // the untouched blocks first
  CHECK(pa_allocate_slots(p, 5, 0, 13 * 16, nullptr, 0, &n) == PA_OK && n == 13);
  CHECK(pa_allocate_slots(p, 6, 0, 48, ids, 16, &n) == PA_OK && n == 3);
  CHECK(ids[0] == order[2] && ids[1] == order[0] && ids[2] == order[1]);
  // slot mapping: block id * 16 + position % 16; positions past the blocks are errors
  int32_t slots[48];
  CHECK(pa_slot_mapping(p, 6, 0, 48, slots) == PA_OK);
  for (int j = 0; j < 48; ++j) CHECK(slots[j] == ids[j / 16] * 16 + j % 16);
  CHECK(pa_slot_mapping(p, 6, 40, 9, slots) == PA_ERR_INVALID);
  CHECK(pa_block_table_row(p, 6, row, 2, -1) == PA_ERR_INVALID);  // holds 3 > width 2
  check_invariants(p, 16);
  pa_pool_destroy(p);
}

void bad_arguments() {
  int32_t bad[4] = {0, 1, 1, 3};  // not a permutation
  CHECK(pa_pool_create(4, 16, bad) == nullptr);
  CHECK(pa_pool_create(0, 16, nullptr) == nullptr);
  CHECK(pa_pool_create(4, 0, nullptr) == nullptr);
  CHECK(pa_pool_create(int64_t(1) << 28, 16, nullptr) == nullptr);  // slots past int32
  CHECK(pa_allocate_slots(nullptr, 0, 0, 1, nullptr, 0, nullptr) == PA_ERR_INVALID);
  pa_pool* p = pa_pool_create(8, 16, nullptr);
  CHECK(p != nullptr);
  CHECK(pa_allocate_slots(p, 0, -1, 1, nullptr, 0, nullptr) == PA_ERR_INVALID);
  int32_t id = 5;
  CHECK(pa_share_prefix(p, 0, &id, 1) == PA_ERR_INVALID);  // not allocated
  CHECK(pa_share_prefix(p, 0, nullptr, 1) == PA_ERR_INVALID);
  uint64_t key = 7;
  CHECK(pa_prefix_register(p, 0, &key, 1) == PA_ERR_INVALID);  // holds no block
  CHECK(pa_prefix_match(p, 0, nullptr, 1, nullptr) == PA_ERR_INVALID);
  CHECK(pa_block_table_row(p, 0, nullptr, 4, -1) == PA_ERR_INVALID);
  CHECK(pa_slot_mapping(p, 0, -1, 1, &id) == PA_ERR_INVALID);
  CHECK(pa_refcount(p, 8) < 0 && pa_refcount(p, -1) < 0 && pa_num_free(nullptr) < 0);
  pa_pool_destroy(p);
}

void prefix_index() {
  pa_pool* p = pa_pool_create(8, 16, nullptr);
  int32_t n = 0;
  CHECK(pa_allocate_slots(p, 1, 0, 40, nullptr, 0, &n) == PA_OK && n == 3);
  const uint64_t keys[3] = {11, 22, 33};
  CHECK(pa_prefix_register(p, 1, keys, 2) == PA_OK && pa_prefix_cached(p) == 2);
  const uint64_t other[1] = {99};
  CHECK(pa_prefix_register(p, 1, other, 1) == PA_ERR_INVALID);  // block 0 already has key 11
  int32_t hit = -1;
  CHECK(pa_prefix_match(p, 2, keys, 3, &hit) == PA_OK && hit == 2);  // live blocks shared
  CHECK(pa_refcount(p, 0) == 2 && pa_refcount(p, 1) == 2);
  CHECK(pa_prefix_match(p, 2, keys, 1, &hit) == PA_ERR_INVALID);  // already holds blocks
  CHECK(pa_free(p, 1) == PA_OK && pa_free(p, 2) == PA_OK && pa_num_free(p) == 8);
  // released blocks keep their keys until the queue hands them out again
  CHECK(pa_prefix_match(p, 3, keys, 2, &hit) == PA_OK && hit == 2 && pa_num_free(p) == 6);
  CHECK(pa_free(p, 3) == PA_OK);
  CHECK(pa_allocate_slots(p, 4, 0, 128, nullptr, 0, &n) == PA_OK && n == 8);
  CHECK(pa_prefix_cached(p) == 0);  // every block was handed out: no key survives
  CHECK(pa_prefix_match(p, 5, keys, 2, &hit) == PA_OK && hit == 0);
  check_invariants(p, 8);
  pa_pool_destroy(p);
}

void random_operations() {
  const int64_t nb = 64;
  std::vector<int32_t> order(nb);
  for (int64_t i = 0; i < nb; ++i) order[i] = int32_t(i);
  for (int64_t i = nb - 1; i > 0; --i) std::swap(order[i], order[rnd(uint32_t(i + 1))]);
  pa_pool* p = pa_pool_create(nb, 16, order.data());
  CHECK(p != nullptr);
  std::vector<int64_t> tokens(kReqs, 0);
  std::vector<int32_t> buf(nb + 8);
  for (int step = 0; step < 20000; ++step) {
    const int64_t q = rnd(kReqs);
    const int32_t held = pa_num_req_blocks(p, q);
    switch (rnd(7)) {
      case 0:
      case 1: {  // grow by a few tokens; all or nothing when the pool is short
        const int64_t add = 1 + rnd(40), before = pa_num_free(p);
        int32_t n = 0;
        const int rc = pa_allocate_slots(p, q, tokens[q], add, buf.data(), int32_t(buf.size()), &n);
        if (rc == PA_OK) {
          tokens[q] += add;
          CHECK(pa_num_req_blocks(p, q) == held + n);
        } else {
          CHECK(rc == PA_ERR_NO_BLOCKS && pa_num_free(p) == before && pa_num_req_blocks(p, q) == held);
        }
        break;
      }
      case 2: {  // release
        CHECK(pa_free(p, q) == PA_OK);
        tokens[q] = 0;
        break;
      }
      case 3: {  // an empty request shares a leading run of another one's blocks
        const int64_t src = rnd(kReqs);
        const int32_t have = pa_num_req_blocks(p, src);
        if (held == 0 && src != q && have > 0) {
          CHECK(pa_block_table_row(p, src, buf.data(), int32_t(buf.size()), -1) == PA_OK);
          const int32_t k = 1 + int32_t(rnd(uint32_t(have)));
          CHECK(pa_share_prefix(p, q, buf.data(), k) == PA_OK);
          tokens[q] = int64_t(k) * 16;
        }
        break;
      }
      case 4: {  // register leading blocks under keys from a small space (collisions happen)
        if (held > 0) {
          const int32_t k = 1 + int32_t(rnd(uint32_t(held)));
          std::vector<uint64_t> keys(k);
          for (int32_t i = 0; i < k; ++i) keys[i] = 1000 + rnd(12);
          const int rc = pa_prefix_register(p, q, keys.data(), k);
          CHECK(rc == PA_OK || rc == PA_ERR_INVALID);
        }
        break;
      }
      case 5: {  // an empty request looks its prompt up in the index
        if (held == 0) {
          std::vector<uint64_t> keys(1 + rnd(4));
          for (auto& key : keys) key = 1000 + rnd(12);
          int32_t hit = -1;
          CHECK(pa_prefix_match(p, q, keys.data(), int32_t(keys.size()), &hit) == PA_OK);
          CHECK(hit >= 0 && hit <= int32_t(keys.size()) && pa_num_req_blocks(p, q) == hit);
          tokens[q] = int64_t(hit) * 16;
        }
        break;
      }
      default: {  // tables and slots of what the request holds
        const int32_t w = held + int32_t(rnd(3));
        CHECK(pa_block_table_row(p, q, buf.data(), w, -7) == PA_OK);
        for (int32_t i = held; i < w; ++i) CHECK(buf[i] == -7);
        for (int32_t i = 0; i < held; ++i) CHECK(pa_refcount(p, buf[i]) >= 1);
        if (held > 0) {
          std::vector<int32_t> slots(size_t(held) * 16);
          CHECK(pa_slot_mapping(p, q, 0, held * 16, slots.data()) == PA_OK);
          for (int32_t j = 0; j < held * 16; ++j) CHECK(slots[j] == buf[j / 16] * 16 + j % 16);
        }
        CHECK(pa_block_table_row(p, q, buf.data(), held - 1, 0) == PA_ERR_INVALID);  // too narrow
      }
    }
    if (step % 97 == 0) check_invariants(p, nb);
  }
  check_invariants(p, nb);
  pa_pool_destroy(p);
}

void validator() {
  // two sequences: a 17-token prefill over nothing cached, and a decode over 33 cached tokens
  pa_pool* p = pa_pool_create(16, 16, nullptr);
  int32_t n = 0;
  CHECK(pa_allocate_slots(p, 0, 0, 17, nullptr, 0, &n) == PA_OK);
  CHECK(pa_allocate_slots(p, 1, 0, 34, nullptr, 0, &n) == PA_OK);
  const int32_t S = 2, T = 18, W = 4;
  std::vector<int32_t> bt(S * W), slots(T);
  CHECK(pa_block_table_row(p, 0, bt.data(), W, -1) == PA_OK);
  CHECK(pa_block_table_row(p, 1, bt.data() + W, W, -1) == PA_OK);
  CHECK(pa_slot_mapping(p, 0, 0, 17, slots.data()) == PA_OK);
  CHECK(pa_slot_mapping(p, 1, 33, 1, slots.data() + 17) == PA_OK);
  int32_t seq_lens[2] = {17, 34}, qsl[3] = {0, 17, 18}, ctx[2] = {0, 33};
  auto v = [&](const int32_t* s) {
    return pa_validate_metadata(bt.data(), seq_lens, qsl, ctx, s, S, T, W, 16, 16);
  };
  CHECK(v(slots.data()) == PA_OK);
  CHECK(v(nullptr) == PA_OK);
  bt[1] = 16;  // a used block id past the pool
  CHECK(v(slots.data()) == PA_ERR_INVALID);
  CHECK(pa_block_table_row(p, 0, bt.data(), W, -1) == PA_OK);
  bt[2] = 99;  // padding past the sequence's two blocks: never read, so not checked
  CHECK(v(slots.data()) == PA_OK);
  CHECK(pa_block_table_row(p, 0, bt.data(), W, -1) == PA_OK);
  slots[3] = slots[4];  // duplicate slot
  CHECK(v(slots.data()) == PA_ERR_INVALID);
  CHECK(pa_slot_mapping(p, 0, 0, 17, slots.data()) == PA_OK);
  seq_lens[1] = 35;  // seq_lens != context + query rows
  CHECK(v(slots.data()) == PA_ERR_INVALID);
  seq_lens[1] = 34;
  qsl[1] = 19;  // query_start_loc not non-decreasing
  CHECK(v(slots.data()) == PA_ERR_INVALID);
  qsl[1] = 17;
  CHECK(pa_validate_metadata(bt.data(), seq_lens, qsl, ctx, slots.data(), S, T, 2, 16, 16) ==
        PA_ERR_INVALID);  // 34 tokens need 3 blocks > 2 per row
  CHECK(v(slots.data()) == PA_OK);
  pa_pool_destroy(p);
}

}  // namespace

int main() {
  worked_example_and_exhaustion();
  bad_arguments();
  prefix_index();
  validator();
  random_operations();
  std::printf("host pool and validator: %d checks passed\n", g_checks);
  return 0;
}
