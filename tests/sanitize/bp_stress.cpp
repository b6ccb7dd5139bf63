// Drives every entry point of the host block pool (include/pa_blocks.h)
// through seeded random operation sequences, with the pool's own invariants
// checked after every step.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py; any out-of-bounds
// access, use after free or undefined behaviour aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa_blocks.h"

#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::abort();                                                      \
    }                                                                    \
  } while (0)

namespace {

// Free queue length must equal the number of blocks nobody holds, and every
// live request's table entries must be held (or -1 after a window release).
void invariants(pa_block_pool* p, int32_t nb, const std::map<int64_t, int32_t>& live) {
  std::vector<int32_t> q((size_t)nb);
  const int32_t nq = pa_bp_free_queue(p, q.data(), nb);
  CHECK(nq == pa_bp_num_free(p));
  int32_t zero = 0;
  for (int32_t b = 0; b < nb; ++b) zero += pa_bp_ref_count(p, b) == 0;
  CHECK(zero == nq);
  for (int32_t i = 0; i < nq; ++i) CHECK(pa_bp_ref_count(p, q[(size_t)i]) == 0);
  for (const auto& kv : live) {
    std::vector<int32_t> row(4096);
    const int32_t n = pa_bp_request_blocks(p, kv.first, row.data(), 4096);
    CHECK(n >= 0);
    for (int32_t j = 0; j < n && j < 4096; ++j)
      CHECK(row[(size_t)j] == -1 || pa_bp_ref_count(p, row[(size_t)j]) > 0);
  }
}

void run(uint32_t seed, int32_t nb, int32_t bs) {
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return (int)(rng() % (uint32_t)(hi - lo + 1)) + lo; };
  pa_block_pool* p = pa_bp_create(nb, bs);
  CHECK(p);
  std::vector<std::vector<int32_t>> prompts;
  for (int i = 0; i < 6; ++i) {
    std::vector<int32_t> t((size_t)uni(1, 6 * bs));
    for (auto& x : t) x = uni(0, 50000);
    prompts.push_back(t);
  }
  std::map<int64_t, int32_t> live;                      // request -> tokens held
  std::map<int64_t, std::vector<int32_t>> toks;
  const char extra[] = "tenant";
  for (int step = 0; step < 3000; ++step) {
    const int op = uni(0, 11);
    const int64_t any = live.empty() ? -1 : std::next(live.begin(), uni(0, (int)live.size() - 1))->first;
    if (op <= 1) {                                      // new request from a prompt
      std::vector<int32_t> t = prompts[(size_t)uni(0, 5)];
      for (int i = uni(0, bs); i > 0; --i) t.push_back(uni(0, 50000));
      int32_t cached = -1;
      const int st = pa_bp_allocate_request(p, step, t.data(), (int32_t)t.size(),
                                            op ? extra : nullptr, op ? 6 : 0, &cached);
      CHECK(st == 0 || st == PA_ERR_NO_BLOCKS);
      if (st == 0) {
        CHECK(cached % bs == 0 && cached < (int32_t)t.size());
        live[step] = (int32_t)t.size();
        toks[step] = t;
      }
    } else if (op == 2 && any >= 0) {                   // K/V written: cache
      CHECK(pa_bp_cache_request(p, any, toks[any].data(), (int32_t)toks[any].size(), nullptr, 0) == 0);
    } else if (op == 3 && any >= 0) {                   // growth
      const int32_t n = live[any] + uni(1, 2 * bs);
      const int st = pa_bp_append_slots(p, any, n);
      CHECK(st == 0 || st == PA_ERR_NO_BLOCKS);
      if (st == 0) {
        while ((int32_t)toks[any].size() < n) toks[any].push_back(uni(0, 50000));
        live[any] = n;
      }
    } else if (op == 4 && any >= 0) {                   // finished
      CHECK(pa_bp_free_request(p, any) == 0);
      live.erase(any);
      toks.erase(any);
    } else if (op == 5 && any >= 0) {                   // sliding-window release
      CHECK(pa_bp_remove_skipped_blocks(p, any, live[any], uni(1, 3 * bs)) >= 0);
    } else if (op == 6 && any >= 0) {                   // fork
      const int64_t child = 1000000 + step;
      CHECK(pa_bp_fork_request(p, any, child) == 0);
      live[child] = live[any];
      toks[child] = toks[any];
    } else if (op == 7 && any >= 0) {                   // copy-on-write before a write
      int64_t pair[2] = {-1, -1};
      const int32_t pos = uni(0, live[any] - 1);
      const int st = pa_bp_prepare_write(p, any, pos, pair);
      CHECK(st == 0 || st == 1 || st == PA_ERR_NO_BLOCKS || st == PA_ERR_INVALID_ARG);
      if (st == 1) CHECK(pair[0] >= 0 && pair[1] >= 0 && pair[0] != pair[1]);
    } else if (op == 8 && !live.empty()) {              // one batched step
      std::vector<int64_t> ids;
      std::vector<int32_t> after;
      for (const auto& kv : live)
        if (uni(0, 1)) { ids.push_back(kv.first); after.push_back(kv.second + uni(0, bs)); }
      const int st = pa_bp_append_slots_batch(p, ids.data(), after.data(), (int32_t)ids.size());
      CHECK(st == 0 || st == PA_ERR_NO_BLOCKS);
      if (st == 0)
        for (size_t i = 0; i < ids.size(); ++i) {
          live[ids[i]] = after[i];
          while ((int32_t)toks[ids[i]].size() < after[i]) toks[ids[i]].push_back(uni(0, 50000));
        }
    } else if (op == 9) {                               // block-level calls
      int32_t got[4];
      const int n = uni(0, 4);
      if (pa_bp_get_new_blocks(p, n, got) == 0) {
        std::vector<int32_t> back(got, got + n);
        CHECK(pa_bp_touch(p, back.data(), n) == 0);
        std::vector<int32_t> twice;
        for (int32_t b : back) { twice.push_back(b); twice.push_back(b); }
        pa_block_hash h;
        for (int32_t b : back) {
          pa_hash_block_tokens(nullptr, &b, 1, nullptr, 0, &h);
          CHECK(pa_bp_cache_block(p, b, &h) == 0);
        }
        CHECK(pa_bp_free_blocks(p, twice.data(), (int32_t)twice.size()) == 0);
      }
      CHECK(pa_bp_touch(p, got, -1) < 0);
      const int32_t bad = nb;
      CHECK(pa_bp_free_blocks(p, &bad, 1) < 0);
      CHECK(pa_bp_ref_count(p, -1) < 0 && pa_bp_block_hash(p, nb, nullptr) < 0);
    } else {                                            // lookups and hashing
      const auto& t = prompts[(size_t)uni(0, 5)];
      std::vector<pa_block_hash> hs(t.size() / (size_t)bs + 1);
      const int32_t full = pa_hash_blocks(t.data(), (int32_t)t.size(), bs, extra, 6, hs.data(),
                                          (int32_t)hs.size());
      CHECK(full == (int32_t)t.size() / bs);
      std::vector<int32_t> out(hs.size());
      CHECK(pa_bp_lookup(p, hs.data(), full, out.data()) >= 0);
    }
    invariants(p, nb, live);
  }
  for (const auto& kv : live) CHECK(pa_bp_free_request(p, kv.first) == 0);
  CHECK(pa_bp_num_free(p) == nb);
  pa_bp_destroy(p);
}

}  // namespace

int main() {
  for (uint32_t seed = 1; seed <= 8; ++seed) run(seed, 16 + 8 * (int32_t)seed, 1 + (int32_t)seed % 5 * 3);
  CHECK(pa_bp_create(0, 16) == nullptr);
  std::printf("bp_stress ok\n");
  return 0;
}
