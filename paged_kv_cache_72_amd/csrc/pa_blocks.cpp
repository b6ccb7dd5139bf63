// pa_blocks.cpp -- the host block pool with prefix caching (declared in
// include/pa_blocks.h).  Host code only; it produces the block tables, slot
// numbers and copy pairs that the device calls consume.
//
// What it implements (the pages' rules):
//   * all blocks with reference count 0 -- never used, or freed but still
//     carrying the hash of a cached block -- sit in one doubly linked free
//     queue; blocks are handed out from the head ("KV Cache memory core",
//     section 2.3, BlockPool sketch and the six-block walkthrough);
//   * handing out a block that still carries a hash drops it from the hash
//     index: eviction is a side effect of allocation, with no separate pass
//     (same passage; "vLLM intro part 2", section 6.3 step 3);
//   * a block whose count reaches 0 goes to the tail if it carries a hash and
//     to the head if not; a request frees its blocks last to first (same
//     passages);
//   * a prefix hit on a free block unlinks it from the middle of the queue in
//     O(1) -- the reason the queue is a doubly linked list ("vLLM intro part 2",
//     section 6.2);
//   * block hashes are chained, h_i = SHA-256(h_{i-1} | tokens | extra keys),
//     and only full blocks are hashed; lookup walks the chain from the first
//     block and stops at the first miss ("vLLM intro part 2", section 6.1;
//     "KV Cache memory core", section 4.1);
//   * forked sequences share blocks by count, and a write into a block whose
//     own count is above 1 first moves the writer to a copy ("GPU memory & KV
//     cache", copy-on-write steps).
// Open points of the pages are settled as follows: NONE_HASH is 32 zero bytes;
// the hash input is the parent's 32 bytes, then the token ids as little-endian
// int32, then the extra-key bytes; unhashed blocks freed in one call are
// prepended one after another; a request's lookup never covers its last token,
// so at most (n - 1) / block_size blocks hit; among blocks with equal hashes
// the one cached first is returned.
//
// SHA-256 follows FIPS 180-4; its constants are the fractional parts of the
// square and cube roots of the first primes, computed here at start-up.
#include <cpuid.h>
#include <immintrin.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_blocks.h"

namespace {

// ------------------------------------------------------------------ SHA-256

struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Consts() {
    int primes[64], np = 0;
    for (int c = 2; np < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d)
        if (c % d == 0) { prime = false; break; }
      if (prime) primes[np++] = c;
    }
    for (int i = 0; i < 64; ++i) {
      long double r = cbrtl((long double)primes[i]);
      k[i] = (uint32_t)(uint64_t)std::floor((r - std::floor(r)) * 4294967296.0L);
    }
    for (int i = 0; i < 8; ++i) {
      long double r = sqrtl((long double)primes[i]);
      h0[i] = (uint32_t)(uint64_t)std::floor((r - std::floor(r)) * 4294967296.0L);
    }
  }
};

const Sha256Consts& sha_consts() {
  static const Sha256Consts c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// One compression of a 64-byte block into state h (FIPS 180-4, section 6.2.2).
void compress_portable(uint32_t h[8], const uint8_t* m) {
  const uint32_t* K = sha_consts().k;
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)m[4 * t] << 24 | (uint32_t)m[4 * t + 1] << 16 |
           (uint32_t)m[4 * t + 2] << 8 | (uint32_t)m[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = w[t - 16] + s0 + w[t - 7] + s1;
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + K[t] + w[t];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + mj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d;
  h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

// The same compression with the x86 SHA extensions (SHA256RNDS2 does two
// rounds on the state split as (a, b, e, f) and (c, d, g, h); SHA256MSG1 and
// SHA256MSG2 extend the message schedule four words at a time).
__attribute__((target("sha,sse4.1,ssse3"))) void compress_x86(uint32_t h[8],
                                                              const uint8_t* m) {
  const uint32_t* K = sha_consts().k;
  const __m128i bswap = _mm_set_epi64x(0x0c0d0e0f08090a0bULL, 0x0405060700010203ULL);
  __m128i tmp = _mm_shuffle_epi32(_mm_loadu_si128((const __m128i*)&h[0]), 0xB1);   // c d a b
  __m128i st1 = _mm_shuffle_epi32(_mm_loadu_si128((const __m128i*)&h[4]), 0x1B);   // h g f e
  __m128i st0 = _mm_alignr_epi8(tmp, st1, 8);                                       // a b e f
  st1 = _mm_blend_epi16(st1, tmp, 0xF0);                                            // c d g h
  const __m128i save0 = st0, save1 = st1;
  __m128i w[4];
  for (int j = 0; j < 4; ++j)
    w[j] = _mm_shuffle_epi8(_mm_loadu_si128((const __m128i*)(m + 16 * j)), bswap);
  for (int j = 0; j < 16; ++j) {
    __m128i& wj = w[j & 3];                   // words 4j .. 4j + 3
    if (j >= 4) {
      // W[t] = W[t-16] + s0(W[t-15]) + W[t-7] + s1(W[t-2]) for four t at once
      const __m128i prev = w[(j + 3) & 3], prev2 = w[(j + 2) & 3];
      wj = _mm_sha256msg2_epu32(
          _mm_add_epi32(_mm_sha256msg1_epu32(wj, w[(j + 1) & 3]), _mm_alignr_epi8(prev, prev2, 4)),
          prev);
    }
    __m128i msg = _mm_add_epi32(wj, _mm_loadu_si128((const __m128i*)&K[4 * j]));
    st1 = _mm_sha256rnds2_epu32(st1, st0, msg);
    msg = _mm_shuffle_epi32(msg, 0x0E);
    st0 = _mm_sha256rnds2_epu32(st0, st1, msg);
  }
  st0 = _mm_add_epi32(st0, save0);
  st1 = _mm_add_epi32(st1, save1);
  tmp = _mm_shuffle_epi32(st0, 0x1B);                                               // f e b a
  st1 = _mm_shuffle_epi32(st1, 0xB1);                                               // d c h g
  _mm_storeu_si128((__m128i*)&h[0], _mm_blend_epi16(tmp, st1, 0xF0));               // a b c d
  _mm_storeu_si128((__m128i*)&h[4], _mm_alignr_epi8(st1, tmp, 8));                  // e f g h
}

// The x86 path when the CPU has the SHA extensions, unless PA_SHA256_PORTABLE
// is set in the environment (to exercise the portable path).
bool use_x86_sha() {
  static const bool on = [] {
    const char* env = std::getenv("PA_SHA256_PORTABLE");
    if (env && *env && *env != '0') return false;
    unsigned a, b, c, d;
    return __get_cpuid_count(7, 0, &a, &b, &c, &d) && ((b >> 29) & 1u);
  }();
  return on;
}

// SHA-256 of a message already assembled in memory (padding appended here).
void sha256(const uint8_t* msg, size_t n, uint8_t out[32]) {
  uint32_t h[8];
  std::memcpy(h, sha_consts().h0, sizeof h);
  void (*compress)(uint32_t*, const uint8_t*) = use_x86_sha() ? compress_x86 : compress_portable;
  size_t full = n / 64;
  for (size_t i = 0; i < full; ++i) compress(h, msg + 64 * i);
  uint8_t tail[128] = {0};
  const size_t rem = n - 64 * full;
  std::memcpy(tail, msg + 64 * full, rem);
  tail[rem] = 0x80;
  const size_t tl = rem + 1 + 8 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)n * 8;
  for (int i = 0; i < 8; ++i) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  compress(h, tail);
  if (tl == 128) compress(h, tail + 64);
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

// h = SHA-256(parent or 32 zero bytes | tokens as int32 little-endian | extra)
void hash_block(const pa_block_hash* parent, const int32_t* tokens, int32_t n,
                const void* extra, int32_t extra_len, pa_block_hash* out) {
  const size_t len = 32 + 4 * (size_t)n + (extra && extra_len > 0 ? (size_t)extra_len : 0);
  uint8_t small[512];
  std::vector<uint8_t> big;
  uint8_t* m = small;
  if (len > sizeof small) {
    big.resize(len);
    m = big.data();
  }
  if (parent) std::memcpy(m, parent->bytes, 32);
  else std::memset(m, 0, 32);
  uint8_t* p = m + 32;
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t v = (uint32_t)tokens[i];
    p[4 * i] = (uint8_t)v;
    p[4 * i + 1] = (uint8_t)(v >> 8);
    p[4 * i + 2] = (uint8_t)(v >> 16);
    p[4 * i + 3] = (uint8_t)(v >> 24);
  }
  if (extra && extra_len > 0) std::memcpy(p + 4 * (size_t)n, extra, (size_t)extra_len);
  sha256(m, len, out->bytes);
}

struct HashKey {
  uint8_t b[32];
  bool operator==(const HashKey& o) const { return std::memcmp(b, o.b, 32) == 0; }
};
struct HashKeyHash {
  size_t operator()(const HashKey& k) const {
    size_t v;
    std::memcpy(&v, k.b, sizeof v);     // already uniformly distributed
    return v;
  }
};

thread_local std::string g_err;
int fail(int code, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace

struct pa_block_pool {
  int32_t block_size;
  std::vector<int32_t> ref;
  std::vector<int32_t> prev, next;          // free queue links; -1 = none
  std::vector<uint8_t> in_queue;
  std::vector<uint8_t> hashed;
  std::vector<HashKey> hash;
  int32_t head = -1, tail = -1, nfree = 0;
  // hash -> blocks carrying it, in caching order
  std::unordered_map<HashKey, std::vector<int32_t>, HashKeyHash> index;
  std::unordered_map<int64_t, std::vector<int32_t>> requests;

  bool valid(int32_t b) const { return b >= 0 && b < (int32_t)ref.size(); }

  void unlink(int32_t b) {
    const int32_t p = prev[b], n = next[b];
    if (p >= 0) next[p] = n; else head = n;
    if (n >= 0) prev[n] = p; else tail = p;
    prev[b] = next[b] = -1;
    in_queue[b] = 0;
    --nfree;
  }
  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_queue[b] = 1;
    ++nfree;
  }
  void push_head(int32_t b) {
    next[b] = head;
    prev[b] = -1;
    if (head >= 0) prev[head] = b; else tail = b;
    head = b;
    in_queue[b] = 1;
    ++nfree;
  }
  void evict(int32_t b) {
    if (!hashed[b]) return;
    auto it = index.find(hash[b]);
    if (it != index.end()) {
      auto& v = it->second;
      for (size_t i = 0; i < v.size(); ++i)
        if (v[i] == b) { v.erase(v.begin() + (long)i); break; }
      if (v.empty()) index.erase(it);
    }
    hashed[b] = 0;
  }
  void take(int32_t n, int32_t* out) {
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = head;
      unlink(b);
      evict(b);
      ++ref[b];
      out[i] = b;
    }
  }
  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (hashed[b]) push_tail(b); else push_head(b);
    }
  }
  void hold(int32_t b) {
    if (ref[b] == 0) unlink(b);
    ++ref[b];
  }
  void cache(int32_t b, const HashKey& k) {
    if (hashed[b]) return;
    hashed[b] = 1;
    hash[b] = k;
    index[k].push_back(b);
  }
  int32_t lookup(const pa_block_hash* hashes, int32_t n, int32_t* out) const {
    int32_t hits = 0;
    for (; hits < n; ++hits) {
      HashKey k;
      std::memcpy(k.b, hashes[hits].bytes, 32);
      auto it = index.find(k);
      if (it == index.end() || it->second.empty()) break;
      if (out) out[hits] = it->second.front();
    }
    return hits;
  }
};

namespace {

std::vector<pa_block_hash> chain(const int32_t* tokens, int32_t n, int32_t bs, const void* extra,
                                 int32_t extra_len) {
  std::vector<pa_block_hash> h((size_t)(n / bs));
  for (int32_t i = 0; i < n / bs; ++i)
    hash_block(i ? &h[(size_t)i - 1] : nullptr, tokens + (int64_t)i * bs, bs, extra, extra_len,
               &h[(size_t)i]);
  return h;
}

int check_ids(const pa_block_pool* p, const int32_t* ids, int32_t n) {
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "count %d < 0", n);
  if (n && !ids) return fail(PA_ERR_INVALID_ARG, "block id array is NULL");
  for (int32_t i = 0; i < n; ++i)
    if (!p->valid(ids[i])) return fail(PA_ERR_INVALID_ARG, "block id %d out of range", ids[i]);
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_bp_last_error(void) { return g_err.c_str(); }

pa_block_pool* pa_bp_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) {
    fail(PA_ERR_INVALID_ARG, "num_blocks %d and block_size %d must be >= 1", num_blocks,
         block_size);
    return nullptr;
  }
  pa_block_pool* p = new pa_block_pool;
  p->block_size = block_size;
  p->ref.assign((size_t)num_blocks, 0);
  p->prev.assign((size_t)num_blocks, -1);
  p->next.assign((size_t)num_blocks, -1);
  p->in_queue.assign((size_t)num_blocks, 0);
  p->hashed.assign((size_t)num_blocks, 0);
  p->hash.resize((size_t)num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) p->push_tail(b);
  return p;
}

void pa_bp_destroy(pa_block_pool* p) { delete p; }

int32_t pa_bp_num_free(const pa_block_pool* p) { return p ? p->nfree : 0; }

int32_t pa_bp_ref_count(const pa_block_pool* p, int32_t block) {
  if (!p || !p->valid(block)) return fail(PA_ERR_INVALID_ARG, "bad pool or block %d", block);
  return p->ref[(size_t)block];
}

int pa_bp_block_hash(const pa_block_pool* p, int32_t block, pa_block_hash* out) {
  if (!p || !p->valid(block)) return fail(PA_ERR_INVALID_ARG, "bad pool or block %d", block);
  if (!p->hashed[(size_t)block]) return 0;
  if (out) std::memcpy(out->bytes, p->hash[(size_t)block].b, 32);
  return 1;
}

int32_t pa_bp_free_queue(const pa_block_pool* p, int32_t* out, int32_t cap) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  int32_t n = 0;
  for (int32_t b = p->head; b >= 0; b = p->next[(size_t)b], ++n)
    if (out && n < cap) out[n] = b;
  return n;
}

int pa_bp_get_new_blocks(pa_block_pool* p, int32_t n, int32_t* out) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || (n && !out)) return fail(PA_ERR_INVALID_ARG, "bad count %d or output", n);
  if (n > p->nfree)
    return fail(PA_ERR_NO_BLOCKS, "%d blocks requested, %d free", n, p->nfree);
  p->take(n, out);
  return PA_OK;
}

int pa_bp_free_blocks(pa_block_pool* p, const int32_t* ids, int32_t n) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (int st = check_ids(p, ids, n)) return st;
  // every id must be held as often as it is listed
  std::unordered_map<int32_t, int32_t> cnt;
  for (int32_t i = 0; i < n; ++i)
    if (++cnt[ids[i]] > p->ref[(size_t)ids[i]])
      return fail(PA_ERR_INVALID_ARG, "block %d freed more often than held", ids[i]);
  for (int32_t i = 0; i < n; ++i) p->release(ids[i]);
  return PA_OK;
}

int pa_bp_touch(pa_block_pool* p, const int32_t* ids, int32_t n) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (int st = check_ids(p, ids, n)) return st;
  for (int32_t i = 0; i < n; ++i) p->hold(ids[i]);
  return PA_OK;
}

int pa_bp_cache_block(pa_block_pool* p, int32_t block, const pa_block_hash* h) {
  if (!p || !h || !p->valid(block)) return fail(PA_ERR_INVALID_ARG, "bad pool, hash or block");
  if (p->ref[(size_t)block] == 0)
    return fail(PA_ERR_INVALID_ARG, "block %d is not held", block);
  HashKey k;
  std::memcpy(k.b, h->bytes, 32);
  p->cache(block, k);
  return PA_OK;
}

int32_t pa_bp_lookup(const pa_block_pool* p, const pa_block_hash* hashes, int32_t n,
                     int32_t* out) {
  if (!p || n < 0 || (n && !hashes)) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  return p->lookup(hashes, n, out);
}

void pa_hash_block_tokens(const pa_block_hash* parent, const int32_t* tokens, int32_t n,
                          const void* extra, int32_t extra_len, pa_block_hash* out) {
  if (!out) return;
  hash_block(parent, tokens, n < 0 ? 0 : n, extra, extra_len, out);
}

int pa_bp_allocate_request(pa_block_pool* p, int64_t rid, const int32_t* tokens, int32_t n,
                           const void* extra, int32_t extra_len, int32_t* num_cached_tokens) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || (n && !tokens)) return fail(PA_ERR_INVALID_ARG, "bad token array");
  if (p->requests.count(rid)) return fail(PA_ERR_INVALID_ARG, "request %lld exists", (long long)rid);
  const int32_t bs = p->block_size;
  const std::vector<pa_block_hash> h = chain(tokens, n, bs, extra, extra_len);
  const int32_t usable = n > 0 ? (n - 1) / bs : 0;
  std::vector<int32_t> hits((size_t)usable);
  const int32_t nh = p->lookup(h.data(), usable, hits.data());
  hits.resize((size_t)nh);
  const int32_t need = (n + bs - 1) / bs - nh;
  int32_t hit_free = 0;
  for (int32_t b : hits) hit_free += p->ref[(size_t)b] == 0;
  if (need > p->nfree - hit_free)
    return fail(PA_ERR_NO_BLOCKS, "%d new blocks needed, %d free", need, p->nfree - hit_free);
  for (int32_t b : hits) p->hold(b);
  std::vector<int32_t> blocks = hits;
  blocks.resize((size_t)(nh + need));
  p->take(need, blocks.data() + nh);
  p->requests[rid] = std::move(blocks);
  if (num_cached_tokens) *num_cached_tokens = nh * bs;
  return PA_OK;
}

int pa_bp_cache_request(pa_block_pool* p, int64_t rid, const int32_t* tokens, int32_t n,
                        const void* extra, int32_t extra_len) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  if (n < 0 || (n && !tokens)) return fail(PA_ERR_INVALID_ARG, "bad token array");
  const std::vector<pa_block_hash> h = chain(tokens, n, p->block_size, extra, extra_len);
  const size_t m = std::min(h.size(), it->second.size());
  for (size_t i = 0; i < m; ++i) {
    if (it->second[i] < 0) continue;           // released by the sliding window
    HashKey k;
    std::memcpy(k.b, h[i].bytes, 32);
    p->cache(it->second[i], k);
  }
  return PA_OK;
}

int pa_bp_append_slots(pa_block_pool* p, int64_t rid, int32_t num_tokens_after) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  if (num_tokens_after < 0) return fail(PA_ERR_INVALID_ARG, "negative token count");
  const int32_t need =
      (num_tokens_after + p->block_size - 1) / p->block_size - (int32_t)it->second.size();
  if (need <= 0) return PA_OK;
  if (need > p->nfree) return fail(PA_ERR_NO_BLOCKS, "%d blocks needed, %d free", need, p->nfree);
  const size_t old = it->second.size();
  it->second.resize(old + (size_t)need);
  p->take(need, it->second.data() + old);
  return PA_OK;
}

int pa_bp_append_slots_batch(pa_block_pool* p, const int64_t* requests,
                             const int32_t* num_tokens_after, int32_t n) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || (n && (!requests || !num_tokens_after)))
    return fail(PA_ERR_INVALID_ARG, "bad request arrays");
  // validate everything and count the blocks first: a failed call changes nothing
  std::vector<std::vector<int32_t>*> rows((size_t)n);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->requests.find(requests[i]);
    if (it == p->requests.end())
      return fail(PA_ERR_INVALID_ARG, "no request %lld (entry %d)", (long long)requests[i], i);
    if (num_tokens_after[i] < 0) return fail(PA_ERR_INVALID_ARG, "negative token count (entry %d)", i);
    for (int32_t j = 0; j < i; ++j)
      if (rows[(size_t)j] == &it->second)
        return fail(PA_ERR_INVALID_ARG, "request %lld listed twice", (long long)requests[i]);
    rows[(size_t)i] = &it->second;
    const int32_t need =
        (num_tokens_after[i] + p->block_size - 1) / p->block_size - (int32_t)it->second.size();
    if (need > 0) total += need;
  }
  if (total > p->nfree)
    return fail(PA_ERR_NO_BLOCKS, "%lld blocks needed, %d free", (long long)total, p->nfree);
  for (int32_t i = 0; i < n; ++i) {
    std::vector<int32_t>& v = *rows[(size_t)i];
    const int32_t need = (num_tokens_after[i] + p->block_size - 1) / p->block_size - (int32_t)v.size();
    if (need <= 0) continue;
    const size_t old = v.size();
    v.resize(old + (size_t)need);
    p->take(need, v.data() + old);
  }
  return PA_OK;
}

int32_t pa_hash_blocks(const int32_t* tokens, int32_t num_tokens, int32_t block_size,
                       const void* extra, int32_t extra_len, pa_block_hash* out, int32_t cap) {
  if (num_tokens < 0 || (num_tokens && !tokens) || block_size < 1 || cap < 0 ||
      (cap && !out) || extra_len < 0 || (extra_len && !extra))
    return fail(PA_ERR_INVALID_ARG, "bad arguments");
  const int32_t full = num_tokens / block_size;
  const pa_block_hash* parent = nullptr;
  const int32_t m = full < cap ? full : cap;
  for (int32_t i = 0; i < m; ++i) {
    hash_block(parent, tokens + (int64_t)i * block_size, block_size, extra, extra_len, out + i);
    parent = out + i;
  }
  return full;
}

int pa_bp_free_request(pa_block_pool* p, int64_t rid) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  const std::vector<int32_t>& v = it->second;
  for (size_t i = v.size(); i-- > 0;)
    if (v[i] >= 0) p->release(v[i]);           // -1: released by the sliding window
  p->requests.erase(it);
  return PA_OK;
}

int32_t pa_bp_request_blocks(const pa_block_pool* p, int64_t rid, int32_t* out, int32_t cap) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  const int32_t n = (int32_t)it->second.size();
  for (int32_t i = 0; out && i < n && i < cap; ++i) out[i] = it->second[(size_t)i];
  return n;
}

int32_t pa_bp_remove_skipped_blocks(pa_block_pool* p, int64_t rid, int32_t num_tokens,
                                    int32_t window) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  if (num_tokens < 0 || window < 1) return fail(PA_ERR_INVALID_ARG, "bad token count or window");
  const int64_t first = (int64_t)num_tokens - window + 1;   // first position still seen
  if (first <= 0) return 0;
  int64_t nfull = first / p->block_size;                     // blocks wholly before it
  if (nfull > (int64_t)it->second.size()) nfull = (int64_t)it->second.size();
  int32_t released = 0;
  for (int64_t j = nfull; j-- > 0;) {                        // last to first, as free does
    int32_t& b = it->second[(size_t)j];
    if (b < 0) continue;
    p->release(b);
    b = -1;
    ++released;
  }
  return released;
}

int pa_bp_fork_request(pa_block_pool* p, int64_t parent, int64_t child) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(parent);
  if (it == p->requests.end())
    return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)parent);
  if (p->requests.count(child)) return fail(PA_ERR_INVALID_ARG, "request %lld exists", (long long)child);
  std::vector<int32_t> v = it->second;
  for (int32_t b : v)
    if (b >= 0) ++p->ref[(size_t)b];
  p->requests[child] = std::move(v);
  return PA_OK;
}

int pa_bp_prepare_write(pa_block_pool* p, int64_t rid, int32_t position, int64_t* copy_pair) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  auto it = p->requests.find(rid);
  if (it == p->requests.end()) return fail(PA_ERR_INVALID_ARG, "no request %lld", (long long)rid);
  if (position < 0) return fail(PA_ERR_INVALID_ARG, "negative position");
  const int32_t j = position / p->block_size;
  if (j >= (int32_t)it->second.size())
    return fail(PA_ERR_INVALID_ARG, "position %d beyond the request's blocks", position);
  const int32_t b = it->second[(size_t)j];
  if (b < 0) return fail(PA_ERR_INVALID_ARG, "position %d lies in a released block", position);
  if (p->ref[(size_t)b] <= 1) return 0;
  if (p->nfree < 1) return fail(PA_ERR_NO_BLOCKS, "no free block for copy-on-write");
  int32_t nb;
  p->take(1, &nb);
  p->release(b);
  it->second[(size_t)j] = nb;
  if (copy_pair) {
    copy_pair[0] = b;
    copy_pair[1] = nb;
  }
  return 1;
}

}  // extern "C"
