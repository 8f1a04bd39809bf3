// pa_alloc.cpp -- the block allocator declared in include/pa_alloc.h (host
// code only): blocks on demand, release at the end of a sequence, prefix
// caching of complete blocks under a chained FNV-1a hash.
//
// The free queue is an intrusive doubly linked list over block ids, so
// taking the front, joining either end and removing a block that a prefix
// hit revives are all O(1). A call first plans (prefix hits, blocks to take),
// checks the pool, and only then changes state.
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"
#include "pa_alloc.h"
#include "pa_error.h"

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

// 64-bit FNV-1a (Fowler, Noll, Vo): per byte, xor it in, then multiply by
// the prime modulo 2^64.
inline uint64_t fnv1a_bytes(uint64_t h, const uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// H(parent, tokens): the parent hash as 8 little-endian bytes, then each
// token id as 4 little-endian bytes.
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint8_t b[8];
  for (int i = 0; i < 8; ++i) b[i] = (uint8_t)(parent >> (8 * i));
  uint64_t h = fnv1a_bytes(kFnvOffset, b, 8);
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t u = (uint32_t)tokens[t];
    const uint8_t tb[4] = {(uint8_t)u, (uint8_t)(u >> 8), (uint8_t)(u >> 16), (uint8_t)(u >> 24)};
    h = fnv1a_bytes(h, tb, 4);
  }
  return h;
}

struct Seq {
  std::vector<int32_t> blocks;
  int64_t length = 0;
  uint64_t parent = 0;            // hash of the last complete block (0 before the first)
  std::vector<int32_t> tail;      // token ids of the incomplete last block
  bool hashable = true;           // every token so far came with its id
  bool matching = true;           // every block so far was a prefix hit
  int32_t ring = 0;               // > 0: a ring of this many blocks (position t in block (t/bs) mod ring)
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t bs = 16;
  bool prefix = true;
  // Free queue: prev/next links, -1 ends; head/tail; in_queue flags.
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_queue;
  int32_t head = -1, tail = -1, queued = 0;
  std::vector<int32_t> ref;
  std::vector<uint64_t> hash_of;
  std::vector<uint8_t> has_hash;
  std::unordered_map<uint64_t, int32_t> cached;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t queried = 0, hits = 0;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_queue[b] = 1;
    ++queued;
  }
  void push_front(int32_t b) {
    next[b] = head;
    prev[b] = -1;
    if (head >= 0) prev[head] = b; else tail = b;
    head = b;
    in_queue[b] = 1;
    ++queued;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_queue[b] = 0;
    --queued;
  }
  int32_t pop_front() {
    const int32_t b = head;
    unlink(b);
    return b;
  }

  int append(int64_t sid, int32_t n, const int32_t* tokens, int64_t* slots, int32_t* cached_out);
};

int pa_allocator::append(int64_t sid, int32_t n, const int32_t* tokens, int64_t* slots, int32_t* cached_out) {
  auto it = seqs.find(sid);
  if (it == seqs.end()) return pa::fail(PA_ERR_INVALID_ARG, "no live sequence %lld", (long long)sid);
  if (n < 0) return pa::fail(PA_ERR_INVALID_ARG, "token count %d < 0", n);
  if (n > 0 && !slots) return pa::fail(PA_ERR_INVALID_ARG, "slot_ids is NULL");
  Seq& s = it->second;

  // Plan the leading prefix hits.
  std::vector<std::pair<int32_t, uint64_t>> hit;
  int64_t looked = 0;
  if (prefix && tokens && s.hashable && s.matching && s.length % bs == 0 && n > 0) {
    const int32_t may_hit = (n - 1) / bs;
    uint64_t parent = s.parent;
    for (int32_t i = 0; i < may_hit; ++i) {
      const uint64_t h = block_hash(parent, tokens + (size_t)i * bs, bs);
      ++looked;
      auto c = cached.find(h);
      if (c == cached.end()) break;
      hit.emplace_back(c->second, h);
      parent = h;
    }
  }
  const int32_t cached_tokens = (int32_t)hit.size() * bs;
  int64_t total_blocks = (s.length + n + bs - 1) / bs;
  if (s.ring > 0 && total_blocks > s.ring) total_blocks = s.ring;
  const int64_t fresh = total_blocks - (int64_t)s.blocks.size() - (int64_t)hit.size();
  int64_t from_queue = fresh;
  for (const auto& h : hit)
    if (ref[h.first] == 0) ++from_queue;
  if (from_queue > queued)
    return pa::fail(PA_ERR_NO_BLOCKS, "sequence %lld needs %lld free blocks, %d are free", (long long)sid,
                    (long long)from_queue, queued);

  // Commit.
  queried += looked;
  hits += (int64_t)hit.size();
  int32_t k = 0;
  for (const auto& h : hit) {
    if (ref[h.first] == 0) unlink(h.first);
    ++ref[h.first];
    s.blocks.push_back(h.first);
    s.parent = h.second;
    s.length += bs;
    for (int32_t j = 0; j < bs; ++j) slots[k++] = -1;
  }
  if (!tokens && n > 0) s.hashable = false;
  if (n > cached_tokens) s.matching = false;
  // A ring position that a later token of this call overwrites is not written at all.
  const int64_t keep_from = s.ring > 0 ? s.length + (n - cached_tokens) - (int64_t)s.ring * bs : INT64_MIN;
  for (int32_t i = cached_tokens; i < n; ++i) {
    const int64_t pos = s.length;
    const int64_t entry = s.ring > 0 ? (pos / bs) % s.ring : pos / bs;
    if (entry == (int64_t)s.blocks.size()) {
      const int32_t b = pop_front();
      if (has_hash[b]) {
        cached.erase(hash_of[b]);
        has_hash[b] = 0;
      }
      ref[b] = 1;
      s.blocks.push_back(b);
    }
    slots[k++] = pos < keep_from ? -1 : (int64_t)s.blocks[entry] * bs + pos % bs;
    s.length = pos + 1;
    if (s.hashable) s.tail.push_back(tokens[i]);
    if (s.length % bs == 0) {
      if (prefix && s.hashable) {
        const uint64_t h = block_hash(s.parent, s.tail.data(), bs);
        const int32_t b = s.blocks.back();
        if (!cached.count(h) && !has_hash[b]) {
          cached.emplace(h, b);
          hash_of[b] = h;
          has_hash[b] = 1;
        }
        s.parent = h;
      }
      s.tail.clear();
    }
  }
  if (cached_out) *cached_out = cached_tokens;
  return PA_OK;
}

extern "C" {

int pa_alloc_create(int32_t num_blocks, int32_t block_size, int32_t prefix_cache, pa_allocator** out) {
  pa::clear_error();
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return pa::fail(PA_ERR_INVALID_ARG, "num_blocks and block_size must be >= 1");
  if (prefix_cache != 0 && prefix_cache != 1) return pa::fail(PA_ERR_INVALID_ARG, "prefix_cache must be 0 or 1");
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "out of host memory");
  try {
    a->num_blocks = num_blocks;
    a->bs = block_size;
    a->prefix = prefix_cache != 0;
    a->prev.assign(num_blocks, -1);
    a->next.assign(num_blocks, -1);
    a->in_queue.assign(num_blocks, 0);
    a->ref.assign(num_blocks, 0);
    a->hash_of.assign(num_blocks, 0);
    a->has_hash.assign(num_blocks, 0);
  } catch (...) {
    delete a;
    return pa::fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  for (int32_t b = 0; b < num_blocks; ++b) a->push_back(b);
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int pa_alloc_add(pa_allocator* a, int64_t seq_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  if (a->seqs.count(seq_id)) return pa::fail(PA_ERR_INVALID_ARG, "sequence %lld is live", (long long)seq_id);
  a->seqs.emplace(seq_id, Seq());
  return PA_OK;
}

int pa_alloc_add_ring(pa_allocator* a, int64_t seq_id, int32_t ring_blocks) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  if (ring_blocks < 1) return pa::fail(PA_ERR_INVALID_ARG, "ring_blocks must be >= 1 (got %d)", ring_blocks);
  if (a->seqs.count(seq_id)) return pa::fail(PA_ERR_INVALID_ARG, "sequence %lld is live", (long long)seq_id);
  Seq s;
  s.ring = ring_blocks;
  s.hashable = false;
  s.matching = false;
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_alloc_append(pa_allocator* a, int64_t seq_id, int32_t n, const int32_t* tokens, int64_t* slot_ids,
                    int32_t* cached) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  try {
    return a->append(seq_id, n, tokens, slot_ids, cached);
  } catch (...) {
    return pa::fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
}

int pa_alloc_append_batch(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids, const int32_t* counts,
                          const int32_t* tokens, int64_t* slot_ids, int32_t* cached, int32_t* done) {
  pa::clear_error();
  if (done) *done = 0;
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  if (num_seqs < 0) return pa::fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
  if (num_seqs > 0 && (!seq_ids || !counts)) return pa::fail(PA_ERR_INVALID_ARG, "seq_ids or counts is NULL");
  size_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int rc;
    try {
      rc = a->append(seq_ids[i], counts[i], tokens ? tokens + off : nullptr, slot_ids ? slot_ids + off : nullptr,
                     cached ? cached + i : nullptr);
    } catch (...) {
      rc = pa::fail(PA_ERR_INVALID_ARG, "out of host memory");
    }
    if (rc != PA_OK) return rc;
    off += (size_t)counts[i];
    if (done) *done = i + 1;
  }
  return PA_OK;
}

int pa_alloc_release(pa_allocator* a, int64_t seq_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID_ARG, "no live sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
    if (--a->ref[*b] == 0) {
      if (a->has_hash[*b]) a->push_back(*b); else a->push_front(*b);
    }
  }
  a->seqs.erase(it);
  return PA_OK;
}

int32_t pa_alloc_num_free(const pa_allocator* a) { return a ? a->queued : -1; }

int pa_alloc_block_table(const pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids, int32_t max_blocks,
                         int32_t* table, int32_t* seq_lens) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  if (num_seqs < 0 || max_blocks < 0) return pa::fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs > 0 && (!seq_ids || !seq_lens || (max_blocks > 0 && !table)))
    return pa::fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  for (int32_t i = 0; i < num_seqs; ++i) {   // check everything before writing anything
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID_ARG, "no live sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return pa::fail(PA_ERR_INVALID_ARG, "sequence %lld holds %zu blocks > max_blocks %d", (long long)seq_ids[i],
                      it->second.blocks.size(), max_blocks);
    if (it->second.length > INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARG, "sequence %lld is longer than 2^31-1 tokens", (long long)seq_ids[i]);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = table + (size_t)i * max_blocks;
    const size_t nb = s.blocks.size();
    if (nb) std::memcpy(row, s.blocks.data(), nb * sizeof(int32_t));
    for (size_t j = nb; j < (size_t)max_blocks; ++j) row[j] = 0;
    seq_lens[i] = (int32_t)s.length;
  }
  return PA_OK;
}

int pa_alloc_stats(const pa_allocator* a, int64_t* queried, int64_t* hits) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID_ARG, "allocator is NULL");
  if (queried) *queried = a->queried;
  if (hits) *hits = a->hits;
  return PA_OK;
}

int pa_alloc_free_queue(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* count) {
  pa::clear_error();
  if (!a || !count) return pa::fail(PA_ERR_INVALID_ARG, "allocator or count is NULL");
  if (cap > 0 && !out) return pa::fail(PA_ERR_INVALID_ARG, "out is NULL");
  int32_t i = 0;
  for (int32_t b = a->head; b >= 0 && i < cap; b = a->next[b]) out[i++] = b;
  *count = a->queued;
  return PA_OK;
}

}  // extern "C"
