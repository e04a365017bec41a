// Host-side block allocator of the paged KV cache: the step before the
// decode kernels, which produces the block tables and slots they consume.
//
// Behaviour (faulkner, "Prefix Caching 与 Copy-on-Write" and the allocator
// reference section; qwbw 4.3):
// * a full block is identified by a chained hash H_k = Hash(H_{k-1}, tokens
//   of block k), H_{-1} = 0, the hash being BLAKE2b with an 8-byte digest
//   over the parent (8 bytes, little-endian) and each token id (4 bytes,
//   little-endian);
// * a block whose reference count drops to zero keeps its hash and is parked
//   at the most recently used end of an LRU list of evictable blocks; fresh
//   blocks come from the least recently used end and lose their hash;
// * a new prompt matches its leading full blocks by hash in order (a hit
//   only increments the block's count) and stops at the first miss or at
//   the partial last block; its later full blocks are registered under
//   their hashes;
// * appending a token to a full tail block takes a fresh block; appending to
//   a partly filled tail shared by several sequences (count > 1) is a
//   copy-on-write: a fresh block receives the slots (the caller copies the
//   rows on the device with copy_blocks) and the old block's count drops;
// * running out of blocks is KVP_ERR_OUT_OF_MEMORY (the listing's
//   MemoryError), and a call that cannot be met changes nothing.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "internal.h"

namespace {

// ---------------------------------------------------------------- BLAKE2b
// RFC 7693, unkeyed, digest of outlen bytes (1 ... 64).
class Blake2b {
 public:
  explicit Blake2b(size_t outlen) : outlen_(outlen) {
    for (int i = 0; i < 8; ++i) h_[i] = kIV[i];
    h_[0] ^= 0x01010000ull ^ (uint64_t)outlen;   // parameter block: depth 1, fanout 1, no key
  }
  void update(const uint8_t* in, size_t n) {
    for (size_t i = 0; i < n; ++i) {
      if (c_ == 128) {                           // a full buffer is compressed only once more input arrives
        t_ += 128;
        compress(false);
        c_ = 0;
      }
      buf_[c_++] = in[i];
    }
  }
  void final(uint8_t* out) {
    t_ += c_;
    std::memset(buf_ + c_, 0, 128 - c_);
    compress(true);
    for (size_t i = 0; i < outlen_; ++i) out[i] = (uint8_t)(h_[i / 8] >> (8 * (i % 8)));
  }

 private:
  static constexpr uint64_t kIV[8] = {0x6A09E667F3BCC908ull, 0xBB67AE8584CAA73Bull, 0x3C6EF372FE94F82Bull,
                                      0xA54FF53A5F1D36F1ull, 0x510E527FADE682D1ull, 0x9B05688C2B3E6C1Full,
                                      0x1F83D9ABFB41BD6Bull, 0x5BE0CD19137E2179ull};
  static constexpr uint8_t kSigma[10][16] = {
      {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}, {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3},
      {11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4}, {7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8},
      {9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13}, {2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9},
      {12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11}, {13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10},
      {6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5}, {10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0}};
  static uint64_t rotr(uint64_t x, int n) { return (x >> n) | (x << (64 - n)); }
  static void mix(uint64_t* v, int a, int b, int c, int d, uint64_t x, uint64_t y) {
    v[a] = v[a] + v[b] + x;
    v[d] = rotr(v[d] ^ v[a], 32);
    v[c] = v[c] + v[d];
    v[b] = rotr(v[b] ^ v[c], 24);
    v[a] = v[a] + v[b] + y;
    v[d] = rotr(v[d] ^ v[a], 16);
    v[c] = v[c] + v[d];
    v[b] = rotr(v[b] ^ v[c], 63);
  }
  void compress(bool last) {
    uint64_t m[16], v[16];
    for (int i = 0; i < 16; ++i) {
      uint64_t w = 0;
      for (int j = 7; j >= 0; --j) w = (w << 8) | buf_[8 * i + j];
      m[i] = w;
    }
    for (int i = 0; i < 8; ++i) {
      v[i] = h_[i];
      v[i + 8] = kIV[i];
    }
    v[12] ^= t_;                                 // low 64 bits of the byte count (prompts stay far below 2^64)
    if (last) v[14] = ~v[14];
    for (int r = 0; r < 12; ++r) {
      const uint8_t* s = kSigma[r % 10];
      mix(v, 0, 4, 8, 12, m[s[0]], m[s[1]]);
      mix(v, 1, 5, 9, 13, m[s[2]], m[s[3]]);
      mix(v, 2, 6, 10, 14, m[s[4]], m[s[5]]);
      mix(v, 3, 7, 11, 15, m[s[6]], m[s[7]]);
      mix(v, 0, 5, 10, 15, m[s[8]], m[s[9]]);
      mix(v, 1, 6, 11, 12, m[s[10]], m[s[11]]);
      mix(v, 2, 7, 8, 13, m[s[12]], m[s[13]]);
      mix(v, 3, 4, 9, 14, m[s[14]], m[s[15]]);
    }
    for (int i = 0; i < 8; ++i) h_[i] ^= v[i] ^ v[i + 8];
  }
  uint64_t h_[8];
  uint64_t t_ = 0;
  uint8_t buf_[128];
  size_t c_ = 0;
  size_t outlen_;
};
constexpr uint64_t Blake2b::kIV[8];
constexpr uint8_t Blake2b::kSigma[10][16];

uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int64_t n) {
  Blake2b b(8);
  uint8_t p[8];
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(parent >> (8 * i));
  b.update(p, 8);
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t t = (uint32_t)tokens[i];
    const uint8_t w[4] = {(uint8_t)t, (uint8_t)(t >> 8), (uint8_t)(t >> 16), (uint8_t)(t >> 24)};
    b.update(w, 4);
  }
  uint8_t out[8];
  b.final(out);
  uint64_t h = 0;
  for (int i = 7; i >= 0; --i) h = (h << 8) | out[i];
  return h;
}

kvp_status afail(kvp_status st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  pkv::set_last_error(buf);
  return st;
}

void pkv_allocator_clear_error() { pkv::set_last_error(""); }

}  // namespace

struct kvp_allocator {
  int64_t n = 0;
  int32_t bs = 0;
  std::vector<int32_t> ref;        // reference count per block
  std::vector<int32_t> fill;       // slots in use per block
  std::vector<uint64_t> hash;
  std::vector<uint8_t> hashed;
  // evictable blocks: a doubly linked list from the least (head) to the most
  // (tail) recently used, -1 terminated; in_list marks membership
  std::vector<int64_t> prev, next;
  std::vector<uint8_t> in_list;
  int64_t head = -1, tail = -1, n_free = 0;
  std::unordered_map<uint64_t, int32_t> by_hash;

  void push_mru(int64_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_list[b] = 1;
    ++n_free;
  }
  void unlink(int64_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    in_list[b] = 0;
    --n_free;
  }
  // a fresh block from the LRU end (the caller has checked one is free)
  int32_t take() {
    const int64_t b = head;
    unlink(b);
    if (hashed[b]) {
      auto it = by_hash.find(hash[b]);
      if (it != by_hash.end() && it->second == b) by_hash.erase(it);
      hashed[b] = 0;
    }
    fill[b] = 0;
    ref[b] = 1;
    return (int32_t)b;
  }
};

extern "C" {

kvp_status kvp_allocator_create(int64_t num_blocks, int32_t block_size, const int32_t* initial_order,
                                kvp_allocator** out) {
  pkv_allocator_clear_error();
  if (!out) return afail(KVP_ERR_INVALID_ARG, "kvp_allocator_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > ((int64_t)1 << 31) - 1 || block_size <= 0)
    return afail(KVP_ERR_INVALID_ARG, "kvp_allocator_create: num_blocks must be in [1, 2^31) and block_size > 0");
  kvp_allocator* a = new (std::nothrow) kvp_allocator;
  if (!a) return afail(KVP_ERR_OUT_OF_MEMORY, "kvp_allocator_create: host allocation failed");
  try {
    a->n = num_blocks;
    a->bs = block_size;
    a->ref.assign(num_blocks, 0);
    a->fill.assign(num_blocks, 0);
    a->hash.assign(num_blocks, 0);
    a->hashed.assign(num_blocks, 0);
    a->prev.assign(num_blocks, -1);
    a->next.assign(num_blocks, -1);
    a->in_list.assign(num_blocks, 0);
  } catch (...) {
    delete a;
    return afail(KVP_ERR_OUT_OF_MEMORY, "kvp_allocator_create: host allocation failed");
  }
  for (int64_t i = 0; i < num_blocks; ++i) {
    const int64_t b = initial_order ? initial_order[i] : i;
    if (b < 0 || b >= num_blocks || a->in_list[b]) {
      delete a;
      return afail(KVP_ERR_INVALID_ARG, "kvp_allocator_create: initial_order is not a permutation of the block ids");
    }
    a->push_mru(b);
  }
  *out = a;
  return KVP_OK;
}

void kvp_allocator_destroy(kvp_allocator* a) { delete a; }

uint64_t kvp_block_hash(uint64_t parent, const int32_t* token_ids, int32_t n) {
  return chain_hash(parent, token_ids, n < 0 ? 0 : n);
}

kvp_status kvp_allocate_prompt(kvp_allocator* a, const int32_t* token_ids, int64_t num_tokens,
                               int32_t* block_table, int32_t max_blocks, int32_t* num_blocks,
                               int64_t* cached_tokens) {
  pkv_allocator_clear_error();
  if (!a || !num_blocks || !cached_tokens || num_tokens < 0 || (num_tokens > 0 && (!token_ids || !block_table)))
    return afail(KVP_ERR_INVALID_ARG, "kvp_allocate_prompt: NULL pointer or negative length");
  const int64_t bs = a->bs;
  const int64_t nb = (num_tokens + bs - 1) / bs;
  if (nb > max_blocks) return afail(KVP_ERR_INVALID_ARG, "kvp_allocate_prompt: %lld blocks needed, the table holds %d",
                                    (long long)nb, max_blocks);
  // all or nothing: the leading hits (those parked in the evictable list
  // leave it), then the fresh blocks still needed
  int64_t hits = 0, parked = 0;
  uint64_t parent = 0;
  std::vector<int32_t> hit_blocks;
  for (int64_t k = 0; (k + 1) * bs <= num_tokens; ++k) {
    parent = chain_hash(parent, token_ids + k * bs, bs);
    auto it = a->by_hash.find(parent);
    if (it == a->by_hash.end()) break;
    hit_blocks.push_back(it->second);
    if (a->ref[it->second] == 0) ++parked;
    ++hits;
  }
  if (nb - hits > a->n_free - parked)
    return afail(KVP_ERR_OUT_OF_MEMORY, "kvp_allocate_prompt: out of KV cache blocks (%lld needed, %lld free)",
                 (long long)(nb - hits), (long long)(a->n_free - parked));
  parent = 0;
  for (int64_t k = 0; k < nb; ++k) {
    const int64_t len = std::min<int64_t>(bs, num_tokens - k * bs);
    if (k < hits) {
      const int32_t b = hit_blocks[k];
      if (a->ref[b] == 0) a->unlink(b);
      ++a->ref[b];
      block_table[k] = b;
      parent = a->hash[b];
      continue;
    }
    const int32_t b = a->take();
    a->fill[b] = (int32_t)len;
    if (len == bs) {
      parent = chain_hash(parent, token_ids + k * bs, bs);
      a->hash[b] = parent;
      a->hashed[b] = 1;
      a->by_hash[parent] = b;
    }
    block_table[k] = b;
  }
  *num_blocks = (int32_t)nb;
  *cached_tokens = hits * bs;
  return KVP_OK;
}

kvp_status kvp_append_slot(kvp_allocator* a, int32_t* block_table, int32_t* num_blocks, int32_t max_blocks,
                           int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  pkv_allocator_clear_error();
  if (!a || !block_table || !num_blocks || !slot || !cow_src || !cow_dst || *num_blocks <= 0)
    return afail(KVP_ERR_INVALID_ARG, "kvp_append_slot: NULL pointer or empty table");
  *cow_src = *cow_dst = -1;
  const int32_t last = block_table[*num_blocks - 1];
  if (last < 0 || last >= a->n || a->ref[last] <= 0)
    return afail(KVP_ERR_INVALID_ARG, "kvp_append_slot: the tail block %d is not held", last);
  if (a->fill[last] == a->bs) {
    if (*num_blocks >= max_blocks) return afail(KVP_ERR_INVALID_ARG, "kvp_append_slot: the block table is full");
    if (a->n_free == 0) return afail(KVP_ERR_OUT_OF_MEMORY, "kvp_append_slot: out of KV cache blocks");
    const int32_t b = a->take();
    a->fill[b] = 1;
    block_table[(*num_blocks)++] = b;
    *slot = (int64_t)b * a->bs;
    return KVP_OK;
  }
  if (a->ref[last] > 1) {
    if (a->n_free == 0) return afail(KVP_ERR_OUT_OF_MEMORY, "kvp_append_slot: out of KV cache blocks");
    const int32_t b = a->take();
    --a->ref[last];
    a->fill[b] = a->fill[last] + 1;
    block_table[*num_blocks - 1] = b;
    *cow_src = last;
    *cow_dst = b;
    *slot = (int64_t)b * a->bs + a->fill[b] - 1;
    return KVP_OK;
  }
  ++a->fill[last];
  *slot = (int64_t)last * a->bs + a->fill[last] - 1;
  return KVP_OK;
}

kvp_status kvp_fork_sequence(kvp_allocator* a, const int32_t* block_table, int32_t num_blocks) {
  pkv_allocator_clear_error();
  if (!a || (num_blocks > 0 && !block_table) || num_blocks < 0)
    return afail(KVP_ERR_INVALID_ARG, "kvp_fork_sequence: NULL pointer or negative length");
  for (int32_t i = 0; i < num_blocks; ++i)
    if (block_table[i] < 0 || block_table[i] >= a->n || a->ref[block_table[i]] <= 0)
      return afail(KVP_ERR_INVALID_ARG, "kvp_fork_sequence: block %d is not held", block_table[i]);
  for (int32_t i = 0; i < num_blocks; ++i) ++a->ref[block_table[i]];
  return KVP_OK;
}

kvp_status kvp_free_sequence(kvp_allocator* a, const int32_t* block_table, int32_t num_blocks) {
  pkv_allocator_clear_error();
  if (!a || (num_blocks > 0 && !block_table) || num_blocks < 0)
    return afail(KVP_ERR_INVALID_ARG, "kvp_free_sequence: NULL pointer or negative length");
  std::unordered_map<int32_t, int32_t> uses;
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = block_table[i];
    if (b < 0 || b >= a->n) return afail(KVP_ERR_INVALID_ARG, "kvp_free_sequence: block %d out of range", b);
    if (++uses[b] > a->ref[b])
      return afail(KVP_ERR_INVALID_ARG, "kvp_free_sequence: block %d freed more often than it is held", b);
  }
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = block_table[i];
    if (--a->ref[b] == 0) a->push_mru(b);
  }
  return KVP_OK;
}

kvp_status kvp_allocator_block_state(const kvp_allocator* a, int32_t block, int32_t* ref_count, int32_t* fill,
                                     int32_t* hashed, uint64_t* hash) {
  pkv_allocator_clear_error();
  if (!a || block < 0 || block >= a->n || !ref_count || !fill || !hashed || !hash)
    return afail(KVP_ERR_INVALID_ARG, "kvp_allocator_block_state: bad argument");
  *ref_count = a->ref[block];
  *fill = a->fill[block];
  *hashed = a->hashed[block];
  *hash = a->hash[block];
  return KVP_OK;
}

int64_t kvp_allocator_evictable(const kvp_allocator* a, int32_t* out, int64_t capacity) {
  if (!a) return -1;
  int64_t k = 0;
  for (int64_t b = a->head; b >= 0; b = a->next[b]) {
    if (out && k < capacity) out[k] = (int32_t)b;
    ++k;
  }
  return k;
}

}  // extern "C"
