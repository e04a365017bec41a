// C-ABI host layer: argument validation, pool management, split planning,
// workspace sizing and kernel dispatch.  Every check runs on the host before
// anything is enqueued; failures return a status and set a per-thread message.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pagedkv.h"
#include "internal.h"
#include "probes.h"

namespace {

thread_local std::string g_last_error;

kvp_status fail(kvp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvp_status ok() {
  g_last_error.clear();
  return KVP_OK;
}

kvp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t dtype_bytes(kvp_dtype t) {
  switch (t) {
    case KVP_F32: return 4;
    case KVP_BF16: return 2;
    case KVP_INT8: return 1;
    case KVP_INT4: return 1;   // two codes per byte: rows are row_bytes(), not d * this
  }
  return 0;
}

bool dtype_valid(int t) { return t == KVP_F32 || t == KVP_BF16 || t == KVP_INT8 || t == KVP_INT4; }

bool quantized(kvp_dtype t) { return t == KVP_INT8 || t == KVP_INT4; }

// Bytes of one head's row of d elements.
size_t row_bytes(kvp_dtype t, int64_t d) { return t == KVP_INT4 ? (size_t)d / 2 : (size_t)d * dtype_bytes(t); }

struct PoolLayout {
  size_t k_off = 0, v_off = 0, ks_off = 0, vs_off = 0, total = 0;
  size_t k_bytes = 0, v_bytes = 0, s_bytes = 0;
};

const char* pool_desc_error(const kvp_pool_desc* d) {
  if (!d) return "pool description is NULL";
  if (d->num_blocks <= 0) return "num_blocks must be > 0";
  if (!is_pow2(d->block_size) || d->block_size > 256) return "block_size must be a power of two in [1, 256]";
  if (d->n_kv <= 0) return "n_kv must be > 0";
  if (d->d_k <= 0 || d->d_v <= 0) return "d_k and d_v must be > 0";
  if (!dtype_valid(d->dtype)) return "unknown pool dtype";
  if (d->latent != 0 && d->latent != 1) return "latent must be 0 or 1";
  if (d->latent && d->n_kv != 1) return "a latent pool has n_kv == 1";
  if (d->latent && d->d_v > d->d_k) return "a latent pool needs d_v <= d_k";
  if (d->latent && quantized(d->dtype)) return "INT8 and INT4 latent pools are not supported";
  if (d->dtype == KVP_INT4 && (d->d_k % 8 || d->d_v % 8)) return "INT4 rows need d a multiple of 8";
  const size_t eb = dtype_bytes(d->dtype);
  if (row_bytes(d->dtype, d->d_k) % 4 || row_bytes(d->dtype, d->d_v) % 4) return "row bytes must be a multiple of 4";
  // K + V + scales per slot, times the slots, must stay far from size_t's end
  const double per_slot = (double)d->n_kv * ((double)(d->d_k + d->d_v) * eb + 8.0);
  if ((double)d->num_blocks * d->block_size * per_slot > 1.0e18) return "pool larger than 1e18 bytes";
  return nullptr;
}

PoolLayout pool_layout(const kvp_pool_desc* d) {
  PoolLayout L;
  const size_t slots = (size_t)d->num_blocks * (size_t)d->block_size;
  L.k_bytes = slots * d->n_kv * row_bytes(d->dtype, d->d_k);
  L.v_bytes = d->latent ? 0 : slots * d->n_kv * row_bytes(d->dtype, d->d_v);
  L.s_bytes = quantized(d->dtype) ? slots * d->n_kv * sizeof(float) : 0;
  size_t off = 0;
  L.k_off = off; off = round_up(off + L.k_bytes, 256);
  L.v_off = off; off = round_up(off + L.v_bytes, 256);
  L.ks_off = off; off = round_up(off + L.s_bytes, 256);
  L.vs_off = off; off = round_up(off + (d->latent ? 0 : L.s_bytes), 256);
  L.total = off;
  return L;
}

}  // namespace

namespace pkv {
void set_last_error(const char* msg) { g_last_error = msg; }
}  // namespace pkv

struct kvp_pool {
  kvp_pool_desc desc;
  PoolLayout layout;
  uint8_t* base = nullptr;
  bool owned = false;
};

namespace {

// Live pools, so that the debug mode can find the block count of a pool
// passed to a decode call as a raw pointer.
std::mutex g_pools_mu;
std::vector<const kvp_pool*> g_pools;

void register_pool(const kvp_pool* p) {
  std::lock_guard<std::mutex> lk(g_pools_mu);
  g_pools.push_back(p);
}

void unregister_pool(const kvp_pool* p) {
  std::lock_guard<std::mutex> lk(g_pools_mu);
  for (size_t i = 0; i < g_pools.size(); ++i)
    if (g_pools[i] == p) { g_pools[i] = g_pools.back(); g_pools.pop_back(); break; }
}

// Block count of the live pool whose memory holds ptr (-1 if none does).
int64_t registered_blocks(const void* ptr) {
  std::lock_guard<std::mutex> lk(g_pools_mu);
  const uint8_t* a = static_cast<const uint8_t*>(ptr);
  for (const kvp_pool* p : g_pools)
    if (a >= p->base && a < p->base + p->layout.total) return p->desc.num_blocks;
  return -1;
}

}  // namespace

extern "C" {

const char* kvp_last_error(void) { return g_last_error.c_str(); }

const char* kvp_version(void) { return "pagedkv 0.1 (gfx950)"; }

size_t kv_pool_required_bytes(const kvp_pool_desc* desc) {
  if (pool_desc_error(desc)) return 0;
  return pool_layout(desc).total;
}

kvp_status kv_pool_create(const kvp_pool_desc* desc, void* storage, size_t storage_bytes,
                          kvp_pool** out) {
  if (!out) return fail(KVP_ERR_INVALID_ARG, "kv_pool_create: out is NULL");
  *out = nullptr;
  if (const char* e = pool_desc_error(desc)) return fail(KVP_ERR_INVALID_ARG, "kv_pool_create: %s", e);
  PoolLayout L = pool_layout(desc);
  uint8_t* base = nullptr;
  bool owned = false;
  if (storage) {
    if (!aligned(storage, 256)) return fail(KVP_ERR_INVALID_ARG, "kv_pool_create: storage must be 256-byte aligned");
    if (storage_bytes < L.total)
      return fail(KVP_ERR_INVALID_ARG, "kv_pool_create: storage has %zu bytes, pool needs %zu",
                  storage_bytes, L.total);
    base = static_cast<uint8_t*>(storage);
  } else {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, L.total);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(KVP_ERR_OUT_OF_MEMORY, "kv_pool_create: out of device memory for %zu bytes (%s)",
                  L.total, hipGetErrorString(e));
    }
    base = static_cast<uint8_t*>(p);
    owned = true;
  }
  kvp_pool* pool = new (std::nothrow) kvp_pool;
  if (!pool) {
    if (owned) (void)hipFree(base);
    return fail(KVP_ERR_OUT_OF_MEMORY, "kv_pool_create: host allocation failed");
  }
  pool->desc = *desc;
  pool->layout = L;
  pool->base = base;
  pool->owned = owned;
  register_pool(pool);
  *out = pool;
  return ok();
}

void kv_pool_destroy(kvp_pool* pool) {
  if (!pool) return;
  unregister_pool(pool);
  if (pool->owned && pool->base) (void)hipFree(pool->base);
  delete pool;
}

kvp_status kv_pool_view_get(const kvp_pool* pool, kvp_pool_view* out) {
  if (!pool || !out) return fail(KVP_ERR_INVALID_ARG, "kv_pool_view_get: NULL argument");
  const PoolLayout& L = pool->layout;
  out->k = pool->base + L.k_off;
  out->v = pool->desc.latent ? out->k : pool->base + L.v_off;
  out->k_scale = quantized(pool->desc.dtype) ? reinterpret_cast<float*>(pool->base + L.ks_off) : nullptr;
  out->v_scale = (quantized(pool->desc.dtype) && !pool->desc.latent)
                     ? reinterpret_cast<float*>(pool->base + L.vs_off) : nullptr;
  out->total_bytes = L.total;
  out->desc = pool->desc;
  return ok();
}

kvp_status paged_slot_mapping(const int32_t* block_table, int32_t max_blocks_per_seq,
                              int32_t block_size, const int32_t* seq_ids, const int32_t* positions,
                              int64_t num_tokens, int64_t* slots, void* stream) {
  if (num_tokens < 0) return fail(KVP_ERR_INVALID_ARG, "paged_slot_mapping: num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!block_table || !seq_ids || !positions || !slots)
    return fail(KVP_ERR_INVALID_ARG, "paged_slot_mapping: NULL pointer");
  if (max_blocks_per_seq <= 0) return fail(KVP_ERR_INVALID_ARG, "paged_slot_mapping: max_blocks_per_seq must be > 0");
  if (!is_pow2(block_size) || block_size > 256)
    return fail(KVP_ERR_INVALID_ARG, "paged_slot_mapping: block_size must be a power of two in [1, 256]");
  return hip_status(pkv::launch_slot_mapping(block_table, max_blocks_per_seq, log2i(block_size),
                                             seq_ids, positions, num_tokens, slots,
                                             static_cast<hipStream_t>(stream)),
                    "paged_slot_mapping");
}

}  // extern "C"

// ---------------------------------------------------------------- decode
namespace {

enum class Variant { Float, Int8, Int4, Mla };

bool quant_variant(Variant v) { return v == Variant::Int8 || v == Variant::Int4; }

const char* decode_desc_error(const kvp_decode_desc* d) {
  if (!d) return "decode description is NULL";
  if (d->B < 0) return "B must be >= 0";
  if (d->n_h <= 0 || d->n_kv <= 0) return "n_h and n_kv must be > 0";
  if (d->n_h % d->n_kv) return "n_h must be a multiple of n_kv";
  if (d->d_k <= 0 || d->d_v <= 0) return "d_k and d_v must be > 0";
  if (!is_pow2(d->block_size) || d->block_size > 256) return "block_size must be a power of two in [1, 256]";
  if (d->max_blocks_per_seq <= 0) return "max_blocks_per_seq must be > 0";
  if (d->max_context_len < 0) return "max_context_len must be >= 0";
  if ((int64_t)d->max_context_len > (int64_t)d->max_blocks_per_seq * d->block_size)
    return "max_context_len exceeds max_blocks_per_seq * block_size";
  if (d->q_dtype != KVP_F32 && d->q_dtype != KVP_BF16) return "q_dtype must be F32 or BF16";
  if (!dtype_valid(d->kv_dtype)) return "unknown kv_dtype";
  if (d->split_tokens < 0) return "split_tokens must be >= 0";
  if (d->total_context_len < 0) return "total_context_len must be >= 0";
  if (d->workgroups < 0) return "workgroups must be >= 0";
  if (d->shared_prefix_tokens < 0) return "shared_prefix_tokens must be >= 0";
  if (d->window < 0) return "window must be >= 0";
  return nullptr;
}

// The description the work is planned on: with a sliding window a sequence
// is read from its window's start rounded down to 16, so its length for
// planning is at most window + 15.
kvp_decode_desc planning_desc(const kvp_decode_desc* d) {
  kvp_decode_desc e = *d;
  if (d->window > 0) {
    const int64_t span = (int64_t)d->window + 15;
    if (e.max_context_len > span) e.max_context_len = (int32_t)span;
    if (e.total_context_len > 0 && e.total_context_len > (int64_t)d->B * span) e.total_context_len = (int64_t)d->B * span;
    e.shared_prefix_tokens = 0;
  }
  return e;
}

Variant variant_of(const kvp_decode_desc* d) {
  if (d->kv_dtype == KVP_INT8) return Variant::Int8;
  if (d->kv_dtype == KVP_INT4) return Variant::Int4;
  if (d->n_kv == 1 && d->d_k != d->d_v) return Variant::Mla;
  return Variant::Float;
}

int granule(Variant) { return pkv::kGqaSplitGranule; }

// Compute units of the current device (cached per device; 256 when no
// device can be queried, e.g. on a host without a GPU).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
      (void)hipGetLastError();
      cu = 256;
    }
    cached[dev] = cu;
  }
  return cached[dev];
}

// MLA: tiles of 32 tokens over the whole batch, split into W contiguous
// ranges.  An upper bound of the tile count comes from the host-side sizes.
int64_t mla_tile_bound(const kvp_decode_desc* d) {
  const int64_t per_seq = ((int64_t)d->max_context_len + pkv::kMlaTileTokens - 1) / pkv::kMlaTileTokens;
  int64_t bound = (int64_t)d->B * per_seq;
  if (d->total_context_len > 0) {
    const int64_t hint = (d->total_context_len + pkv::kMlaTileTokens - 1) / pkv::kMlaTileTokens + d->B;
    if (hint < bound) bound = hint;
  }
  return bound;
}

int32_t mla_workgroups(const kvp_decode_desc* d) {
  if (d->workgroups > 0) return d->workgroups;
  int64_t w = device_cus();
  const int64_t bound = mla_tile_bound(d);
  if (bound < w) w = bound;
  return (int32_t)(w < 1 ? 1 : w);
}

struct MlaWorkspace {
  size_t meta = 0, ml = 0, o = 0;
  size_t total() const { return meta + ml + o; }
};

MlaWorkspace mla_workspace(const kvp_decode_desc* d) {
  MlaWorkspace m;
  const int32_t W = mla_workgroups(d);
  m.meta = round_up((size_t)d->B * 2 * sizeof(int32_t), 256);
  if (W > 1) {
    // per piece: (max, sum) per head in fp32; the unnormalised output of
    // every head of the launched head groups in bf16
    const size_t rows = (size_t)(W + d->B) * d->n_h;
    const size_t o_rows = (size_t)(W + d->B) * pkv::mla_head_groups(d->n_h) * pkv::kMlaHeadsPerGroup;
    m.ml = round_up(rows * 2 * sizeof(float), 256);
    m.o = round_up(o_rows * d->d_v * sizeof(uint16_t), 256);
  }
  return m;
}

// Context split size, in multiples of the kernel's granule (split grids).
// Uniform batches: about kTargetUnits workgroups doing real work (two
// resident per compute unit on 256 CUs: exactly one round); longer splits
// amortise each workgroup's set-up and merge.  Ragged INT8 batches with a
// total hint on the LDS-ring kernel (the compact grid below): the shortest
// split whose workgroups still fit one round of two per compute unit,
// counting about half a partial split per sequence and KV-head group
// (skewed INT8 batch: 1536, 81.0 us against 82.4 us at 1024, 87.6 us at
// 1280, where a few workgroups spill into a second round, and 97 us at
// 2048).  (Ragged bf16 batches with a hint take the stream grid instead.)
// Other ragged cases take about four times kTargetUnits shorter splits,
// which even out the loads.
constexpr int64_t kTargetUnits = 512;
constexpr int64_t kTargetUnitsRagged = 2048;
constexpr int32_t kMaxSplit = 8192;

// A split stages at most kBtSlots block-table entries in LDS (INT8 caches:
// kBtSlotsInt8, part of the INT8 ring kernel's smaller LDS footprint).
constexpr int32_t kBtSlots = 512;
constexpr int32_t kBtSlotsInt8 = 256;

int32_t max_split(const kvp_decode_desc* d, Variant v) {
  // a windowed split starts anywhere in a block, so it may touch one block more
  const int64_t cap = (int64_t)((quant_variant(v) ? kBtSlotsInt8 : kBtSlots) - (d->window > 0 ? 1 : 0)) *
                      d->block_size;
  return (int32_t)(cap < kMaxSplit ? cap : kMaxSplit);
}

// KV heads per workgroup of the LDS-ring kernel for this description, 0 when
// the description does not run on it.
int ring_kv_group(const kvp_decode_desc* d, Variant v) {
  if (!(v == Variant::Float || quant_variant(v)) || d->n_kv <= 0) return 0;
  const int gq = d->n_h / d->n_kv;
  const bool qb = d->q_dtype == KVP_BF16;
  const pkv::KV kv = v == Variant::Int4 ? pkv::KV::INT4 : v == Variant::Int8 ? pkv::KV::INT8
                                        : (d->kv_dtype == KVP_BF16 ? pkv::KV::BF16 : pkv::KV::F32);
  if (!pkv::gqa_ring_supported(kv, qb, d->d_k, d->d_v, gq)) return 0;
  return pkv::gqa_ring_kv_group(kv, qb, d->d_k, d->d_v, gq, d->n_kv);
}

// Ragged bf16 batches with a total hint on the LDS-ring kernel (no split
// forced, B <= kCompactMaxB): the stream grid, which cuts the batch's tokens
// into equal ranges, one per workgroup, so that no workgroup waits on a long
// sequence's last split (8B-shaped batch: 43.5 against 47.5 us on the
// compact grid; three workgroups per compute unit 55.4 us).  Workgroups per
// KV-head group: one round of two per compute unit, each range at least
// kStreamMinTokens tokens by the hint.  0 = a split grid.  INT8 pools keep
// the compact split grid: there the stream grid ran 89.5 against 81.6 us
// (with one, two or three workgroups per compute unit: 116.5, 89.5, 89.2),
// the equal ranges all streaming at once drawing less bandwidth from their
// 256-byte code runs than the uneven units, whose short ones finish early.
constexpr int64_t kStreamMinTokens = 256;

int32_t stream_wgs(const kvp_decode_desc* d, Variant v) {
  if (d->split_tokens > 0 || d->total_context_len <= 0 || d->B <= 0 || d->B > pkv::kCompactMaxB) return 0;
  if (4 * d->total_context_len >= 3 * (int64_t)d->B * d->max_context_len) return 0;   // not ragged
  if ((int64_t)d->B * ((int64_t)d->max_context_len + 15) >= ((int64_t)1 << 31)) return 0;
  if (v != Variant::Float) return 0;
  const int kh = ring_kv_group(d, v);
  if (kh == 0) return 0;
  const int64_t groups = d->n_kv / kh;
  int64_t w = 2 * (int64_t)device_cus() / groups;
  const int64_t by_len = (d->total_context_len + kStreamMinTokens - 1) / kStreamMinTokens;
  if (w > by_len) w = by_len;
  if (w > 65535) w = 65535;
  return (int32_t)(w < 1 ? 1 : w);
}

// Ragged INT8 batches with a total hint on the LDS-ring kernel (no split
// forced, B <= kCompactMaxB): the compact grid, which launches only the
// splits that exist.
bool compact_ok(const kvp_decode_desc* d, Variant v) {
  return quant_variant(v) && d->split_tokens == 0 && d->total_context_len > 0 && d->B > 0 &&
         d->B <= pkv::kCompactMaxB && 4 * d->total_context_len < 3 * (int64_t)d->B * d->max_context_len &&
         ring_kv_group(d, v) > 0;
}

int32_t plan_split(const kvp_decode_desc* d, Variant v) {
  const int g = granule(v);
  if (d->split_tokens > 0) return d->split_tokens;
  int64_t total = d->total_context_len > 0 ? d->total_context_len : (int64_t)d->B * d->max_context_len;
  // a sliding window reads at most window + 15 tokens (the start rounds down
  // to 16), the grid covering them; the work is sized by the window itself,
  // so an aligned window splits evenly (4096 -> 8 x 512 rather than 8 x 576)
  if (d->window > 0) total = std::min(total, (int64_t)d->B * d->window);
  int64_t heads = v == Variant::Mla ? 1 : d->n_kv;
  const int kh = ring_kv_group(d, v);
  if (kh > 0) heads /= kh;                      // the ring kernel's KV-head groups
  const int64_t work = total * heads;
  const bool ragged = 4 * total < 3 * (int64_t)d->B * d->max_context_len;
  int64_t split;
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t avail = slots - (((int64_t)d->B + 1) / 2) * heads;
  if (compact_ok(d, v) && 4 * avail >= slots) {
    split = (work + avail - 1) / avail;
  } else {
    const int64_t units = ragged ? kTargetUnitsRagged : kTargetUnits;
    split = (work + units - 1) / units;
  }
  split = (split + g - 1) / g * g;
  if (split < g) split = g;
  if (split > max_split(d, v)) split = max_split(d, v);
  return (int32_t)split;
}

int32_t num_splits_of(const kvp_decode_desc* d, int32_t split) {
  if (d->max_context_len <= 0) return 1;
  return (d->max_context_len + split - 1) / split;
}

// Shared prefix on the stream grid (paged_decode_attention, bf16, two KV
// heads per workgroup): the hint rounded down to whole 64-token stages,
// chunks of kPrefixChunk tokens, two prefix workgroups (one per KV head of
// the pair) per chunk and group of prefix_seqs_per_wg(g) sequences, and the
// stream workgroups for the tokens past the prefix filling the rest of one
// round of two workgroups per compute unit.  On the 8B-shaped layer with
// allocator-built tables and per-sequence stream pieces, 128 / 192 / 256-token
// chunks ran 34.9 / 32.7 / 33.0 us (fewer prefix workgroups leave more for
// the stream pieces, and fewer prefix pieces to merge), and a third
// workgroup per compute unit 41.1 us.
#ifndef PKV_PREFIX_CHUNK
#define PKV_PREFIX_CHUNK 192
#endif
#ifndef PKV_PREFIX_ROUND
#define PKV_PREFIX_ROUND 2
#endif
constexpr int32_t kPrefixChunk = PKV_PREFIX_CHUNK;

struct PrefixPlan {
  int32_t tokens = 0, chunk = 0, wgs = 0, stream = 0;
  int32_t pieces(const kvp_decode_desc* d) const {   // prefix pieces: chunks x B
    return tokens ? (tokens + chunk - 1) / chunk * d->B : 0;
  }
};

PrefixPlan prefix_plan(const kvp_decode_desc* d, Variant v) {
  PrefixPlan pp;
  if (d->shared_prefix_tokens <= 0 || v != Variant::Float || d->kv_dtype != KVP_BF16 ||
      d->q_dtype != KVP_BF16 || d->split_tokens > 0 || d->B <= 0 || d->B > pkv::kCompactMaxB ||
      d->d_k != 128 || d->d_v != 128 || ring_kv_group(d, v) != 2)
    return pp;
  const int g = d->n_h / d->n_kv;
  if (g != 4 && g != 8 && g != 16) return pp;
  if ((int64_t)d->B * ((int64_t)d->max_context_len + 15) >= ((int64_t)1 << 31)) return pp;
  const int32_t S = std::min(d->shared_prefix_tokens, d->max_context_len) & ~63;
  if (S < 64) return pp;
  int32_t ch = kPrefixChunk;
  while (ch > 64 && (ch >> log2i(d->block_size)) + 2 > kBtSlots) ch -= 64;
  const int64_t nc = (S + ch - 1) / ch;
  const int64_t ncg = (d->B + pkv::prefix_seqs_per_wg(g) - 1) / pkv::prefix_seqs_per_wg(g);
  const int64_t wgs = 2 * nc * ncg;
  const int64_t groups = d->n_kv / 2;
  const int64_t total = d->total_context_len > 0 ? d->total_context_len : (int64_t)d->B * d->max_context_len;
  int64_t w = PKV_PREFIX_ROUND * (int64_t)device_cus() / groups - wgs;
  const int64_t by_len = (total + kStreamMinTokens - 1) / kStreamMinTokens;
  if (w > by_len) w = by_len;
  if (w < 1) w = 1;
  if (w + wgs > 65535) return pp;
  pp.tokens = S;
  pp.chunk = ch;
  pp.wgs = (int32_t)wgs;
  pp.stream = (int32_t)w;
  return pp;
}

// Stream grid workspace: [part_o pieces x n_h x d_v][part_ml pieces x n_h x
// 2][seq_meta B x 2 int32], each region 256-byte aligned; pieces = wgs + B
// (+ the prefix pieces).
struct StreamWorkspace {
  size_t o_bytes, ml_bytes, meta_bytes;
  size_t total() const { return o_bytes + ml_bytes + meta_bytes; }
};
StreamWorkspace stream_workspace(const kvp_decode_desc* d, int32_t wgs, int32_t extra_pieces = 0) {
  const size_t rows = ((size_t)wgs + d->B + (size_t)extra_pieces) * d->n_h;
  return {round_up(rows * d->d_v * sizeof(float), 256), round_up(rows * 2 * sizeof(float), 256),
          round_up((size_t)d->B * 2 * sizeof(int32_t), 256)};
}

size_t workspace_plain(const kvp_decode_desc* d, Variant v);

// The shared-prefix hint applies to paged_decode_attention only; the same
// description on another entry point runs without it, so the size covers
// both.
size_t workspace_for(const kvp_decode_desc* d, Variant v) {
  const size_t plain = workspace_plain(d, v);
  const PrefixPlan pp = prefix_plan(d, v);
  if (pp.tokens == 0) return plain;
  return std::max(plain, stream_workspace(d, pp.stream, pp.pieces(d)).total());
}

size_t workspace_plain(const kvp_decode_desc* d, Variant v) {
  if (v == Variant::Mla) return d->B > 0 ? mla_workspace(d).total() : 0;
  const int32_t sw = stream_wgs(d, v);
  if (sw > 0) return stream_workspace(d, sw).total();
  const int32_t split = plan_split(d, v);
  const int32_t ns = num_splits_of(d, split);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)d->B * d->n_h * ns;
  return round_up(rows * d->d_v * sizeof(float), 256) + round_up(rows * 2 * sizeof(float), 256);
}

kvp_status check_workspace(const char* fn, size_t need, const void* workspace, size_t workspace_bytes) {
  if (need == 0) return KVP_OK;
  if (!workspace) return fail(KVP_ERR_INVALID_ARG, "%s: workspace of %zu bytes required", fn, need);
  if (workspace_bytes < need)
    return fail(KVP_ERR_INVALID_ARG, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(KVP_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  return KVP_OK;
}

// The MLA kernel: persistent workgroups over the batch's 32-token tiles
// (shape checks already done by decode_common).
kvp_status launch_mla(const char* fn, const void* q, const void* pool, const int32_t* block_table,
                      const int32_t* context_lens, float scale, void* out,
                      const kvp_decode_desc* d, void* workspace, size_t workspace_bytes,
                      void* stream, const void* k_new = nullptr) {
  if (d->B > pkv::kMlaMaxBatch) return fail(KVP_ERR_UNSUPPORTED, "%s: MLA batch must be <= %d", fn, pkv::kMlaMaxBatch);
  const int64_t per_seq = ((int64_t)d->max_context_len + pkv::kMlaTileTokens - 1) / pkv::kMlaTileTokens;
  if ((int64_t)d->B * per_seq >= ((int64_t)1 << 31))
    return fail(KVP_ERR_UNSUPPORTED, "%s: too many context tiles in one batch", fn);
  if (d->workgroups > 65535) return fail(KVP_ERR_INVALID_ARG, "%s: workgroups must be <= 65535", fn);
  const MlaWorkspace m = mla_workspace(d);
  const kvp_status ws = check_workspace(fn, m.total(), workspace, workspace_bytes);
  if (ws != KVP_OK) return ws;
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  pkv::DecodeParams p{};
  p.q = q;
  p.k = pool;
  p.v = pool;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.seq_meta = reinterpret_cast<int32_t*>(wsb);
  p.part_ml = m.ml ? reinterpret_cast<float*>(wsb + m.meta) : nullptr;
  p.part_o = m.o ? reinterpret_cast<float*>(wsb + m.meta + m.ml) : nullptr;
  p.scale = scale;
  p.B = d->B;
  p.n_h = d->n_h;
  p.n_kv = 1;
  p.d_k = d->d_k;
  p.d_v = d->d_v;
  p.block_shift = log2i(d->block_size);
  p.max_blocks_per_seq = d->max_blocks_per_seq;
  p.q_bf16 = true;
  p.kv = pkv::KV::BF16;
  p.workgroups = mla_workgroups(d);
  p.k_new = k_new;
  return hip_status(pkv::launch_decode_mla(p, static_cast<hipStream_t>(stream)), fn);
}

// Rows of new tokens into a pool (reshape_and_cache, and the append path
// of paged_decode_attention_append when the decode kernel does not write
// them itself): bit copy for float pools, quantize-on-write for INT8.
kvp_status write_rows(kvp_pool* pool, const void* k_new, const void* v_new, kvp_dtype in_dtype,
                      const pkv::SlotSource& slots, int64_t num_tokens, void* stream, const char* fn) {
  const kvp_pool_desc& d = pool->desc;
  if (!k_new) return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!d.latent && !v_new) return fail(KVP_ERR_INVALID_ARG, "%s: v_new is NULL", fn);
  if (!dtype_valid(in_dtype)) return fail(KVP_ERR_INVALID_ARG, "%s: unknown in_dtype", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  kvp_pool_view v;
  kv_pool_view_get(pool, &v);
  if (d.dtype == KVP_INT4) {
    if (in_dtype != KVP_F32 && in_dtype != KVP_BF16)
      return fail(KVP_ERR_INVALID_ARG, "%s: INT4 pools take F32 or BF16 rows", fn);
    return hip_status(pkv::launch_cache_quant_int4(static_cast<uint8_t*>(v.k), v.k_scale, k_new, d.d_k,
                                                  static_cast<uint8_t*>(v.v), v.v_scale, v_new, d.d_v,
                                                  in_dtype == KVP_BF16, slots, num_tokens, d.n_kv,
                                                  __builtin_ctz((unsigned)d.block_size), st),
                      fn);
  }
  if (d.dtype == KVP_INT8) {
    if (in_dtype == KVP_INT8 || in_dtype == KVP_INT4)
      return fail(KVP_ERR_INVALID_ARG, "%s: INT8 pools take F32 or BF16 rows", fn);
    const bool bf = in_dtype == KVP_BF16;
    return hip_status(pkv::launch_cache_quant_int8(static_cast<int8_t*>(v.k), v.k_scale, k_new, d.d_k,
                                                  static_cast<int8_t*>(v.v), v.v_scale, v_new, d.d_v,
                                                  bf, slots, num_tokens, d.n_kv,
                                                  __builtin_ctz((unsigned)d.block_size), st),
                      fn);
  }
  if (in_dtype != d.dtype) return fail(KVP_ERR_INVALID_ARG, "%s: rows must have the pool's dtype", fn);
  const size_t eb = dtype_bytes(d.dtype);
  // K and V rows in one launch (a latent pool has no V region)
  return hip_status(pkv::launch_cache_copy(v.k, k_new, (int64_t)d.n_kv * d.d_k * eb,
                                           d.latent ? nullptr : v.v, v_new,
                                           (int64_t)d.n_kv * d.d_v * eb, slots, num_tokens, st),
                    fn);
}

// The checks of paged_decode_validate (synchronises the stream): context
// lengths within [0, max_context_len], table entries a sequence uses within
// [0, num_blocks).
kvp_status check_tables(const char* fn, const int32_t* block_table, const int32_t* context_lens,
                        const kvp_decode_desc* desc, int64_t num_blocks, void* stream) {
  if (desc->B == 0) return ok();
  if (!block_table || !context_lens) return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<int32_t> ctx(desc->B);
  std::vector<int32_t> bt((size_t)desc->B * desc->max_blocks_per_seq);
  hipError_t e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e, fn);
  for (int32_t b = 0; b < desc->B; ++b) {
    const int32_t c = ctx[b];
    if (c < 0 || c > desc->max_context_len)
      return fail(KVP_ERR_INVALID_ARG, "%s: context_lens[%d] = %d outside [0, %d]", fn, b, c,
                  desc->max_context_len);
    const int32_t nb = (int32_t)(((int64_t)c + desc->block_size - 1) / desc->block_size);
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t p = bt[(size_t)b * desc->max_blocks_per_seq + j];
      if (p < 0 || p >= num_blocks)
        return fail(KVP_ERR_INVALID_ARG, "%s: block_table[%d][%d] = %d outside [0, %lld)", fn, b, j, p,
                    (long long)num_blocks);
    }
  }
  return ok();
}

// Debug mode: PAGEDKV_VALIDATE set to anything but "0" (read at every call).
bool validate_mode() {
  const char* v = std::getenv("PAGEDKV_VALIDATE");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

// Blocks of block_bytes each that fit in the memory a pool pointer reaches:
// the pool's own count for a pool made by kv_pool_create, else what fits
// between ptr and the end of its device allocation.
int64_t blocks_reachable(const void* ptr, size_t block_bytes) {
  const int64_t reg = registered_blocks(ptr);
  if (reg >= 0) return reg;
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(ptr)) != hipSuccess || !base) {
    (void)hipGetLastError();
    return 0;
  }
  const size_t used = static_cast<const uint8_t*>(ptr) - static_cast<const uint8_t*>(base);
  return used >= size ? 0 : (int64_t)((size - used) / block_bytes);
}

// INT4 sink rows of paged_decode_attention_int4.
struct SinkRows {
  const void* k;
  const void* v;
  int32_t n;
};

// The append request of paged_decode_attention_append (null for a plain decode).
struct AppendRows {
  kvp_pool* pool;
  const void* k_new;
  const void* v_new;
};

kvp_status decode_common(Variant var, const char* fn, const void* q, const void* k,
                         const void* v, const float* ks, const float* vs,
                         const int32_t* block_table, const int32_t* context_lens, float scale,
                         void* out, const kvp_decode_desc* d, void* workspace,
                         size_t workspace_bytes, void* stream, const AppendRows* app = nullptr,
                         const SinkRows* sink = nullptr) {
  if (const char* e = decode_desc_error(d)) return fail(KVP_ERR_INVALID_ARG, "%s: %s", fn, e);
  if (variant_of(d) != var) {
    if (var == Variant::Int8) return fail(KVP_ERR_INVALID_ARG, "%s: desc->kv_dtype must be KVP_INT8", fn);
    if (var == Variant::Int4) return fail(KVP_ERR_INVALID_ARG, "%s: desc->kv_dtype must be KVP_INT4", fn);
    if (d->kv_dtype == KVP_INT4) return fail(KVP_ERR_INVALID_ARG, "%s: use paged_decode_attention_int4 for INT4 pools", fn);
    if (var == Variant::Mla) return fail(KVP_ERR_INVALID_ARG, "%s: MLA needs n_kv == 1 and d_v < d_k", fn);
    if (d->kv_dtype == KVP_INT8) return fail(KVP_ERR_INVALID_ARG, "%s: use paged_decode_attention_int8 for INT8 pools", fn);
    return fail(KVP_ERR_INVALID_ARG, "%s: n_kv == 1 with d_v != d_k is the MLA layout; use paged_decode_attention_mla", fn);
  }
  if (d->B == 0) return ok();
  if (!q || !k || !block_table || !context_lens || !out) return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (var != Variant::Mla && !v) return fail(KVP_ERR_INVALID_ARG, "%s: v pool is NULL", fn);
  if (quant_variant(var) && (!ks || !vs)) return fail(KVP_ERR_INVALID_ARG, "%s: NULL scale array", fn);
  if (quant_variant(var) && (!aligned(ks, 4) || !aligned(vs, 4)))
    return fail(KVP_ERR_INVALID_ARG, "%s: scale arrays must be 4-byte aligned", fn);
  if (var == Variant::Int4) {
    if (!sink || sink->n < 0 || sink->n > pkv::kMaxSink)
      return fail(KVP_ERR_INVALID_ARG, "%s: n_sink must be in [0, %d]", fn, pkv::kMaxSink);
    if (sink->n > 0 && (!sink->k || !sink->v || !aligned(sink->k, 16) || !aligned(sink->v, 16)))
      return fail(KVP_ERR_INVALID_ARG, "%s: sink rows NULL or not 16-byte aligned", fn);
    if (app) return fail(KVP_ERR_UNSUPPORTED, "%s: INT4 pools decode through paged_decode_attention_int4", fn);
  }
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(KVP_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k, 16) || (v && !aligned(v, 16)))
    return fail(KVP_ERR_INVALID_ARG, "%s: q, out and pools must be 16-byte aligned", fn);
  if (!aligned(block_table, 4) || !aligned(context_lens, 4))
    return fail(KVP_ERR_INVALID_ARG, "%s: tables must be 4-byte aligned", fn);
  if (d->B > 65535 || d->n_kv > 65535) return fail(KVP_ERR_UNSUPPORTED, "%s: B and n_kv must be <= 65535", fn);

  const int g = d->n_h / d->n_kv;
  const bool q_bf16 = d->q_dtype == KVP_BF16;
  if (var == Variant::Float) {
    if (d->kv_dtype != d->q_dtype)
      return fail(KVP_ERR_UNSUPPORTED, "%s: q and the pools must have the same dtype", fn);
    const pkv::KV kv = d->kv_dtype == KVP_BF16 ? pkv::KV::BF16 : pkv::KV::F32;
    if (!pkv::gqa_supported(kv, q_bf16, d->d_k, d->d_v, g))
      return fail(KVP_ERR_UNSUPPORTED, "%s: no kernel for dtype %d, d_k %d, d_v %d, g %d", fn,
                  (int)d->kv_dtype, d->d_k, d->d_v, g);
  } else if (var == Variant::Int8) {
    if (!pkv::gqa_supported(pkv::KV::INT8, q_bf16, d->d_k, d->d_v, g))
      return fail(KVP_ERR_UNSUPPORTED, "%s: no INT8 kernel for q dtype %d, d_k %d, d_v %d, g %d", fn,
                  (int)d->q_dtype, d->d_k, d->d_v, g);
  } else if (var == Variant::Int4) {
    if (!pkv::gqa_supported(pkv::KV::INT4, q_bf16, d->d_k, d->d_v, g) || d->n_kv % 2)
      return fail(KVP_ERR_UNSUPPORTED, "%s: INT4 needs bf16 q, d_k = d_v = 128, g in {4, 8, 16} and even n_kv", fn);
    if (d->window > 0) return fail(KVP_ERR_UNSUPPORTED, "%s: no sliding window on INT4 pools", fn);
  } else {
    if (d->kv_dtype != KVP_BF16 || !q_bf16 || !pkv::mla_supported(d->d_k, d->d_v, d->n_h, d->block_size))
      return fail(KVP_ERR_UNSUPPORTED, "%s: no MLA kernel for n_h %d, d_k %d, d_v %d, block %d", fn,
                  d->n_h, d->d_k, d->d_v, d->block_size);
  }

  if (d->window > 0) {
    if (var == Variant::Mla || !pkv::gqa_ring_supported(var == Variant::Int8 ? pkv::KV::INT8 : pkv::KV::BF16, q_bf16,
                                                         d->d_k, d->d_v, g) ||
        (var == Variant::Float && d->kv_dtype != KVP_BF16))
      return fail(KVP_ERR_UNSUPPORTED, "%s: a sliding window needs bf16 or INT8 pools with g in {4, 8, 16} and d in {64, 128}", fn);
  }
  if (validate_mode()) {
    int64_t nb;
    if (app) {
      nb = app->pool->desc.num_blocks;
    } else {
      const size_t bsz = (size_t)d->block_size * d->n_kv;
      nb = blocks_reachable(k, bsz * row_bytes(d->kv_dtype, d->d_k));
      if (var != Variant::Mla) {
        const int64_t nv = blocks_reachable(v, bsz * row_bytes(d->kv_dtype, d->d_v));
        if (nv < nb) nb = nv;
      }
      if (quant_variant(var)) {
        const int64_t ns = std::min(blocks_reachable(ks, bsz * 4), blocks_reachable(vs, bsz * 4));
        if (ns < nb) nb = ns;
      }
    }
    const kvp_status vs_rc = check_tables(fn, block_table, context_lens, d, nb, stream);
    if (vs_rc != KVP_OK) return vs_rc;
  }

  // Append: the bf16 and INT8 LDS-ring kernels write the new rows themselves
  // (one launch; INT8 quantizes them on the way); every other kernel gets
  // them from the cache kernel first.
  const bool fused_append =
      app && q_bf16 &&
      ((var == Variant::Float && d->kv_dtype == KVP_BF16 &&
        pkv::gqa_ring_supported(pkv::KV::BF16, true, d->d_k, d->d_v, g)) ||
       (var == Variant::Int8 && pkv::gqa_ring_supported(pkv::KV::INT8, true, d->d_k, d->d_v, g)) ||
       var == Variant::Mla);
  if (app && !fused_append) {
    if (!aligned(app->k_new, 4) || (app->v_new && !aligned(app->v_new, 4)))
      return fail(KVP_ERR_INVALID_ARG, "%s: k_new and v_new must be 4-byte aligned", fn);
    pkv::SlotSource src{};
    src.block_table = block_table;
    src.context_lens = context_lens;
    src.max_blocks_per_seq = d->max_blocks_per_seq;
    src.block_shift = log2i(d->block_size);
    const kvp_status rc = write_rows(app->pool, app->k_new, app->v_new, d->q_dtype, src, d->B, stream, fn);
    if (rc != KVP_OK) return rc;
  }

  if (var == Variant::Mla) return launch_mla(fn, q, k, block_table, context_lens, scale, out, d,
                                             workspace, workspace_bytes, stream,
                                             fused_append ? app->k_new : nullptr);
  const kvp_decode_desc pdesc = planning_desc(d);
  const kvp_decode_desc* const dd = d;
  d = &pdesc;                                     // planning from here on (validation is done)
  const int gr = granule(var);
  if (d->split_tokens > 0 && (d->split_tokens % gr || d->split_tokens > max_split(d, var)))
    return fail(KVP_ERR_INVALID_ARG, "%s: split_tokens must be a multiple of %d and <= %d", fn, gr,
                max_split(d, var));
  const int32_t split = plan_split(d, var);
  const int32_t ns = num_splits_of(d, split);
  const size_t need = workspace_for(d, var);
  if (need > 0) {
    if (!workspace) return fail(KVP_ERR_INVALID_ARG, "%s: workspace of %zu bytes required", fn, need);
    if (workspace_bytes < need)
      return fail(KVP_ERR_INVALID_ARG, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(KVP_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  }
  // the shared prefix (plain calls only: an append runs without it)
  const PrefixPlan pp = app ? PrefixPlan{} : prefix_plan(d, var);
  const int32_t sw = pp.tokens ? pp.stream : stream_wgs(d, var);
  if (sw == 0 && ns > 1024)
    return fail(KVP_ERR_UNSUPPORTED, "%s: more than 1024 context splits (raise split_tokens)", fn);

  pkv::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = var == Variant::Mla ? k : v;
  p.k_scale = ks;
  p.v_scale = vs;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  if (sw > 0) {
    const StreamWorkspace sws = stream_workspace(d, sw, pp.pieces(d));
    uint8_t* w = static_cast<uint8_t*>(workspace);
    p.part_o = reinterpret_cast<float*>(w);
    p.part_ml = reinterpret_cast<float*>(w + sws.o_bytes);
    p.seq_meta = reinterpret_cast<int32_t*>(w + sws.o_bytes + sws.ml_bytes);
    p.stream_wgs = sw;
    p.prefix_tokens = pp.tokens;
    p.prefix_chunk = pp.chunk;
    p.prefix_wgs = pp.wgs;
  } else if (need > 0) {
    const size_t rows = (size_t)d->B * d->n_h * ns;
    // [part_o][part_ml]
    uint8_t* w = static_cast<uint8_t*>(workspace);
    const size_t o_bytes = round_up(rows * d->d_v * sizeof(float), 256);
    p.part_o = reinterpret_cast<float*>(w);
    p.part_ml = reinterpret_cast<float*>(w + o_bytes);
  }
  p.scale = scale;
  p.B = d->B;
  p.n_h = d->n_h;
  p.n_kv = d->n_kv;
  p.d_k = d->d_k;
  p.d_v = d->d_v;
  p.block_shift = log2i(d->block_size);
  p.max_blocks_per_seq = d->max_blocks_per_seq;
  p.split_tokens = split;
  p.num_splits = ns;
  p.q_bf16 = q_bf16;
  p.kv = var == Variant::Int4   ? pkv::KV::INT4
         : var == Variant::Int8 ? pkv::KV::INT8
                                : (d->kv_dtype == KVP_BF16 ? pkv::KV::BF16 : pkv::KV::F32);
  if (sink) {
    p.sink_k = sink->k;
    p.sink_v = sink->v;
    p.n_sink = sink->n;
  }
  p.window = dd->window;
  if (fused_append) {
    p.k_new = app->k_new;
    p.v_new = app->v_new;
  }
  // Ragged INT8 batches: launch only the splits that exist (grid from the
  // host's total, which only sizes it: the kernel covers every unit whatever
  // that total says).
  if (sw == 0 && ns > 1 && compact_ok(d, var)) {
    int64_t units = d->total_context_len / split + d->B;
    if (units > (int64_t)d->B * ns) units = (int64_t)d->B * ns;
    if (units > 65535) units = 65535;
    p.compact_units = (int32_t)units;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(pkv::launch_decode_gqa(p, st), fn);
}

}  // namespace

extern "C" {

kvp_status reshape_and_cache(kvp_pool* pool, const void* k_new, const void* v_new,
                             kvp_dtype in_dtype, const int64_t* slot_mapping, int64_t num_tokens,
                             void* stream) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "reshape_and_cache: pool is NULL");
  if (num_tokens < 0) return fail(KVP_ERR_INVALID_ARG, "reshape_and_cache: num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!slot_mapping) return fail(KVP_ERR_INVALID_ARG, "reshape_and_cache: NULL pointer");
  pkv::SlotSource src{};
  src.slots = slot_mapping;
  return write_rows(pool, k_new, v_new, in_dtype, src, num_tokens, stream, "reshape_and_cache");
}

size_t paged_decode_workspace_size(const kvp_decode_desc* desc) {
  if (decode_desc_error(desc)) return 0;
  const kvp_decode_desc pd = planning_desc(desc);
  return workspace_for(&pd, variant_of(desc));
}

int32_t paged_decode_split_tokens(const kvp_decode_desc* desc_in) {
  if (decode_desc_error(desc_in)) return 0;
  const kvp_decode_desc pd = planning_desc(desc_in);
  const kvp_decode_desc* desc = &pd;
  if (variant_of(desc) == Variant::Mla) return pkv::kMlaTileTokens;
  const int32_t sw = stream_wgs(desc, variant_of(desc));
  if (sw > 0) {
    // stream grid: the tokens of one workgroup's range, by the hint
    const int64_t t = (desc->total_context_len + 15 * (int64_t)desc->B + sw - 1) / sw;
    return (int32_t)(t < 16 ? 16 : (t + 15) / 16 * 16);
  }
  return plan_split(desc, variant_of(desc));
}

int32_t paged_decode_mla_workgroups(const kvp_decode_desc* desc) {
  if (decode_desc_error(desc) || variant_of(desc) != Variant::Mla) return 0;
  return mla_workgroups(desc);
}

kvp_status paged_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* context_lens,
                                  float scale, void* out, const kvp_decode_desc* desc,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(Variant::Float, "paged_decode_attention", q, k_pool, v_pool, nullptr,
                       nullptr, block_table, context_lens, scale, out, desc, workspace,
                       workspace_bytes, stream);
}

kvp_status paged_decode_attention_int8(const void* q, const int8_t* k_codes, const float* k_scale,
                                       const int8_t* v_codes, const float* v_scale,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       float scale, void* out, const kvp_decode_desc* desc,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(Variant::Int8, "paged_decode_attention_int8", q, k_codes, v_codes, k_scale,
                       v_scale, block_table, context_lens, scale, out, desc, workspace,
                       workspace_bytes, stream);
}

kvp_status paged_decode_attention_int4(const void* q, const uint8_t* k_codes, const float* k_scale,
                                       const uint8_t* v_codes, const float* v_scale, const void* sink_k,
                                       const void* sink_v, int32_t n_sink, const int32_t* block_table,
                                       const int32_t* context_lens, float scale, void* out,
                                       const kvp_decode_desc* desc, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  const SinkRows sink{sink_k, sink_v, n_sink};
  return decode_common(Variant::Int4, "paged_decode_attention_int4", q, k_codes, v_codes, k_scale, v_scale,
                       block_table, context_lens, scale, out, desc, workspace, workspace_bytes, stream, nullptr,
                       &sink);
}

kvp_status paged_decode_attention_mla(const void* q, const void* latent_pool,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      float scale, void* out, const kvp_decode_desc* desc,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(Variant::Mla, "paged_decode_attention_mla", q, latent_pool, latent_pool,
                       nullptr, nullptr, block_table, context_lens, scale, out, desc, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"

namespace {

kvp_status append_impl(const char* fn, kvp_pool* pool, const void* q, const void* k_new,
                       const void* v_new, const int32_t* block_table, const int32_t* context_lens,
                       float scale, void* out, const kvp_decode_desc* desc, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (const char* e = decode_desc_error(desc)) return fail(KVP_ERR_INVALID_ARG, "%s: %s", fn, e);
  const kvp_pool_desc& pd = pool->desc;
  if (pd.n_kv != desc->n_kv || pd.d_k != desc->d_k || pd.d_v != desc->d_v ||
      pd.block_size != desc->block_size || pd.dtype != desc->kv_dtype)
    return fail(KVP_ERR_INVALID_ARG, "%s: the pool's n_kv, d_k, d_v, block_size or dtype differs from desc", fn);
  const Variant var = variant_of(desc);
  if (var == Variant::Int4)
    return fail(KVP_ERR_UNSUPPORTED, "%s: INT4 pools decode through paged_decode_attention_int4 "
                "(write the rows with reshape_and_cache)", fn);
  if (pd.latent != (var == Variant::Mla))
    return fail(KVP_ERR_INVALID_ARG, "%s: a latent pool goes with an MLA description and only with one", fn);
  if (desc->B == 0) return ok();
  if (!k_new || (!pd.latent && !v_new)) return fail(KVP_ERR_INVALID_ARG, "%s: NULL k_new or v_new", fn);
  if (!aligned(k_new, 16) || (!pd.latent && !aligned(v_new, 16)))
    return fail(KVP_ERR_INVALID_ARG, "%s: k_new and v_new must be 16-byte aligned", fn);
  kvp_pool_view v;
  kv_pool_view_get(pool, &v);
  const AppendRows app{pool, k_new, pd.latent ? nullptr : v_new};
  if (var == Variant::Int8)
    return decode_common(var, fn, q, v.k, v.v, v.k_scale, v.v_scale, block_table, context_lens, scale,
                         out, desc, workspace, workspace_bytes, stream, &app);
  if (var == Variant::Mla)
    return decode_common(var, fn, q, v.k, v.k, nullptr, nullptr, block_table, context_lens, scale, out,
                         desc, workspace, workspace_bytes, stream, &app);
  return decode_common(var, fn, q, v.k, v.v, nullptr, nullptr, block_table, context_lens, scale, out,
                       desc, workspace, workspace_bytes, stream, &app);
}

// ---- static scratch of paged_decode_attention_append_noalloc
//
// One array per device, held from the library's load until the process
// ends.  Host code never uses the array's name as an address (on the host it
// names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kvp_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(KVP_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!ptr || !aligned(ptr, 256)) return fail(KVP_ERR_HIP, "%s: scratch address %p is not usable", fn, ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVP_OK;
}

}  // namespace

extern "C" {

kvp_status paged_decode_attention_append(kvp_pool* pool, const void* q, const void* k_new,
                                         const void* v_new, const int32_t* block_table,
                                         const int32_t* context_lens, float scale, void* out,
                                         const kvp_decode_desc* desc, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return append_impl("paged_decode_attention_append", pool, q, k_new, v_new, block_table, context_lens,
                     scale, out, desc, workspace, workspace_bytes, stream);
}

kvp_status paged_decode_attention_append_noalloc(kvp_pool* pool, const void* q, const void* k_new,
                                                 const void* v_new, const int32_t* block_table,
                                                 const int32_t* context_lens, float scale, void* out,
                                                 const kvp_decode_desc* desc, void* stream) {
  const char* fn = "paged_decode_attention_append_noalloc";
  if (const char* e = decode_desc_error(desc)) return fail(KVP_ERR_INVALID_ARG, "%s: %s", fn, e);
  const kvp_decode_desc pd = planning_desc(desc);
  const size_t need = workspace_for(&pd, variant_of(desc));
  if (need > kScratchBytes)
    return fail(KVP_ERR_UNSUPPORTED,
                "%s: the call needs %zu bytes of scratch, the static buffer holds %zu "
                "(use paged_decode_attention_append with a workspace)", fn, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const kvp_status rc = scratch_address(fn, &ws);
    if (rc != KVP_OK) return rc;
  }
  return append_impl(fn, pool, q, k_new, v_new, block_table, context_lens, scale, out, desc, ws,
                     need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"

namespace {

// The pool's regions block by block: K, V, K scales, V scales.
pkv::PoolRegions pool_regions(const kvp_pool* pool) {
  pkv::PoolRegions r{};
  const kvp_pool_desc& d = pool->desc;
  const PoolLayout& L = pool->layout;
  const int64_t slots_per_block = d.block_size;
  const size_t eb = dtype_bytes(d.dtype);
  r.num_blocks = d.num_blocks;
  r.base[0] = pool->base + L.k_off;
  r.bytes[0] = slots_per_block * d.n_kv * d.d_k * (int64_t)eb;
  if (!d.latent) {
    r.base[1] = pool->base + L.v_off;
    r.bytes[1] = slots_per_block * d.n_kv * d.d_v * (int64_t)eb;
  }
  if (d.dtype == KVP_INT8) {
    r.base[2] = pool->base + L.ks_off;
    r.bytes[2] = slots_per_block * d.n_kv * 4;
    if (!d.latent) {
      r.base[3] = pool->base + L.vs_off;
      r.bytes[3] = slots_per_block * d.n_kv * 4;
    }
  }
  return r;
}

int64_t regions_total(const pkv::PoolRegions& r) { return r.bytes[0] + r.bytes[1] + r.bytes[2] + r.bytes[3]; }

}  // namespace

extern "C" {

kvp_status paged_prefill_attention(const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* start_pos,
                                   const int32_t* chunk_lens, float scale, void* out,
                                   const kvp_decode_desc* d, int32_t max_chunk, void* stream) {
  const char* fn = "paged_prefill_attention";
  if (const char* e = decode_desc_error(d)) return fail(KVP_ERR_INVALID_ARG, "%s: %s", fn, e);
  if (max_chunk < 0) return fail(KVP_ERR_INVALID_ARG, "%s: max_chunk < 0", fn);
  if (d->B == 0 || max_chunk == 0) return ok();
  if (!q || !k_pool || !v_pool || !block_table || !start_pos || !chunk_lens || !out)
    return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(KVP_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_table, 4) || !aligned(start_pos, 4) || !aligned(chunk_lens, 4))
    return fail(KVP_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const int g = d->n_h / d->n_kv;
  if (d->q_dtype != KVP_BF16 || d->kv_dtype != KVP_BF16 || !pkv::prefill_supported(d->d_k, d->d_v, g))
    return fail(KVP_ERR_UNSUPPORTED, "%s: bf16 with d_k = d_v = 128 and g in {1, 2, 4, 8, 16} only", fn);
  if (d->B > 65535 || d->n_kv > 65535 || max_chunk > 65535 * 8)
    return fail(KVP_ERR_UNSUPPORTED, "%s: B, n_kv or max_chunk too large", fn);
  if (validate_mode()) {
    // the positions each chunk reaches, checked like a decode of length start + chunk
    std::vector<int32_t> sp(d->B), cl(d->B);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(sp.data(), start_pos, sp.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(cl.data(), chunk_lens, cl.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e, fn);
    for (int32_t b = 0; b < d->B; ++b)
      if (sp[b] < 0 || cl[b] < 0 || cl[b] > max_chunk || (int64_t)sp[b] + cl[b] > d->max_context_len)
        return fail(KVP_ERR_INVALID_ARG, "%s: start_pos[%d] = %d, chunk_lens[%d] = %d out of range", fn, b, sp[b], b,
                    cl[b]);
  }
  pkv::PrefillParams p{};
  p.q = q;
  p.k = k_pool;
  p.v = v_pool;
  p.block_table = block_table;
  p.start_pos = start_pos;
  p.chunk_lens = chunk_lens;
  p.out = out;
  p.scale = scale;
  p.B = d->B;
  p.max_chunk = max_chunk;
  p.n_h = d->n_h;
  p.n_kv = d->n_kv;
  p.d_k = d->d_k;
  p.d_v = d->d_v;
  p.block_shift = log2i(d->block_size);
  p.max_blocks_per_seq = d->max_blocks_per_seq;
  return hip_status(pkv::launch_prefill_paged(p, static_cast<hipStream_t>(stream)), fn);
}

kvp_status kvp_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || bytes % 16 || workgroups < 0)
    return fail(KVP_ERR_INVALID_ARG, "kvp_stream_read: NULL or misaligned buffer, or bytes not a multiple of 16");
  const int wg = workgroups > 0 ? workgroups : 2 * device_cus();
  return hip_status(pkv::launch_stream_read(buf, (int64_t)bytes, sink, wg, static_cast<hipStream_t>(stream)),
                    "kvp_stream_read");
}

kvp_status kvp_mfma_peak(float* sink, int32_t workgroups, int32_t iterations, void* stream) {
  if (!sink || !aligned(sink, 4) || workgroups < 0 || iterations <= 0)
    return fail(KVP_ERR_INVALID_ARG, "kvp_mfma_peak: NULL or misaligned sink, workgroups < 0 or iterations <= 0");
  const int wg = workgroups > 0 ? workgroups : 4 * device_cus();
  return hip_status(pkv::launch_mfma_peak(sink, wg, iterations, static_cast<hipStream_t>(stream)), "kvp_mfma_peak");
}

size_t kv_pool_block_bytes(const kvp_pool* pool) {
  if (!pool) return 0;
  return (size_t)regions_total(pool_regions(pool));
}

kvp_status copy_blocks(kvp_pool* pool, const int32_t* pairs, int64_t num_pairs, void* stream) {
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "copy_blocks: pool is NULL");
  if (num_pairs < 0) return fail(KVP_ERR_INVALID_ARG, "copy_blocks: num_pairs < 0");
  if (num_pairs == 0) return ok();
  if (!pairs || !aligned(pairs, 4)) return fail(KVP_ERR_INVALID_ARG, "copy_blocks: pairs NULL or misaligned");
  if (num_pairs > 0x7fffffff) return fail(KVP_ERR_UNSUPPORTED, "copy_blocks: too many pairs");
  return hip_status(pkv::launch_copy_blocks(pool_regions(pool), pairs, num_pairs, static_cast<hipStream_t>(stream)),
                    "copy_blocks");
}

kvp_status swap_out_blocks(const kvp_pool* pool, const int32_t* blocks, int64_t n, void* staging, void* host_dst,
                           void* stream) {
  const char* fn = "swap_out_blocks";
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (n < 0) return fail(KVP_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (n == 0) return ok();
  if (!blocks || !staging || !host_dst) return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned(blocks, 4) || !aligned(staging, 16)) return fail(KVP_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  if (n > 0x7fffffff) return fail(KVP_ERR_UNSUPPORTED, "%s: too many blocks", fn);
  const pkv::PoolRegions r = pool_regions(pool);
  const int64_t total = regions_total(r);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = pkv::launch_stage_blocks(r, blocks, n, static_cast<uint8_t*>(staging), total, true, st);
  if (e == hipSuccess) e = hipMemcpyAsync(host_dst, staging, (size_t)(n * total), hipMemcpyDeviceToHost, st);
  return hip_status(e, fn);
}

kvp_status swap_in_blocks(kvp_pool* pool, const int32_t* blocks, int64_t n, void* staging, const void* host_src,
                          void* stream) {
  const char* fn = "swap_in_blocks";
  if (!pool) return fail(KVP_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (n < 0) return fail(KVP_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (n == 0) return ok();
  if (!blocks || !staging || !host_src) return fail(KVP_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned(blocks, 4) || !aligned(staging, 16)) return fail(KVP_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  if (n > 0x7fffffff) return fail(KVP_ERR_UNSUPPORTED, "%s: too many blocks", fn);
  const pkv::PoolRegions r = pool_regions(pool);
  const int64_t total = regions_total(r);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(staging, host_src, (size_t)(n * total), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = pkv::launch_stage_blocks(r, blocks, n, static_cast<uint8_t*>(staging), total, false, st);
  return hip_status(e, fn);
}

kvp_status paged_gather(const void* pool, int32_t elem_bytes, int32_t block_size, int32_t n_kv,
                        int32_t d, const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t B, int32_t max_context_len, void* out,
                        void* stream) {
  if (B < 0 || max_context_len < 0) return fail(KVP_ERR_INVALID_ARG, "paged_gather: negative size");
  if (B == 0 || max_context_len == 0) return ok();
  if (!pool || !block_table || !context_lens || !out) return fail(KVP_ERR_INVALID_ARG, "paged_gather: NULL pointer");
  if (!(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4))
    return fail(KVP_ERR_INVALID_ARG, "paged_gather: elem_bytes must be 1, 2 or 4");
  if (!is_pow2(block_size) || block_size > 256)
    return fail(KVP_ERR_INVALID_ARG, "paged_gather: block_size must be a power of two in [1, 256]");
  if (n_kv <= 0 || d <= 0 || max_blocks_per_seq <= 0) return fail(KVP_ERR_INVALID_ARG, "paged_gather: bad shape");
  const int64_t row_bytes = (int64_t)n_kv * d * elem_bytes;
  if (row_bytes % 4) return fail(KVP_ERR_INVALID_ARG, "paged_gather: row bytes must be a multiple of 4");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(KVP_ERR_INVALID_ARG, "paged_gather: max_context_len exceeds the table");
  if (B > 65535) return fail(KVP_ERR_UNSUPPORTED, "paged_gather: B must be <= 65535");
  return hip_status(pkv::launch_gather(pool, row_bytes, log2i(block_size), block_table,
                                       max_blocks_per_seq, context_lens, B, max_context_len, out,
                                       static_cast<hipStream_t>(stream)),
                    "paged_gather");
}

kvp_status paged_decode_validate(const int32_t* block_table, const int32_t* context_lens,
                                 const kvp_decode_desc* desc, int64_t num_blocks, void* stream) {
  if (const char* e = decode_desc_error(desc)) return fail(KVP_ERR_INVALID_ARG, "paged_decode_validate: %s", e);
  return check_tables("paged_decode_validate", block_table, context_lens, desc, num_blocks, stream);
}

}  // extern "C"
