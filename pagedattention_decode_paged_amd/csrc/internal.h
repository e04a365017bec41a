// Internal interface between the C-ABI host layer (pagedkv_api.cpp) and the
// kernel translation units.  Launchers return hipError_t; the host layer has
// already validated every shape and pointer they receive.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// The per-thread message kvp_last_error() returns (set by every entry point).
void set_last_error(const char* msg);

// ---------------------------------------------------------------- cache ops
hipError_t launch_slot_mapping(const int32_t* block_table, int32_t max_blocks_per_seq,
                               int32_t block_shift, const int32_t* seq_ids,
                               const int32_t* positions, int64_t num_tokens,
                               int64_t* slots, hipStream_t stream);

// Where the rows of the new tokens go: an explicit slot per token, or (slots
// null) one token per sequence t at position context_lens[t] - 1, its slot
// read from the block table.  A negative slot (or a position or block the
// table does not map) skips the token.
struct SlotSource {
  const int64_t* slots;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t max_blocks_per_seq;
  int32_t block_shift;
};

__device__ __forceinline__ int64_t slot_of(const SlotSource& s, int64_t t) {
  if (s.slots) return s.slots[t];
  const int32_t pos = s.context_lens[t] - 1;
  if (pos < 0) return -1;
  const int32_t lb = pos >> s.block_shift;
  if (lb >= s.max_blocks_per_seq) return -1;
  const int32_t phys = s.block_table[t * s.max_blocks_per_seq + lb];
  if (phys < 0) return -1;
  return ((int64_t)phys << s.block_shift) + (pos & ((1 << s.block_shift) - 1));
}

// Bit copy of the K rows (and V rows when v_pool is not null) of num_tokens
// tokens into their slots, one launch (row bytes % 4 == 0).
hipError_t launch_cache_copy(void* k_pool, const void* k_src, int64_t k_row_bytes, void* v_pool,
                             const void* v_src, int64_t v_row_bytes, const SlotSource& slots,
                             int64_t num_tokens, hipStream_t stream);

// Quantize-on-write of K and V, one launch: src rows [num_tokens, n_kv, d]
// (f32 or bf16 bits), codes [slots, n_kv, d] int8, scales
// [num_blocks, n_kv, block_size] f32 (block_size = 1 << block_shift).
hipError_t launch_cache_quant_int8(int8_t* k_codes, float* k_scales, const void* k_src, int32_t d_k,
                                   int8_t* v_codes, float* v_scales, const void* v_src, int32_t d_v,
                                   bool src_bf16, const SlotSource& slots, int64_t num_tokens,
                                   int32_t n_kv, int32_t block_shift, hipStream_t stream);

// Block copies over up to four regions of a pool (K, V, K scales, V
// scales): region r of block b is base[r] + b * bytes[r] (bytes[r] a
// multiple of 4, 0 for an absent region).
struct PoolRegions {
  uint8_t* base[4];
  int64_t bytes[4];
  int64_t num_blocks;
};
// pairs [n, 2] (src, dst): block src -> block dst in every region.
hipError_t launch_copy_blocks(const PoolRegions& r, const int32_t* pairs, int64_t n, hipStream_t stream);
// blocks [n]: block blocks[i] <-> staging + i * total, regions in order
// (to_staging: gather, else scatter).
hipError_t launch_stage_blocks(const PoolRegions& r, const int32_t* blocks, int64_t n, uint8_t* staging,
                               int64_t total, bool to_staging, hipStream_t stream);

// INT4 (two codes per byte, element 2i in the low nibble of byte i): codes
// [slots, n_kv, d / 2] uint8, scales as for INT8.
hipError_t launch_cache_quant_int4(uint8_t* k_codes, float* k_scales, const void* k_src, int32_t d_k,
                                   uint8_t* v_codes, float* v_scales, const void* v_src, int32_t d_v,
                                   bool src_bf16, const SlotSource& slots, int64_t num_tokens,
                                   int32_t n_kv, int32_t block_shift, hipStream_t stream);

// Streaming read of bytes (16-byte aligned) with workgroups workgroups of
// 256 lanes (the read-bandwidth ceiling probe).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);

hipError_t launch_gather(const void* pool, int64_t row_bytes, int32_t block_shift,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t B, int32_t max_context_len,
                         void* out, hipStream_t stream);

// ---------------------------------------------------------------- decode
enum class KV { F32, BF16, INT8, INT4 };

struct DecodeParams {
  const void* q;
  const void* k;            // K values or codes
  const void* v;            // V values or codes (== k for latent)
  const float* k_scale;     // INT8 only
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  float* part_o;            // [B, n_h, num_splits, d_v] (num_splits > 1)
  float* part_ml;           // [B, n_h, num_splits, 2]  (max, sum)
  float scale;
  int32_t B, n_h, n_kv, d_k, d_v;
  int32_t block_shift;      // log2(block_size)
  int32_t max_blocks_per_seq;
  int32_t split_tokens;     // multiple of the kernel's per-split granule
  int32_t num_splits;
  bool q_bf16;
  KV kv;
  // MLA, and the LDS-ring kernel's stream grid: persistent workgroups per
  // head group (MLA), and the per-sequence record of which workgroups hold a
  // sequence ([B, 2], in the workspace).
  int32_t workgroups;
  int32_t* seq_meta;
  // Append (bf16 LDS-ring kernel only; null otherwise): the new token's K and
  // V rows [B, n_kv, d], written by the kernel to position context_lens[b] - 1
  // of each sequence (k and v above then point at writable pools).
  const void* k_new;
  const void* v_new;
  // LDS-ring kernel, ragged batches (B <= kCompactMaxB; at most one of the
  // two is set).  Both 0: grid (KV head group, sequence, split).
  // compact_units > 0 (INT8 pools): grid (KV head group, compact_units) over
  // the splits that exist, each workgroup looping over units blockIdx.y +
  // k * compact_units until all are done.  stream_wgs > 0 (bf16 pools): grid
  // (KV head group, stream_wgs), the batch's tokens (each sequence padded to
  // a multiple of 16) cut into stream_wgs equal ranges, one per workgroup;
  // partials go to piece j + b (part_o [stream_wgs + B, n_h, d_v], part_ml
  // [stream_wgs + B, n_h, 2]) and seq_meta [B, 2] receives each sequence's
  // first and last workgroup.
  int32_t compact_units;
  int32_t stream_wgs;
  // Shared prefix (bf16 LDS-ring kernel with two KV heads per workgroup,
  // stream grid only; prefix_tokens = 0: off).  Tokens [0, prefix_tokens) of
  // every sequence are handled by prefix_wgs extra workgroups per KV-head
  // group (grid.y = stream_wgs + prefix_wgs, the prefix ones first), each
  // taking one KV head, one chunk of prefix_chunk tokens and a group of
  // sequences: the chunk's rows of the longest sequence are read once and
  // serve every sequence whose block-table entries over the chunk are the
  // same blocks (checked on the device); any other sequence's chunk runs on
  // its own blocks in the same workgroup.  The stream workgroups take
  // tokens [prefix_tokens, ctx) of each sequence.  Prefix partials of chunk
  // c and sequence b go to piece stream_wgs + B + c * B + b.
  int32_t prefix_tokens;
  int32_t prefix_chunk;
  int32_t prefix_wgs;
  // Sliding window (LDS-ring kernel only; 0: the whole context): a sequence
  // of ctx tokens attends to positions [max(0, ctx - window), ctx).  The
  // kernels start reading at that position rounded down to a multiple of 16
  // (whole DMA rows), mask the positions below it, and skip every block
  // before it.
  int32_t window;
  // INT4 pools (LDS-ring kernel): the first n_sink positions of each
  // sequence are taken from unquantized rows, sink_k / sink_v bf16
  // [B, n_sink, n_kv, d] (null when n_sink is 0).
  const void* sink_k;
  const void* sink_v;
  int32_t n_sink;
};

// First attended position of a sequence of ctx tokens, and the position the
// kernels start reading at (a multiple of 16).
__device__ __forceinline__ int window_lo(const DecodeParams& p, int ctx) {
  return p.window > 0 ? max(ctx - p.window, 0) : 0;
}
__device__ __forceinline__ int window_a0(const DecodeParams& p, int ctx) { return window_lo(p, ctx) & ~15; }

// End of a sequence's part in the shared prefix of S tokens (S > 0, a
// multiple of 64): S for a sequence that reaches it, else its tokens up to
// the last boundary of a whole block and of 16 tokens.  A partly filled
// last block is never shared by a block allocator (only full blocks are
// found by prefix caching), so it joins the sequence's own part instead of
// failing the prefix pass's table check; parts start at multiples of 16.
__device__ __forceinline__ int prefix_end(int ctx, int S, int shift) {
  return ctx >= S ? S : ctx & ~((1 << max(shift, 4)) - 1);
}

// Sequences one prefix workgroup serves: four waves of 32 query columns
// (two 16-column matrix-core blocks), g columns per sequence.
constexpr int prefix_seqs_per_wg(int g) { return 4 * (32 / g); }

constexpr int kCompactMaxB = 512;
constexpr int kMaxSink = 64;        // INT4 pools: most unquantized sink positions

// Chunked prefill (bf16, d = 128): q, out [B, max_chunk, n_h, d]; sequence
// b's chunk_lens[b] query tokens sit at positions start_pos[b] + i.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* start_pos;
  const int32_t* chunk_lens;
  void* out;
  float scale;
  int32_t B, max_chunk, n_h, n_kv, d_k, d_v;
  int32_t block_shift;
  int32_t max_blocks_per_seq;
};
bool prefill_supported(int d_k, int d_v, int g);
hipError_t launch_prefill_paged(const PrefillParams& p, hipStream_t stream);

// GQA/MQA/MHA over float, bf16 or INT8 pools: routes the shapes the
// LDS-ring kernel covers there and the others to the general kernels, then
// launches the split reduce.  Returns hipErrorInvalidValue for a
// (d, g, dtype) combination with no instance.
hipError_t launch_decode_gqa(const DecodeParams& p, hipStream_t stream);

// INT8 pools (fused dequant); called by launch_decode_gqa.
bool int8_supported(bool q_bf16, int d_k, int d_v, int g);
hipError_t launch_decode_int8(const DecodeParams& p, int g, hipStream_t stream);

// Absorbed MLA over a bf16 latent pool (MFMA kernel) plus the merge of
// sequences cut across workgroups.
hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t stream);
int mla_head_groups(int n_h);

// bf16 and INT8 GQA with g in {4, 8}, d in {64, 128}: the LDS-ring kernel
// on the matrix cores (decode_gqa_ring.hip).
bool gqa_ring_supported(KV kv, bool q_bf16, int d_k, int d_v, int g);
// KV heads served by one workgroup of that kernel (1, or 2 / 4 when a
// token's rows of adjacent KV heads are moved together); the split planning
// counts work units per group.
int gqa_ring_kv_group(KV kv, bool q_bf16, int d_k, int d_v, int g, int n_kv);
hipError_t launch_decode_gqa_ring(const DecodeParams& p, hipStream_t stream);

// Whether an instance exists (host-side check before launch).
bool gqa_supported(KV kv, bool q_bf16, int d_k, int d_v, int g);
bool mla_supported(int d_k, int d_v, int n_h, int block_size);

// Context tokens each workgroup of the GQA kernel walks per split must be a
// multiple of this.
constexpr int kGqaSplitGranule = 256;

// MLA: context tiles of 32 tokens; every workgroup stages the batch's tile
// prefix in LDS, which bounds the batch.
constexpr int kMlaTileTokens = 32;
constexpr int kMlaHeadsPerGroup = 128;   // heads per MLA workgroup (one head group)
constexpr int kMlaMaxBatch = 4096;

}  // namespace pkv
