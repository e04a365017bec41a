/*
 * pagedkv.h -- C ABI of a paged-KV-cache single-token decode attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * What is computed (page citations name a page by its site; the same five
 * pages are cited throughout the sources):
 *   faulkner -- "LLM 推理底层：KV Cache 显存几何、GQA/MLA 压缩与 PagedAttention 调度"
 *               (blog.faulkner.fun/posts/llm-kv-cache-and-paged-attention)
 *   qwbw     -- "【infra之路】10-PagedAttention 与 KV Cache 管理" (www.qwbw.cn/news/28817)
 *   guijiagi -- KV cache guide (guijiagi.com/posts/kv-cache-guide/)
 *   talentme -- "KV Cache 显存管理全景 ..." (talentme.airsota.com/.../kv-cache-and-paged-attention)
 *   hx       -- "LLM 推理引擎设计：KV Cache、PagedAttention 与连续批处理"
 *               (hx.sn.cn/archives/llm-inference-engine)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument named as device memory must point to memory of
 *   the current HIP device.  Host pointers are named as such.
 * - Work is enqueued on the caller's stream (a hipStream_t passed as
 *   void*; NULL is the null stream) and the call returns without waiting
 *   for it, except where a function says it synchronises.
 * - The library never frees caller memory and never allocates device
 *   memory outside kv_pool_create (storage == NULL).
 * - Errors: argument and shape checks happen on the host before anything
 *   is enqueued; a failing call returns a negative kvp_status, enqueues
 *   nothing and leaves a message for kvp_last_error() (per thread).
 *   Device data that breaks a documented precondition (a block id out of
 *   range, a context longer than the block table covers) is not checked in
 *   the fast path; paged_decode_validate() checks it on request.
 * - Debug mode: with the environment variable PAGEDKV_VALIDATE set to a
 *   value other than "0" (read at every call), each decode entry point
 *   first runs the checks of paged_decode_validate() on its block table
 *   and context lengths (synchronising the stream) and returns their
 *   status without launching anything when they fail.  The pool's block
 *   count is the pool's own (append; any pointer into a pool made by
 *   kv_pool_create) or, for other memory, the blocks that fit between the
 *   pool pointer and the end of its device allocation.
 * - No C++ exception crosses this interface.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVP_OK = 0,
  KVP_ERR_INVALID_ARG = -1,   /* a null pointer, a bad size or a shape mismatch */
  KVP_ERR_OUT_OF_MEMORY = -2, /* the pool could not be allocated */
  KVP_ERR_UNSUPPORTED = -3,   /* a valid shape/type the library has no kernel for */
  KVP_ERR_HIP = -4            /* the HIP runtime reported an error */
} kvp_status;

typedef enum {
  KVP_F32 = 0,   /* IEEE binary32 */
  KVP_BF16 = 1,  /* bfloat16 (top half of binary32), round-to-nearest-even */
  KVP_INT8 = 2,  /* signed 8-bit codes with one fp32 scale per (slot, KV head) */
  KVP_INT4 = 3   /* signed 4-bit codes, two per byte (element 2i in the low
                    nibble of byte i, two's complement), one fp32 scale per
                    (slot, KV head) */
} kvp_dtype;

/* ------------------------------------------------------------------------
 * KV pool
 *
 * A pool of num_blocks physical blocks, each holding block_size token
 * slots (faulkner, section on logical/physical block mapping; qwbw 3.2).
 * Layout, row-major (talentme chapter 3, the NumPy pool class):
 *   K codes/values  [num_blocks, block_size, n_kv, d_k]
 *   V codes/values  [num_blocks, block_size, n_kv, d_v]
 *   K, V scales     [num_blocks, n_kv, block_size] float   (KVP_INT8, KVP_INT4)
 * (KVP_INT4 rows hold d / 2 bytes: two codes per byte.)
 * Slot s is block s / block_size, offset s % block_size.  The scales are
 * paged like the codes (one per slot and KV head); inside a block, one
 * head's scales are adjacent so that a kernel working on one KV head reads
 * them as contiguous runs.  A latent pool
 * (latent = 1, absorbed MLA; faulkner, matrix absorption section) has
 * n_kv = 1 and no V array: the value of a token is the first d_v columns
 * of its K row.  Each region starts 256-byte aligned.
 * ---------------------------------------------------------------------- */
typedef struct kvp_pool kvp_pool;

typedef struct {
  int64_t num_blocks;   /* > 0 */
  int32_t block_size;   /* power of two, 1 ... 256 */
  int32_t n_kv;         /* KV heads, > 0 */
  int32_t d_k;          /* K row width in elements, > 0 */
  int32_t d_v;          /* V row width in elements, > 0 (<= d_k when latent) */
  kvp_dtype dtype;      /* element type of the pool */
  int32_t latent;       /* 1: V aliases K[..., :d_v]; requires n_kv == 1 */
} kvp_pool_desc;

typedef struct {
  void* k;              /* device: K region */
  void* v;              /* device: V region (== k for a latent pool) */
  float* k_scale;       /* device: K scales (KVP_INT8), else NULL */
  float* v_scale;       /* device: V scales (KVP_INT8, not latent), else NULL */
  size_t total_bytes;   /* bytes the pool occupies from k onward */
  kvp_pool_desc desc;
} kvp_pool_view;

/* Bytes of device storage a pool with this description needs (0 if the
 * description is invalid). */
size_t kv_pool_required_bytes(const kvp_pool_desc* desc);

/* Create a pool.  If storage is NULL the library allocates the memory with
 * hipMalloc on the current device and frees it in kv_pool_destroy
 * (KVP_ERR_OUT_OF_MEMORY if that fails -- the analogue of the allocator
 * running out of physical blocks, faulkner allocator code).  Otherwise
 * storage (device, 256-byte aligned, at least kv_pool_required_bytes) is
 * caller-owned and must outlive the pool.  Contents are not initialised. */
kvp_status kv_pool_create(const kvp_pool_desc* desc, void* storage,
                          size_t storage_bytes, kvp_pool** out);

/* Release the handle (and the memory, if the library allocated it).
 * NULL is a no-op. */
void kv_pool_destroy(kvp_pool* pool);

/* Device addresses and shape of a pool. */
kvp_status kv_pool_view_get(const kvp_pool* pool, kvp_pool_view* out);

/* ------------------------------------------------------------------------
 * Slot mapping (faulkner, logical/physical block mapping; talentme
 * chapter 3, the write_kv lookup): for each token t,
 *   slots[t] = block_table[seq_ids[t]][positions[t] / block_size] * block_size
 *              + positions[t] % block_size
 * as int64.  block_table: device int32 [*, max_blocks_per_seq] row-major.
 * seq_ids, positions: device int32 [num_tokens]; slots: device int64
 * [num_tokens].  A negative seq id or position, or a position whose
 * logical block is >= max_blocks_per_seq, or a negative table entry,
 * yields slot -1 (which reshape_and_cache skips).
 * ---------------------------------------------------------------------- */
kvp_status paged_slot_mapping(const int32_t* block_table, int32_t max_blocks_per_seq,
                              int32_t block_size, const int32_t* seq_ids,
                              const int32_t* positions, int64_t num_tokens,
                              int64_t* slots, void* stream);

/* ------------------------------------------------------------------------
 * reshape_and_cache: scatter the K/V rows of new tokens into their slots
 * (talentme chapter 3, write_kv; qwbw 1.2 appends each step's K/V before
 * attending).
 *   k_new: device [num_tokens, n_kv, d_k] of in_dtype, contiguous
 *   v_new: device [num_tokens, n_kv, d_v] of in_dtype (ignored, may be
 *          NULL, for a latent pool)
 *   slot_mapping: device int64 [num_tokens]; a negative slot skips the
 *          token; a slot >= num_blocks * block_size is a precondition
 *          violation.
 * F32 and BF16 pools store the rows bit for bit (in_dtype must equal the
 * pool dtype).  An INT8 pool quantizes on write (guijiagi 4.2): per (token,
 * head) row, scale = fl32(absmax / 127) and code = clamp(rint(fl32(x /
 * scale)), -128, 127) in IEEE binary32 with round-half-to-even; a zero row
 * gets scale 0 and codes 0.  An INT4 pool the same with absmax / 7 and
 * [-8, 7] (the 4-bit branch), packed two per byte.  in_dtype F32 or BF16
 * (widened exactly).
 * Two tokens mapped to one slot race; the result is one of the rows.
 * ---------------------------------------------------------------------- */
kvp_status reshape_and_cache(kvp_pool* pool, const void* k_new, const void* v_new,
                             kvp_dtype in_dtype, const int64_t* slot_mapping,
                             int64_t num_tokens, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention
 *
 * For every sequence b and query head h (faulkner, first section, o_t;
 * qwbw 3.4 walks the block table; faulkner's MHA/GQA/MLA table for head
 * sharing):
 *   kvh = h / (n_h / n_kv)                  (consecutive head groups)
 *   K_j = k_pool[block_table[b][j / bs]][j % bs][kvh]   for 0 <= j < L,
 *   L   = context_lens[b] (the token being decoded included)
 *   out[b][h] = softmax_j(scale * q[b][h] . K_j) weighted sum of V_j
 * Slots at or beyond L are never read.  L == 0 gives a zero output.
 * The result is unique; kernels accumulate in fp32 (online softmax over
 * context splits merged by log-sum-exp), so it matches the exact value to
 * within rounding.
 *
 *   q:   device [B, n_h, d_k], q_dtype      out: device [B, n_h, d_v], q_dtype
 *   block_table: device int32 [B, max_blocks_per_seq]
 *   context_lens: device int32 [B], each in [0, max_context_len]
 *   max_context_len: a host-side upper bound of every context_lens[b]
 *          (used to size the launch without reading device memory);
 *          must be <= max_blocks_per_seq * block_size.
 * Shapes (g = n_h / n_kv, an integer): bf16 and INT8 pools d_k = d_v in
 * {64, 128}, g in {1, 2, 4, 8, 16}; F32 pools d_k = d_v in {32, 64}, g in
 * {1, 2, 4, 8}; others KVP_ERR_UNSUPPORTED.
 *   workspace: device scratch of at least paged_decode_workspace_size()
 *          bytes (may be NULL when that is 0), 256-byte aligned; it holds
 *          the split partials.  Calls that share a workspace must not
 *          overlap (use one stream, or one workspace per stream).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B, n_h, n_kv, d_k, d_v;
  int32_t block_size;          /* power of two */
  int32_t max_blocks_per_seq;
  int32_t max_context_len;     /* host upper bound of context_lens */
  kvp_dtype q_dtype;           /* F32 or BF16; also the output type */
  kvp_dtype kv_dtype;          /* F32, BF16 or INT8 */
  int32_t split_tokens;        /* tokens per context split; 0 = automatic */
  int64_t total_context_len;   /* optional host hint: sum of context_lens
                                  (0 = unknown; then B * max_context_len is
                                  assumed when sizing splits).  For a ragged
                                  batch (B <= 512) on the GQA path with
                                  g in {4, 8, 16}: bf16 pools cut the batch's
                                  tokens into equal ranges, one per
                                  workgroup (one round of workgroups on the
                                  current device); INT8 pools launch only
                                  the context splits that exist, sized to
                                  one round.  A wrong value costs time,
                                  never results. */
  int32_t workgroups;          /* MLA only: persistent workgroups per group
                                  of 128 heads; 0 = one per compute unit of
                                  the current device (at most the number of
                                  32-token context tiles).  Ignored by the
                                  other entry points. */
  int32_t shared_prefix_tokens; /* optional host hint (0 = none): the first
                                  tokens of the sequences are expected to sit
                                  in the same physical blocks (a shared
                                  prompt prefix; hx 4.2, faulkner prefix
                                  caching).  Used by paged_decode_attention on
                                  bf16 pools with d = 128, g in {4, 8, 16}, even
                                  n_kv, B <= 512 and no forced split (other
                                  calls ignore it): the hint, rounded down to
                                  a multiple of 64 and at most
                                  max_context_len, is cut into chunks, and
                                  each chunk's K/V rows are read once for
                                  every sequence whose block-table entries
                                  over its tokens in the chunk equal those of
                                  the longest sequence (checked on the
                                  device); any other sequence's chunk is read
                                  from its own blocks.  A sequence shorter
                                  than the hint takes part up to its last
                                  whole block and 16-token boundary (a partly
                                  filled last block is never shared by an
                                  allocator); its remaining tokens are read
                                  with its own part.  A wrong value costs
                                  time, never results. */
  int32_t window;              /* sliding window (guijiagi 5.1; 0 = none):
                                  a sequence of L tokens attends to its last
                                  min(L, window) positions only, and blocks
                                  before them are not read.  The block table
                                  must map every position from max(0, L -
                                  window) rounded down to a multiple of 16.
                                  Supported on paged_decode_attention,
                                  paged_decode_attention_int8 and
                                  paged_decode_attention_append for g in
                                  {4, 8, 16}, d in {64, 128} (bf16 and INT8
                                  pools); other shapes and MLA return
                                  KVP_ERR_UNSUPPORTED. */
} kvp_decode_desc;

/* Workspace bytes the call needs for this description (split partials).
 * For MLA and for ragged bf16 batches with a total_context_len hint it
 * depends on the current device's compute units: query it with the device
 * current that runs the call. */
size_t paged_decode_workspace_size(const kvp_decode_desc* desc);

/* Tokens per context split the automatic policy picks (for reporting);
 * for an MLA description, the 32-token tile the work is divided in; for a
 * ragged bf16 batch with a total_context_len hint, the tokens of one
 * workgroup's range by that hint. */
int32_t paged_decode_split_tokens(const kvp_decode_desc* desc);

/* MLA: persistent workgroups per head group the call launches (0 for a
 * description that is not MLA or is invalid).  The workspace size of an
 * MLA call depends on it, so query both with the same device current. */
int32_t paged_decode_mla_workgroups(const kvp_decode_desc* desc);

/* Float pools (F32/BF16 K and V of the same dtype as q; GQA, MQA, MHA). */
kvp_status paged_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* context_lens,
                                  float scale, void* out, const kvp_decode_desc* desc,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* INT8 pools: codes as in the pool layout plus fp32 scales
 * [num_blocks, n_kv, block_size]; dequantization (code * scale,
 * guijiagi 4.2) happens inside the kernel.  desc->kv_dtype == KVP_INT8.
 * Scale arrays must be 4-byte aligned (else KVP_ERR_INVALID_ARG; the same for
 * INT4). */
kvp_status paged_decode_attention_int8(const void* q, const int8_t* k_codes,
                                       const float* k_scale, const int8_t* v_codes,
                                       const float* v_scale, const int32_t* block_table,
                                       const int32_t* context_lens, float scale, void* out,
                                       const kvp_decode_desc* desc, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* INT4 pools with an attention sink (guijiagi 4.2, 4-bit branch, and 4.3):
 * codes [num_blocks, block_size, n_kv, d / 2] (two per byte) and fp32
 * scales [num_blocks, n_kv, block_size], dequantized (code * scale) inside
 * the kernel, except that positions 0 .. n_sink - 1 of every sequence come
 * unquantized from sink_k / sink_v (device bf16 [B, n_sink, n_kv, d]; the
 * first tokens draw attention from every later one, so their quantization
 * error would be amplified).  The pool must still hold a row (any finite
 * values) at every position below the context length.  0 <= n_sink <= 64
 * (sink arrays may be NULL when 0).  desc->kv_dtype == KVP_INT4; bf16 q and
 * out, d_k = d_v = 128, g in {4, 8, 16}, even n_kv; no sliding window.  Other
 * shapes KVP_ERR_UNSUPPORTED. */
kvp_status paged_decode_attention_int4(const void* q, const uint8_t* k_codes, const float* k_scale,
                                       const uint8_t* v_codes, const float* v_scale, const void* sink_k,
                                       const void* sink_v, int32_t n_sink, const int32_t* block_table,
                                       const int32_t* context_lens, float scale, void* out,
                                       const kvp_decode_desc* desc, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Absorbed MLA over a latent pool (faulkner, matrix absorption and
 * decoupled RoPE): q [B, n_h, d_k] already carries W^UK; the pool holds
 * one [c | k_rope] row of d_k bf16 per token (n_kv = 1); the value is the
 * first d_v columns of that row; out [B, n_h, d_v] is in latent space.
 * This build has the kernel for d_k = 576, d_v = 512 (a 512-wide latent
 * plus a 64-wide rope part), bf16 q, pool and output, block_size >= 16,
 * any n_h, B <= 4096; other shapes return KVP_ERR_UNSUPPORTED.  The
 * context of the batch is cut into 32-token tiles that desc->workgroups
 * persistent workgroups share in equal contiguous ranges; a sequence cut
 * between workgroups is merged by log-sum-exp in a second kernel.  The
 * workspace (always needed for MLA) holds a per-sequence record and, when
 * more than one workgroup runs, the partials of the cut sequences: fp32
 * (max, sum) per head and a bf16 unnormalised output per head. */
kvp_status paged_decode_attention_mla(const void* q, const void* latent_pool,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      float scale, void* out, const kvp_decode_desc* desc,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* One decode step in one call (qwbw 1.2: each step appends the new token's
 * K/V, then attends over the whole cache; talentme chapter 3, write_kv
 * followed by the paged attention): writes the new row of every sequence b
 * at position context_lens[b] - 1 (its slot read from block_table), then
 * computes exactly what paged_decode_attention (or _int8 / _mla, chosen by
 * the pool) computes.  Same result, bit for bit, as paged_slot_mapping +
 * reshape_and_cache + the decode call.
 *   pool:  the pool both reads and writes (its n_kv, d_k, d_v, block_size
 *          and dtype must equal desc's; a latent pool goes with an MLA desc)
 *   k_new: device [B, n_kv, d_k] rows in desc->q_dtype (quantized on write
 *          for an INT8 pool), 16-byte aligned; v_new: [B, n_kv, d_v], NULL
 *          for a latent pool
 *   q, block_table, context_lens, scale, out, workspace: as for the decode
 *          call of the pool's kind.
 * Preconditions (the usual decode step): block_table maps every position
 * below context_lens[b] to a block of the pool, the new token's position
 * included (paged_decode_validate checks this), and no other sequence of
 * the call reads the slot a sequence appends to.  A sequence with
 * context_lens[b] = 0 appends nothing and gets a zero output.  For bf16
 * pools and INT8 pools with bf16 rows (g in {4, 8, 16}), and for latent (MLA)
 * pools, the rows are written (INT8: quantized, the same codes and scales as
 * reshape_and_cache) by the attention kernel itself (one launch); otherwise
 * by the cache kernel just before it.
 * Errors as for the decode calls, plus KVP_ERR_INVALID_ARG for a NULL pool
 * or rows, a pool that does not match desc, or misaligned rows.  INT4 pools
 * (whose decode takes sink rows) are not taken here: KVP_ERR_UNSUPPORTED. */
kvp_status paged_decode_attention_append(kvp_pool* pool, const void* q, const void* k_new,
                                         const void* v_new, const int32_t* block_table,
                                         const int32_t* context_lens, float scale, void* out,
                                         const kvp_decode_desc* desc, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as paged_decode_attention_append, with the split partials and
 * records in a library-owned static device buffer instead of a caller
 * workspace.  The buffer holds 64 MiB (67108864 bytes) per device, from
 * the library's load until the process ends; a description whose
 * paged_decode_workspace_size exceeds that returns KVP_ERR_UNSUPPORTED
 * with a message and enqueues nothing.  The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's buffer address once.  Every call on a device
 * shares the device's one buffer, which keeps the last call's contents (no
 * kernel reads a byte of it that the same call did not write first):
 * calls that overlap on one device (different streams, or host threads
 * without ordering) race and give wrong results; order them on one stream.
 * Arguments, results and errors otherwise as for
 * paged_decode_attention_append. */
kvp_status paged_decode_attention_append_noalloc(kvp_pool* pool, const void* q, const void* k_new,
                                                 const void* v_new, const int32_t* block_table,
                                                 const int32_t* context_lens, float scale, void* out,
                                                 const kvp_decode_desc* desc, void* stream);

/* Chunked prefill over the paged cache (faulkner, continuous batching
 * section: a long prompt is taken a fixed number of tokens per step, each
 * chunk attending causally to the cache before it and to itself).  For
 * every sequence b and query token i < chunk_lens[b] at position
 * start_pos[b] + i, with K/V rows for every position up to start_pos[b] +
 * chunk_lens[b] - 1 already in the pool (written by reshape_and_cache):
 *   out[b][i][h] = sum_j softmax_j(scale * q[b][i][h] . K_j) V_j,
 *                  j = 0 .. start_pos[b] + i
 * through the block table (kvh = h / (n_h / n_kv)).
 *   q, out: device [B, max_chunk, n_h, 128] bf16; rows at or past
 *           chunk_lens[b] are not written.
 *   start_pos, chunk_lens: device int32 [B], start_pos[b] >= 0 and
 *           chunk_lens[b] <= max_chunk (device data: checked only under
 *           PAGEDKV_VALIDATE; a sequence outside these bounds or whose
 *           chunk runs past its table is skipped, its rows not written).
 *   desc: B, n_h, n_kv, d_k = d_v = 128, block_size, max_blocks_per_seq,
 *         bf16 q and pool; max_context_len (host bound of start_pos[b] +
 *         chunk_lens[b]) <= max_blocks_per_seq * block_size.  g = n_h /
 *         n_kv in {1, 2, 4, 8, 16}; other shapes KVP_ERR_UNSUPPORTED.
 * No workspace; asynchronous on the stream. */
kvp_status paged_prefill_attention(const void* q, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* start_pos,
                                   const int32_t* chunk_lens, float scale, void* out,
                                   const kvp_decode_desc* desc, int32_t max_chunk, void* stream);

/* ------------------------------------------------------------------------
 * Block allocator (host side; faulkner, "Prefix Caching 与 Copy-on-Write"
 * and the allocator reference section; qwbw 4.3).  It hands out the
 * physical blocks the tables above name: reference counts per block, a
 * chained hash H_k = BLAKE2b-64(H_{k-1} as 8 little-endian bytes, then the
 * block's token ids as 4 little-endian bytes each), H_{-1} = 0, on every
 * full block of a prompt; blocks whose count drops to zero keep their hash
 * and are parked in an LRU list of evictable blocks, from whose least
 * recently used end fresh blocks are taken (losing their hash).  A new
 * prompt reuses its leading full blocks found by hash (a hit increments the
 * count); copy-on-write splits a partly filled tail block shared by several
 * sequences when one of them appends.  An allocator is used by one thread
 * at a time; its calls never touch device memory.  A call that cannot be
 * met returns a status, leaves the allocator unchanged and sets
 * kvp_last_error(); KVP_ERR_OUT_OF_MEMORY means no free block is left (the
 * allocator's MemoryError).
 * ---------------------------------------------------------------------- */
typedef struct kvp_allocator kvp_allocator;

/* num_blocks blocks of block_size slots.  initial_order (host int32
 * [num_blocks], NULL = 0, 1, ...) is a permutation giving the evictable
 * list's order from least to most recently used. */
kvp_status kvp_allocator_create(int64_t num_blocks, int32_t block_size, const int32_t* initial_order,
                                kvp_allocator** out);
void kvp_allocator_destroy(kvp_allocator* allocator);

/* One step of the chained block hash (parent hash, n token ids). */
uint64_t kvp_block_hash(uint64_t parent, const int32_t* token_ids, int32_t n);

/* Blocks for a new prompt of num_tokens token ids (host int32): writes
 * ceil(num_tokens / block_size) entries of block_table (host int32, room
 * for max_blocks), their number to *num_blocks and the tokens found cached
 * (leading full blocks reused) to *cached_tokens. */
kvp_status kvp_allocate_prompt(kvp_allocator* allocator, const int32_t* token_ids, int64_t num_tokens,
                               int32_t* block_table, int32_t max_blocks, int32_t* num_blocks,
                               int64_t* cached_tokens);

/* The slot of one decoded token appended to a sequence whose table (host
 * int32, *num_blocks entries, room for max_blocks) is updated in place: a
 * full tail takes a fresh block; a partly filled tail held by several
 * sequences is copied on write: *cow_src / *cow_dst name the block whose
 * rows the caller copies with copy_blocks before writing the token (both
 * -1 otherwise).  *slot receives block * block_size + offset. */
kvp_status kvp_append_slot(kvp_allocator* allocator, int32_t* block_table, int32_t* num_blocks,
                           int32_t max_blocks, int64_t* slot, int32_t* cow_src, int32_t* cow_dst);

/* Another sequence sharing every block of a table (parallel sampling, beam
 * search: qwbw 4.3): each block's count grows by one. */
kvp_status kvp_fork_sequence(kvp_allocator* allocator, const int32_t* block_table, int32_t num_blocks);

/* Release a sequence: each block's count drops by one; blocks reaching
 * zero are parked at the most recently used end, keeping their hash. */
kvp_status kvp_free_sequence(kvp_allocator* allocator, const int32_t* block_table, int32_t num_blocks);

/* State of one block (for inspection and tests). */
kvp_status kvp_allocator_block_state(const kvp_allocator* allocator, int32_t block, int32_t* ref_count,
                                     int32_t* fill, int32_t* hashed, uint64_t* hash);

/* The evictable blocks from least to most recently used: writes up to
 * capacity ids to out (may be NULL) and returns their total number (-1 for
 * a NULL allocator). */
int64_t kvp_allocator_evictable(const kvp_allocator* allocator, int32_t* out, int64_t capacity);

/* ------------------------------------------------------------------------
 * Block copies and swaps on the device (faulkner, copy-on-write; qwbw 4.3
 * and faulkner's preemption section: a preempted sequence's blocks move to
 * host memory and back).
 * ---------------------------------------------------------------------- */

/* Bytes one block occupies over all of the pool's regions (K, V and, for
 * INT8, both scale arrays). */
size_t kv_pool_block_bytes(const kvp_pool* pool);

/* For each pair (device int32 [num_pairs, 2]: src, dst) every slot of block
 * src is copied onto block dst, in every region of the pool, bit for bit.
 * A pair with a block outside [0, num_blocks) is skipped.  Pairs must have
 * distinct dst blocks none of which is a src of another pair (copy-on-write
 * targets are fresh blocks); otherwise the result is unspecified. */
kvp_status copy_blocks(kvp_pool* pool, const int32_t* pairs, int64_t num_pairs, void* stream);

/* Swap out: the blocks listed in blocks (device int32 [n]) are gathered into
 * staging (device, n * kv_pool_block_bytes bytes, 16-byte aligned), block i
 * at offset i * kv_pool_block_bytes, regions in the order K, V, K scales, V
 * scales, then copied to host_dst (host, same size; pinned memory keeps the
 * copy asynchronous).  Swap in is the inverse: host_src -> staging ->
 * blocks.  Entries outside [0, num_blocks) are skipped. */
kvp_status swap_out_blocks(const kvp_pool* pool, const int32_t* blocks, int64_t n, void* staging,
                           void* host_dst, void* stream);
kvp_status swap_in_blocks(kvp_pool* pool, const int32_t* blocks, int64_t n, void* staging,
                          const void* host_src, void* stream);

/* ------------------------------------------------------------------------
 * Gather (qwbw 3.4: read each physical block through the table): copies
 * rows 0 .. context_lens[b]-1 of every sequence, bit for bit, into
 * out [B, max_context_len, n_kv, d] (device, elem_bytes per element);
 * rows at or beyond a sequence's length are left untouched.
 * ---------------------------------------------------------------------- */
kvp_status paged_gather(const void* pool, int32_t elem_bytes, int32_t block_size,
                        int32_t n_kv, int32_t d, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t B, int32_t max_context_len, void* out, void* stream);

/* Debug check (synchronises the stream, copies the tables to the host):
 * every context length within [0, max_context_len] and every table entry
 * a sequence uses (logical blocks 0 .. ceil(context_lens[b] / block_size)
 * - 1) within [0, num_blocks).  KVP_ERR_INVALID_ARG names the first
 * violation (sequence, logical block and value); KVP_OK otherwise. */
kvp_status paged_decode_validate(const int32_t* block_table, const int32_t* context_lens,
                                 const kvp_decode_desc* desc, int64_t num_blocks,
                                 void* stream);

/* Measurement aid, not part of the decode path: a plain streaming read of
 * buf (device, 16-byte aligned, bytes a multiple of 16) by `workgroups`
 * workgroups of 256 lanes (0 = two per compute unit), each lane with eight
 * 16-byte loads in flight; sink (device, 4 bytes) is written only if the
 * data fold to a fixed key.  Timing it gives the read-bandwidth ceiling of
 * the device that the decode kernels' HBM rates are compared with. */
kvp_status kvp_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

/* Measurement aid, not part of the decode path: `workgroups` workgroups of
 * four wavefronts (0 = four per compute unit), each wavefront running
 * `iterations` rounds of eight independent bf16 matrix instructions
 * (v_mfma_f32_16x16x32_bf16, 16,384 FLOPs each) on register operands; sink
 * (device, 4 bytes) is never written in practice.  FLOPs per call =
 * workgroups x 4 x iterations x 8 x 16384; timing it gives the bf16
 * matrix-core ceiling that the MLA and prefill FLOP rates are compared with. */
kvp_status kvp_mfma_peak(float* sink, int32_t workgroups, int32_t iterations, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* kvp_last_error(void);

/* Library version string. */
const char* kvp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
