// Absorbed MLA decode over a paged bf16 latent cache, on the matrix cores.
//
// What is computed (faulkner, matrix-absorption and decoupled-RoPE
// sections): every query head h of sequence b scores the cached latent row
// [c | k_rope] (d_k = 576 bf16) of each context token with a query that
// already carries W^UK, and the value of a token is the first d_v = 512
// columns of the same row.  One row per token is shared by all heads, so a
// decode step is a small dense contraction per token: 128 heads x 576 for
// the scores and 128 heads x 512 for the values -- the one place on this
// path where the matrix cores pay.
//
// Work split.  The context of the batch is cut into 32-token tiles and the
// flattened list (sequence-major) is divided into W equal, contiguous
// ranges, one per persistent workgroup, so a batch of ragged contexts keeps
// every compute unit equally busy.  A workgroup owns 128 heads: 8 waves
// of 16 (two waves per SIMD), so a wave holds its heads' query fragments
// (72 registers) and output accumulators (128 registers) without spilling.
// A sequence whose tiles all fall in one range is finished in place; a
// sequence cut by range boundaries leaves one fp32 partial (running max,
// sum, unnormalised output) per piece, at slot w + b (unique because w + b
// grows along the staircase of (workgroup, sequence) pairs), and
// mla_combine merges the pieces by log-sum-exp.
//
// Per 32-token tile (one LDS stage) and wave, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T       2 token blocks x 18 k-steps; A = K rows from LDS,
//                     B = Q^T fragments kept in registers
//   online softmax    on the accumulator layout (head = lane % 16, tokens
//                     spread over the 4 lane groups)
//   O^T += V^T P^T    32 column blocks; B = P^T is exactly the lane's own
//                     probabilities (the k order of both operands is
//                     tokens 4g..4g+3, 16+4g..16+4g+3 for lane group g), A
//                     = V^T from two transposed LDS reads of the same tile
// Tiles arrive through the LDS DMA path (global_load_lds_dwordx4), NS stages
// deep, with explicit vmcnt waits.  Row t's 16-byte chunks are permuted
// inside aligned groups of 8 by f(t), which keeps both the 16-row K reads
// and the 4-row transposed V reads free of LDS bank conflicts (64 banks).
#include "device_common.h"
#include "internal.h"

#ifndef PKV_MLA_KAHEAD
#define PKV_MLA_KAHEAD 1
#endif

namespace pkv {
namespace {

using dev::kLog2e;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDk * 2;                    // 1152
constexpr int kRowChunks = kRowBytes / 16;            // 72 16-byte chunks per row
constexpr int kTileTok = kMlaTileTokens;              // 32
constexpr int kStageBytes = kTileTok * kRowBytes;     // 36864
constexpr int kDmaPerTile = kStageBytes / 1024;       // 36 DMA instructions of 64 x 16 B
constexpr int kWavesM = 8;
constexpr int kThreadsM = 64 * kWavesM;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = kHeadsPerWave * kWavesM;
static_assert(kHeadsPerGroup == kMlaHeadsPerGroup, "workspace sizing assumes 128 heads per group");
constexpr int kDmaMax = (kDmaPerTile + kWavesM - 1) / kWavesM;      // 5 (waves 0-3), 4 (waves 4-7)
constexpr int kKSteps = kDk / 32;                     // 18 score k-steps per token block
constexpr int kDvBlocks = kDv / 16;                   // 32 value column blocks
constexpr int kColBlocksPerWave = kDvBlocks / kWavesM;   // 4: a wave's 64 value columns
constexpr int kAccBlocks = kWavesM * kColBlocksPerWave;  // 8 head blocks x 4 column blocks
constexpr int kKAhead = PKV_MLA_KAHEAD;               // k-steps of K operands read ahead
constexpr int kPAhead = 2;                            // head blocks of P operands read ahead
constexpr int kDmaEvery = 3;                          // k-steps between a wave's DMA instructions
static_assert((kDmaMax - 1) * kDmaEvery < kKSteps, "every DMA instruction issues inside the score loop");
constexpr int kTileCap = 256;                         // tiles whose block ids sit in LDS at once
constexpr float kRescaleSlack = 8.f;                  // log2 units a stale max may lag by

static_assert(kDmaPerTile % (kWavesM / 2) == 0 && kDmaPerTile / kWavesM == kDmaMax - 1,
              "waves 0-3 issue one more DMA instruction per tile than waves 4-7");
static_assert(kRowChunks % 8 == 0, "the permutation acts on aligned groups of 8 chunks");

struct MlaParams {
  const uint16_t* q;        // [B, n_h, 576] bf16
  const uint8_t* pool;      // latent rows, 1152 bytes per slot
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;            // [B, n_h, 512] bf16
  uint16_t* part_o;         // [W + B, head groups, 8 waves, 32 blocks, 64 lanes, 4] bf16, unnormalised
  float* part_ml;           // [W + B, n_h, 2]   (running max in log2 units, sum)
  int32_t* seq_meta;        // [B, 2] first and last workgroup holding the sequence
  float scale_log2;         // scale * log2(e)
  int32_t B, n_h, block_shift, max_blocks_per_seq, W;
  const uint16_t* k_new;    // append: [B, 576] bf16 rows for position context_lens[b] - 1 (or null)
};

// Chunk permutation of tile row t (inside each aligned group of 8 chunks):
// chunk c of row t sits at position c ^ (t & 7).  Measured with the LDS
// bank-conflict counter on gfx950, both operand reads are then conflict-free:
// the 16-byte K reads (16 rows, one chunk) and the transposed 8-byte V reads
// (rows 4g..4g+3, chunk pairs); rows t and t + 16 share the permutation.
__device__ __forceinline__ int swz(int t) { return t & 7; }

// Two floats to a packed bf16 pair (low half = a), round to nearest even:
// one v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// s_waitcnt immediate with vmcnt = 0 and the other counters at their
// maximum (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Every LDS access of this wave has completed, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A copy of v the compiler cannot see through: values derived from it are
// recomputed where they are used instead of being kept live across the tile
// loop (the accumulators and query fragments leave few registers free).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// One tile's block ids and fill, staged in LDS for the DMA issue.
struct TileInfo {
  int32_t blk0, blk1;       // physical blocks of rows [0, 16) and [16, 32) when block_size is 16
  int32_t nvalid_row0;      // valid rows | first row inside blk0 << 8
  int32_t seq;
  int32_t j_last;           // tile index in the sequence << 1 | (last tile of the sequence)
};

// LDS DMA of one tile: stage position P (16-byte units, 64 per
// instruction, instruction j = wave + 8 i of the workgroup) holds logical
// chunk c of row t, i.e. P = 72 t + (c ^ swz(t)).
//
// A whole tile inside one block (block size >= 32, tiles start at multiples
// of 32) is one contiguous 36 KB run of 32 rows; since a row holds a whole
// number of 8-chunk groups, position P reads chunk P ^ swz(P / 72) of the
// run: one scalar base per tile and a lane offset.  tile_run returns that
// base, or null for the other tiles.
__device__ __forceinline__ const uint8_t* tile_run(const MlaParams& p, const TileInfo ti) {
  const int nvalid = ti.nvalid_row0 & 0xff;
  const int row0 = ti.nvalid_row0 >> 8;
  if (nvalid != kTileTok || p.block_shift < 5) return nullptr;
  const uint32_t slot0 = __builtin_amdgcn_readfirstlane(((uint32_t)ti.blk0 << p.block_shift) | (uint32_t)row0);
  return p.pool + (uint64_t)slot0 * kRowBytes;
}

// Instruction i of this wave for a whole tile (ln: lane index).
__device__ __forceinline__ void dma_run(const uint8_t* run, uint32_t stage_lds, int wave, int i, int ln) {
  const int j = wave + kWavesM * i;
  if (j < kDmaPerTile) {
    const uint32_t P = (uint32_t)(j * 64 + ln);
    const uint32_t off = 16u * (P ^ (uint32_t)swz((int)(P / (uint32_t)kRowChunks)));
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)(j * 1024));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0), "v"(off), "s"(run) : "memory", "m0");
  }
}

// All of this wave's instructions for any tile: rows at or beyond the
// context re-read the last valid row (finite data for the masked tokens);
// rows [16, 32) may sit in a second block when the block size is 16.
__device__ __forceinline__ void issue_tile(const MlaParams& p, uint32_t stage_lds, const TileInfo ti,
                                           int wave, int lane) {
  const int nvalid = ti.nvalid_row0 & 0xff;
  const int row0 = ti.nvalid_row0 >> 8;
  const int bs_mask = (1 << p.block_shift) - 1;
  const int ln = opaque(lane);
#pragma unroll
  for (int i = 0; i < kDmaMax; ++i) {
    const int j = wave + kWavesM * i;              // instruction index in the tile
    if (j < kDmaPerTile) {
      const int P = j * 64 + ln;                   // stage position in 16-byte units
      const int t = P / kRowChunks, pc = P - t * kRowChunks;
      const uint32_t cbyte = (uint32_t)(((pc & ~7) | ((pc & 7) ^ swz(t))) * 16);
      const int rf = row0 + min(t, nvalid - 1);
      const uint32_t blk = (uint32_t)(rf > bs_mask ? ti.blk1 : ti.blk0);
      const uint32_t slot = (blk << p.block_shift) | (uint32_t)(rf & bs_mask);
      const uint8_t* src = p.pool + (uint64_t)slot * kRowBytes + cbyte;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)(j * 1024));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0), "v"(src) : "memory", "m0");
    }
  }
}

// Global tile x -> sequence by binary search of the tile prefix
// (s_pref[b] <= x < s_pref[b + 1]; sequence b then has a tile).
__device__ __forceinline__ int seq_of_tile(const int32_t* s_pref, int B, int x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Workgroup whose range [floor(wT/W), floor((w+1)T/W)) holds tile x.
__device__ __forceinline__ int owner_of_tile(int64_t x, int64_t T, int64_t W) {
  return (int)(((x + 1) * W - 1) / T);
}

template <int NS>
__global__ void __launch_bounds__(kThreadsM, 1) decode_mla_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[NS * kStageBytes];
  __shared__ int32_t s_pref[kMlaMaxBatch + 1];
  __shared__ uint8_t s_fill[kMlaMaxBatch];    // per sequence: (context - 1) mod 32 (its last tile's rows - 1)
  __shared__ TileInfo s_tile[kTileCap + NS];
  __shared__ int32_t s_scan[kWavesM];
  // probabilities of the tile, one 16-byte B fragment per (head block, lane)
  __shared__ bf16x8_t s_p[kWavesM * 64];
  __shared__ float s_alpha[kHeadsPerGroup];   // rescale factor per head
  __shared__ float s_linv[kHeadsPerGroup];    // 1 / softmax sum per head
  __shared__ __attribute__((aligned(8))) uint8_t s_flag[kWavesM];    // head block rescaled

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int hgroup = blockIdx.y * kHeadsPerGroup;
  const int hbase = hgroup + wave * kHeadsPerWave;   // this wave's heads for the scores
  const bool score_active = hbase < p.n_h;
  const int B = p.B;

  // ---- tile prefix over the batch (every workgroup computes it): each
  // thread sums its share of the sequences, a shuffle scan inside each wave,
  // then the waves' totals (one barrier; the last tile's fill of each
  // sequence is kept for the block-id staging below) ----
  {
    const int per = (B + kThreadsM - 1) / kThreadsM;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int sum = 0;
    for (int b = lo; b < hi; ++b) sum += (p.context_lens[b] + kTileTok - 1) / kTileTok;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int k = 0; k < wave; ++k) run += s_scan[k];
    for (int b = lo; b < hi; ++b) {
      const int c = p.context_lens[b];
      s_pref[b] = run;
      s_fill[b] = (uint8_t)((c - 1) & (kTileTok - 1));
      run += (c + kTileTok - 1) / kTileTok;
    }
    if (tid == kThreadsM - 1) s_pref[B] = run;
    __syncthreads();
  }
  const int T = s_pref[B];
  // Never more workgroups than tiles: then every range below is non-empty,
  // which the combine step relies on when it walks a sequence's pieces.
  const int W = min(p.W, T);
  if (w >= W) return;
  const int start = (int)((int64_t)w * T / W);
  const int end = (int)((int64_t)(w + 1) * T / W);
  const int n = end - start;

  // Per-lane roles (formed per phase from an opaque lane index): lane group
  // g = lane >> 4 (k / token groups), index l16 = lane & 15.  K operand of
  // block mt, k-step ks: row 16 mt + l16, chunk 4 ks + g.  V^T operand of
  // column block m: rows 4 g + (l16 >> 2) (and + 16), 8-byte piece l16 & 3
  // of columns 16 m .. 16 m + 15.
  const uint32_t stage0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)s_stage;

  // ---- block ids of the next tiles, staged in LDS ----
  int c0 = start;
  auto fill_tiles = [&](int first) {
    const int cnt = min(kTileCap + NS, end - first);
    for (int k = tid; k < cnt; k += kThreadsM) {
      const int x = first + k;
      const int b = seq_of_tile(s_pref, B, x);
      const int tok0 = (x - s_pref[b]) * kTileTok;
      const bool last_tile = x + 1 == s_pref[b + 1];
      const int nvalid = last_tile ? s_fill[b] + 1 : kTileTok;
      const int kb = tok0 >> p.block_shift;
      const int row0 = tok0 & ((1 << p.block_shift) - 1);
      const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks_per_seq;
      const int32_t b0 = bt[kb];
      const int32_t b1 = (row0 + nvalid > (1 << p.block_shift)) ? bt[kb + 1] : b0;
      const int jt = x - s_pref[b];
      s_tile[k] = TileInfo{b0, b1, nvalid | (row0 << 8), b, (jt << 1) | (int)last_tile};
    }
  };
  fill_tiles(c0);
  __syncthreads();

  bf16x8_t qf[kKSteps];
  // value accumulators: head block hb, column block cb of this wave's 64
  // columns -> acc[hb * 4 + cb]; lane holds head 16 hb + l16, columns
  // 64 wave + 16 cb + 4 g .. + 3
  f32x4_t acc[kAccBlocks];
  float m_run = -INFINITY, l_run = 0.f;   // scores side: this lane's head (partial sum over g)
  int piece_first = 0;        // tile index in the sequence where this piece began
  int cur_b = -1;

  // A new piece (sequence b from its tile j on): reset the softmax state and
  // the accumulators and load the sequence's queries.  The loads complete
  // in a wait the compiler sees: otherwise it spreads waits for them over
  // the score loop on every tile's path, ending in vmcnt(0), which would
  // also wait for the DMA in flight for the next tiles.
  auto start_piece = [&](int b, int j) {
    cur_b = b;
    piece_first = j;
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int m = 0; m < kAccBlocks; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int ln = opaque(lane), h = hbase + (ln & 15);
    if (score_active && h < p.n_h) {
      const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(p.q + ((int64_t)b * p.n_h + h) * kDk + 8 * (ln >> 4));
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = qp[4 * ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = bf16x8_t{};
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };

  // ---- append: the workgroup holding a sequence's last tile writes the new
  // token's latent row into its slot (position context - 1) and the stores
  // complete before any of its DMA, which reads that slot, is issued ----
  if (p.k_new != nullptr && n > 0) {
    const int b_lo = s_tile[0].seq;
    const int b_hi = seq_of_tile(s_pref, B, end - 1);
    bool any = false;
    for (int b = b_lo; b <= b_hi; ++b) {
      const int nt = s_pref[b + 1] - s_pref[b];
      if (nt == 0 || s_pref[b + 1] - 1 < start || s_pref[b + 1] - 1 >= end) continue;   // no last tile here
      any = true;
      const int pos = (nt - 1) * kTileTok + s_fill[b];
      const int32_t phys = p.block_table[(int64_t)b * p.max_blocks_per_seq + (pos >> p.block_shift)];
      if (phys < 0) continue;                                 // an unmapped block is skipped
      const uint32_t slot = ((uint32_t)phys << p.block_shift) | (uint32_t)(pos & ((1 << p.block_shift) - 1));
      for (int c = tid; c < kRowChunks; c += kThreadsM)
        *reinterpret_cast<dev::u32x4_t*>(const_cast<uint8_t*>(p.pool) + (uint64_t)slot * kRowBytes + 16 * c) =
            *reinterpret_cast<const dev::u32x4_t*>(reinterpret_cast<const uint8_t*>(p.k_new + (int64_t)b * kDk) + 16 * c);
    }
    if (any) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
  }

  // ---- prologue: first NS - 1 tiles in flight ----
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n) issue_tile(p, stage0 + s * kStageBytes, s_tile[s], wave, lane);

  // the first piece's queries load with the first tiles' DMA: one wait for all
  if (n > 0) start_piece(s_tile[0].seq, s_tile[0].j_last >> 1);

  for (int i = 0; i < n; ++i) {
    const int x = start + i;
    // this wave's DMA for tile i has landed (later tiles may still fly),
    // then every wave's has, and every wave is done with tile i - 1
    const int ahead = min(NS - 2, n - 1 - i);
    if (wave < kDmaPerTile - kWavesM * (kDmaMax - 1)) {
      if (NS > 3 && ahead >= 2) wait_vmcnt<2 * kDmaMax>();
      else if (NS > 2 && ahead >= 1) wait_vmcnt<kDmaMax>();
      else wait_vmcnt<0>();
    } else {
      if (NS > 3 && ahead >= 2) wait_vmcnt<2 * (kDmaMax - 1)>();
      else if (NS > 2 && ahead >= 1) wait_vmcnt<kDmaMax - 1>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    if (x - c0 == kTileCap) {   // stage the next run of block ids
      c0 = x;
      fill_tiles(c0);
      __syncthreads();
    }
    const TileInfo ti = s_tile[x - c0];
    const int b = ti.seq;
    const int nvalid = ti.nvalid_row0 & 0xff;
    const int j = ti.j_last >> 1;
    const bool last_of_seq = ti.j_last & 1;
    const uint32_t stage = stage0 + (uint32_t)((i % NS) * kStageBytes);
    if (b != cur_b) start_piece(b, j);   // a new piece

    // Tile i + NS - 1 goes to stage (i - 1) % NS, free now: every wave has
    // passed this tile's barrier.  A whole contiguous tile is issued one
    // instruction every kDmaEvery k-steps of the score loop, so that the
    // workgroup's 36 instructions do not all queue at the same moment;
    // other tiles (and waves without score work) issue theirs here.
    const uint32_t stage_next = stage0 + (uint32_t)(((i + NS - 1) % NS) * kStageBytes);
    const uint8_t* run = nullptr;
    if (i + NS - 1 < n) {
      const TileInfo tn = s_tile[x + NS - 1 - c0];
      run = tile_run(p, tn);
      if (!run) {
        issue_tile(p, stage_next, tn, wave, lane);
      } else if (!score_active) {
        const int ln = opaque(lane);
#pragma unroll
        for (int d = 0; d < kDmaMax; ++d) dma_run(run, stage_next, wave, d, ln);
        run = nullptr;
      }
    }

    // ---- scores of this wave's 16 heads: S^T = K Q^T, two 16-token blocks ----
    bf16x8_t pb = {};
    int rescaled = 0;
    if (score_active) {
      const int ln = opaque(lane), g = ln >> 4, l16 = ln & 15, tk = l16;
      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      // k-step ks of row tk: chunk 4 ks + g at position 8 (ks >> 1) + ((4 (ks & 1) + g) ^ swz(tk));
      // two base pointers (even / odd k-steps) and constant offsets, row tk + 16
      // 16 rows further (swz(tk + 16) = swz(tk))
      const lds_bf16x8_t* kpe =
          (const lds_bf16x8_t*)(uintptr_t)(stage + (uint32_t)(tk * kRowBytes + 16 * (g ^ swz(tk))));
      const lds_bf16x8_t* kpo =
          (const lds_bf16x8_t*)(uintptr_t)(stage + (uint32_t)(tk * kRowBytes + 16 * ((4 + g) ^ swz(tk))));
      auto kread = [&](int ks, int blk) { return ((ks & 1) ? kpo : kpe)[8 * (ks >> 1) + blk * 16 * kRowChunks]; };
      // kKAhead k-steps of operands in flight ahead of the matrix instructions
      bf16x8_t ka0[kKSteps], ka1[kKSteps];
#pragma unroll
      for (int ks = 0; ks < kKAhead; ++ks) {
        ka0[ks] = kread(ks, 0);
        ka1[ks] = kread(ks, 1);
      }
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks % kDmaEvery == 0 && ks / kDmaEvery < kDmaMax && run)
          dma_run(run, stage_next, wave, ks / kDmaEvery, ln);
        if (ks + kKAhead < kKSteps) {
          ka0[ks + kKAhead] = kread(ks + kKAhead, 0);
          ka1[ks + kKAhead] = kread(ks + kKAhead, 1);
        }
        // the reads for the coming k-steps are issued before this step's
        // matrix instructions, which then cover their latency
        __builtin_amdgcn_sched_barrier(0);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[ks], qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[ks], qf[ks], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- online softmax (base 2) for head l16: tokens 4g + e, 16 + 4g + e.
      // With c = |scale log2 e| and the scores negated when the scale is
      // negative, x = c s' and, c being non-negative, max x = c max s'
      // exactly (rounding is monotonic); p = 2^(c s' - m) by one fma.
      float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const float c = fabsf(p.scale_log2);
      if (p.scale_log2 < 0.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = -sv[e];
      }
      if (nvalid < kTileTok) {   // the last tile of a sequence: mask the tokens past its end
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & 4) * 4 + 4 * g + (e & 3) >= nvalid) sv[e] = -INFINITY;
      }
      float smax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      // the same head sits in lanes l16, l16 + 16, l16 + 32, l16 + 48
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
        smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
        smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      const float mx = c * smax;
      if (m_run == -INFINITY) {
        m_run = mx;             // first tile of the piece: nothing accumulated yet
      } else if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        rescaled = 1;
        if (g == 0) s_alpha[wave * kHeadsPerWave + l16] = alpha;
      }
      // probabilities rounded to bf16; the running sum adds the rounded values
      // (dot2 with ones: exact products, fp32 sums)
      const float nm = -m_run;
      if (nvalid < kTileTok) {   // masked tokens get 0 (c may be 0, and 0 * -inf is NaN)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[e] = (__bf16)(sv[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(sv[e], c, nm)));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[e], c, nm));
      }
      const dev::u32x4_t pw = __builtin_bit_cast(dev::u32x4_t, pb);
      constexpr uint32_t kOnes = 0x3f803f80u;   // bf16 (1, 1)
      l_run = dev::dot2_bf16(pw[0], kOnes, l_run);
      l_run = dev::dot2_bf16(pw[1], kOnes, l_run);
      l_run = dev::dot2_bf16(pw[2], kOnes, l_run);
      l_run = dev::dot2_bf16(pw[3], kOnes, l_run);
    }
    // heads past n_h (inactive waves) contribute zero probabilities
    s_p[wave * 64 + opaque(lane)] = pb;
    if (lane == 0) s_flag[wave] = (uint8_t)rescaled;
    lds_barrier();

    // ---- O^T += V^T P^T for this wave's 64 columns and all 128 heads ----
    {
      const uint2 fw = *reinterpret_cast<const uint2*>(s_flag);
      const uint64_t flags = ((uint64_t)__builtin_amdgcn_readfirstlane(fw.y) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane(fw.x);
      const int ln = opaque(lane), g = ln >> 4, l16 = ln & 15;
      const int tv = 4 * g + (l16 >> 2), cp = l16 & 3;
      const uint32_t vb = stage + (uint32_t)(tv * kRowBytes) + 8 * (cp & 1);
      const int sv = swz(tv);
      bf16x8_t va[kColBlocksPerWave];
#pragma unroll
      for (int cb = 0; cb < kColBlocksPerWave; ++cb) {
        const int m = kColBlocksPerWave * wave + cb;
        const uint32_t a = vb + 128 * (m >> 2) + 16 * ((2 * (m & 3) + (cp >> 1)) ^ sv);
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a);
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(a + 16 * kRowBytes));
        va[cb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      bf16x8_t pv[kWavesM];
#pragma unroll
      for (int hb = 0; hb < kPAhead; ++hb) pv[hb] = s_p[hb * 64 + lane];
#pragma unroll
      for (int hb = 0; hb < kWavesM; ++hb) {
        if (hb + kPAhead < kWavesM) pv[hb + kPAhead] = s_p[(hb + kPAhead) * 64 + lane];
        if ((flags >> (8 * hb)) & 1) {
          const float alpha = s_alpha[hb * kHeadsPerWave + l16];
#pragma unroll
          for (int cb = 0; cb < kColBlocksPerWave; ++cb) acc[hb * kColBlocksPerWave + cb] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < kColBlocksPerWave; ++cb)
          acc[hb * kColBlocksPerWave + cb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[cb], pv[hb], acc[hb * kColBlocksPerWave + cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- end of a piece: finish the sequence or leave a partial ----
    if (last_of_seq || i == n - 1) {
      const bool whole = piece_first == 0 && last_of_seq;
      if (piece_first == 0 && tid == 0) {
        // the workgroup holding the first tile records which workgroups
        // hold the sequence (for the combine step)
        const int last = owner_of_tile(s_pref[b + 1] - 1, T, W);
        p.seq_meta[2 * b] = w;
        p.seq_meta[2 * b + 1] = last;
      }
      const int ln = opaque(lane), g = ln >> 4, l16 = ln & 15;
      if (score_active) {
        const int h = hbase + l16;
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (g == 0) {
          s_linv[wave * kHeadsPerWave + l16] = 1.f / l_tot;
          if (!whole && h < p.n_h)
            *reinterpret_cast<float2*>(p.part_ml + 2 * ((int64_t)(w + b) * p.n_h + h)) = float2{m_run, l_tot};
        }
      }
      lds_barrier();
      const int col0 = kColBlocksPerWave * 16 * wave + 4 * g;
      if (whole) {
#pragma unroll
        for (int hb = 0; hb < kWavesM; ++hb) {
          const int ho = hgroup + hb * kHeadsPerWave + l16;
          if (ho < p.n_h) {
            const float inv = s_linv[hb * kHeadsPerWave + l16];
            uint16_t* orow = p.out + ((int64_t)b * p.n_h + ho) * kDv + col0;
#pragma unroll
            for (int cb = 0; cb < kColBlocksPerWave; ++cb) {
              const f32x4_t a = acc[hb * kColBlocksPerWave + cb];
              *reinterpret_cast<dev::u32x2_t*>(orow + 16 * cb) =
                  dev::u32x2_t{pack_bf16(a[0] * inv, a[1] * inv), pack_bf16(a[2] * inv, a[3] * inv)};
            }
          }
        }
      } else {
        // unnormalised partial, rounded to bf16, in the accumulator layout:
        // one contiguous 512-byte run per (wave, block)
        uint16_t* po = p.part_o + ((((int64_t)(w + b) * gridDim.y + blockIdx.y) * kWavesM + wave) *
                                   kAccBlocks * 64 + ln) * 4;
#pragma unroll
        for (int a = 0; a < kAccBlocks; ++a) {
          *reinterpret_cast<dev::u32x2_t*>(po + a * 64 * 4) =
              dev::u32x2_t{pack_bf16(acc[a][0], acc[a][1]), pack_bf16(acc[a][2], acc[a][3])};
        }
      }
      cur_b = -1;
    }
  }
}

// Merge the pieces of the sequences that were cut across workgroups, and
// zero the output of empty sequences.  The partials are read in the layout
// the decode kernel leaves them: workgroup (b, y) with y = (head group,
// wave, 4 accumulator blocks) has thread t handle accumulator block
// 4 (y % 8) + t / 64 of lane t % 64, i.e. four output columns of one head.
constexpr int kCombineThreads = 256;
// a thread takes two adjacent accumulator lanes (two heads, 4 columns each)
constexpr int kCombineSlices = kAccBlocks * 32 / kCombineThreads;   // 4 workgroups per (group, wave)
constexpr int kCombineBatch = 8;

__global__ void __launch_bounds__(kCombineThreads) mla_combine_kernel(MlaParams p) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int slice = blockIdx.y % kCombineSlices;
  const int wave = (blockIdx.y / kCombineSlices) % kWavesM;
  const int hg = blockIdx.y / (kCombineSlices * kWavesM);
  // accumulator block a, lanes ln and ln + 1: heads h and h + 1 (ln even, so
  // both in one 16-head block), the same 4 columns
  const int a = slice * (kCombineThreads / 32) + t / 32, ln = 2 * (t % 32);
  const int h = hg * kHeadsPerGroup + (a / kColBlocksPerWave) * kHeadsPerWave + (ln & 15);
  if (h >= p.n_h) return;
  const bool two = h + 1 < p.n_h;
  const int col = 16 * (kColBlocksPerWave * wave + a % kColBlocksPerWave) + 4 * (ln >> 4);
  uint16_t* orow = p.out + ((int64_t)b * p.n_h + h) * kDv + col;
  const int ctx = p.context_lens[b];
  if (ctx <= 0) {
    *reinterpret_cast<dev::u32x2_t*>(orow) = dev::u32x2_t{0u, 0u};
    if (two) *reinterpret_cast<dev::u32x2_t*>(orow + kDv) = dev::u32x2_t{0u, 0u};
    return;
  }
  const int wf = p.seq_meta[2 * b], wl = p.seq_meta[2 * b + 1];
  if (wf == wl) return;   // finished in place
  const int groups = gridDim.y / (kCombineSlices * kWavesM);
  // pieces in batches of kCombineBatch with every load of a batch issued
  // before any is used; the running maxima are raised batch by batch
  float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f};
  float o[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int s0 = wf; s0 <= wl; s0 += kCombineBatch) {
    float2 ml[kCombineBatch][2];
    dev::u32x4_t v[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int s = s0 + k;
      if (s <= wl) {
        const float* mlp = p.part_ml + 2 * ((int64_t)(s + b) * p.n_h + h);
        ml[k][0] = *reinterpret_cast<const float2*>(mlp);
        ml[k][1] = two ? *reinterpret_cast<const float2*>(mlp + 2) : float2{-INFINITY, 0.f};
        v[k] = *reinterpret_cast<const dev::u32x4_t*>(
            p.part_o + ((((int64_t)(s + b) * groups + hg) * kWavesM + wave) * kAccBlocks * 64 + a * 64 + ln) * 4);
      } else {
        ml[k][0] = ml[k][1] = float2{-INFINITY, 0.f};
        v[k] = dev::u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float mc = M[e];
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) mc = fmaxf(mc, ml[k][e].x);
      // 0 on the first batch (M = -inf); a second head that does not exist
      // stays at -inf throughout and is never stored
      const float r = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[e] - mc);
      L[e] *= r;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[e][c] *= r;
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) {
        const float f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[k][e].x - mc);   // 0 for the padding
        L[e] = fmaf(ml[k][e].y, f, L[e]);
        const uint32_t w0 = v[k][2 * e], w1 = v[k][2 * e + 1];
        o[e][0] = fmaf(__uint_as_float(w0 << 16), f, o[e][0]);
        o[e][1] = fmaf(__uint_as_float(w0 & 0xffff0000u), f, o[e][1]);
        o[e][2] = fmaf(__uint_as_float(w1 << 16), f, o[e][2]);
        o[e][3] = fmaf(__uint_as_float(w1 & 0xffff0000u), f, o[e][3]);
      }
      M[e] = mc;
    }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (e == 1 && !two) break;
    const float inv = 1.f / L[e];
    *reinterpret_cast<dev::u32x2_t*>(orow + e * kDv) =
        dev::u32x2_t{pack_bf16(o[e][0] * inv, o[e][1] * inv), pack_bf16(o[e][2] * inv, o[e][3] * inv)};
  }
}

constexpr int kMlaStages = 3;

}  // namespace

bool mla_supported(int d_k, int d_v, int n_h, int block_size) {
  return d_k == kDk && d_v == kDv && n_h >= 1 && block_size >= 16;
}

int mla_head_groups(int n_h) { return (n_h + kHeadsPerGroup - 1) / kHeadsPerGroup; }

hipError_t launch_decode_mla(const DecodeParams& d, hipStream_t stream) {
  MlaParams p{};
  p.q = static_cast<const uint16_t*>(d.q);
  p.pool = static_cast<const uint8_t*>(d.k);
  p.block_table = d.block_table;
  p.context_lens = d.context_lens;
  p.out = static_cast<uint16_t*>(d.out);
  p.part_o = reinterpret_cast<uint16_t*>(d.part_o);
  p.part_ml = d.part_ml;
  p.seq_meta = d.seq_meta;
  p.scale_log2 = d.scale * kLog2e;
  p.B = d.B;
  p.n_h = d.n_h;
  p.block_shift = d.block_shift;
  p.max_blocks_per_seq = d.max_blocks_per_seq;
  p.W = d.workgroups;
  p.k_new = static_cast<const uint16_t*>(d.k_new);
  const dim3 grid((unsigned)p.W, (unsigned)mla_head_groups(p.n_h));
  hipLaunchKernelGGL((decode_mla_kernel<kMlaStages>), grid, dim3(kThreadsM), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)p.B, grid.y * kWavesM * kCombineSlices),
                     dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
