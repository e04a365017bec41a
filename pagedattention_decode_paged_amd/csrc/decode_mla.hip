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
constexpr int kDmaMax = (kDmaPerTile + kWavesM - 1) / kWavesM;      // 5 (waves 0-3), 4 (waves 4-7)
constexpr int kKSteps = kDk / 32;                     // 18 score k-steps per token block
constexpr int kDvBlocks = kDv / 16;                   // 32 value column blocks
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
  float* part_o;            // [W + B, n_h, 512] unnormalised
  float* part_ml;           // [W + B, n_h, 2]   (running max in log2 units, sum)
  int32_t* seq_meta;        // [B, 2] first and last workgroup holding the sequence
  float scale_log2;         // scale * log2(e)
  int32_t B, n_h, block_shift, max_blocks_per_seq, W;
};

// Chunk permutation of tile row t (inside each aligned group of 8 chunks):
// chunk c of row t sits at position c ^ (t & 7).  Measured with the LDS
// bank-conflict counter on gfx950, both operand reads are then conflict-free:
// the 16-byte K reads (16 rows, one chunk) and the transposed 8-byte V reads
// (rows 4g..4g+3, chunk pairs); rows t and t + 16 share the permutation.
__device__ __forceinline__ int swz(int t) { return t & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Every LDS access of this wave has completed, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One tile's block ids and fill, staged in LDS for the DMA issue.
struct TileInfo {
  int32_t blk0, blk1;       // physical blocks of rows [0, 16) and [16, 32) when block_size is 16
  int32_t nvalid_row0;      // valid rows | first row inside blk0 << 8
  int32_t seq;
};

// Issue this wave's share of the LDS DMA for one tile: stage position P
// (16-byte units, 64 per instruction) holds logical chunk c of row t.  Rows
// at or beyond the context re-read the last valid row (finite data for the
// masked tokens).
__device__ __forceinline__ void issue_tile(const MlaParams& p, uint32_t stage_lds, const TileInfo ti,
                                           int wave, int lane) {
  const int nvalid = ti.nvalid_row0 & 0xff;
  const int row0 = ti.nvalid_row0 >> 8;
  const int bs_mask = (1 << p.block_shift) - 1;
  // opaque copy of the lane index: the per-lane offsets below are recomputed
  // at every tile rather than kept live across the loop (registers are full)
  int ln = lane;
  asm volatile("" : "+v"(ln));
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
  __shared__ TileInfo s_tile[kTileCap + NS];
  __shared__ int32_t s_scan[kThreadsM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int hbase = blockIdx.y * kHeadsPerGroup + wave * kHeadsPerWave;
  const bool wave_active = hbase < p.n_h;
  const int B = p.B;

  // ---- tile prefix over the batch (every workgroup computes it) ----
  {
    const int per = (B + kThreadsM - 1) / kThreadsM;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int sum = 0;
    for (int b = lo; b < hi; ++b) sum += (p.context_lens[b] + kTileTok - 1) / kTileTok;
    s_scan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kThreadsM; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int run = s_scan[tid] - sum;
    for (int b = lo; b < hi; ++b) {
      s_pref[b] = run;
      run += (p.context_lens[b] + kTileTok - 1) / kTileTok;
    }
    if (tid == kThreadsM - 1) s_pref[B] = s_scan[kThreadsM - 1];
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

  // ---- per-lane roles: lane group g (k / token groups), index l16 ----
  const int g = lane >> 4, l16 = lane & 15;
  // K operand of block mt, k-step ks: row 16 mt + l16, chunk 4 ks + g; V^T
  // operand of column block m: rows 4 g + (l16 >> 2) (and + 16), 8-byte
  // piece l16 & 3 of columns 16 m .. 16 m + 15 (offsets formed per tile)
  const int tk = l16, tv = 4 * g + (l16 >> 2), cp = l16 & 3;
  const uint32_t stage0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)s_stage;

  // ---- block ids of the next tiles, staged in LDS ----
  int c0 = start;
  auto fill_tiles = [&](int first) {
    const int cnt = min(kTileCap + NS, end - first);
    for (int k = tid; k < cnt; k += kThreadsM) {
      const int x = first + k;
      const int b = seq_of_tile(s_pref, B, x);
      const int tok0 = (x - s_pref[b]) * kTileTok;
      const int nvalid = min(kTileTok, p.context_lens[b] - tok0);
      const int kb = tok0 >> p.block_shift;
      const int row0 = tok0 & ((1 << p.block_shift) - 1);
      const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks_per_seq;
      const int32_t b0 = bt[kb];
      const int32_t b1 = (row0 + nvalid > (1 << p.block_shift)) ? bt[kb + 1] : b0;
      s_tile[k] = TileInfo{b0, b1, nvalid | (row0 << 8), b};
    }
  };
  fill_tiles(c0);
  __syncthreads();

  // ---- prologue: first NS - 1 tiles in flight ----
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n) issue_tile(p, stage0 + s * kStageBytes, s_tile[s], wave, lane);

  bf16x8_t qf[kKSteps];
  f32x4_t acc[kDvBlocks];
  float m_run = -INFINITY, l_run = 0.f;
  int piece_first = 0;        // tile index in the sequence where this piece began
  int cur_b = -1;
  const int h = hbase + l16;  // this lane's head

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
    const int j = x - s_pref[b];
    const uint32_t stage = stage0 + (uint32_t)((i % NS) * kStageBytes);
    // stage (i - 1) % NS is free: every wave passed this tile's barrier
    if (i + NS - 1 < n)
      issue_tile(p, stage0 + (uint32_t)(((i + NS - 1) % NS) * kStageBytes),
                 s_tile[x + NS - 1 - c0], wave, lane);

    if (b != cur_b) {           // a new piece: load this sequence's queries
      cur_b = b;
      piece_first = j;
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int m = 0; m < kDvBlocks; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (h < p.n_h) {
        const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(p.q + ((int64_t)b * p.n_h + h) * kDk + 8 * g);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = qp[4 * ks];
      } else {
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = bf16x8_t{};
      }
    }

    if (wave_active) {
      // ---- S^T = K Q^T: two 16-token blocks ----
      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const uint32_t kb0 = stage + (uint32_t)(tk * kRowBytes), kb1 = kb0 + 16 * kRowBytes;
      const uint32_t ke = 16 * (g ^ swz(tk)), ko = 16 * ((4 + g) ^ swz(tk));   // swz(tk + 16) = swz(tk)
      auto kc = [&](int ks) { return 128 * (ks >> 1) + ((ks & 1) ? ko : ke); };
      // one k-step of operands in flight ahead of the matrix instructions
      bf16x8_t ka0 = *(const lds_bf16x8_t*)(uintptr_t)(kb0 + kc(0));
      bf16x8_t ka1 = *(const lds_bf16x8_t*)(uintptr_t)(kb1 + kc(0));
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        bf16x8_t kn0 = ka0, kn1 = ka1;
        if (ks + 1 < kKSteps) {
          kn0 = *(const lds_bf16x8_t*)(uintptr_t)(kb0 + kc(ks + 1));
          kn1 = *(const lds_bf16x8_t*)(uintptr_t)(kb1 + kc(ks + 1));
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qf[ks], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        ka0 = kn0;
        ka1 = kn1;
      }

      // ---- online softmax (base 2) for head l16: tokens 4g + e, 16 + 4g + e
      float xv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t0 = 4 * g + e, t1 = 16 + 4 * g + e;
        xv[e] = t0 < nvalid ? s0[e] * p.scale_log2 : -INFINITY;
        xv[4 + e] = t1 < nvalid ? s1[e] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(xv[e], xv[4 + e]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (m_run == -INFINITY) {
        m_run = mx;             // first tile of the piece: nothing accumulated yet
      } else if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int m = 0; m < kDvBlocks; ++m) acc[m] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      bf16x8_t pb;
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(xv[e] - m_run);
        pb[e] = pr;
        lsum += (float)pr;
      }
      l_run += lsum;

      // ---- O^T += V^T P^T over the 32 column blocks ----
      const uint32_t vb = stage + (uint32_t)(tv * kRowBytes) + 8 * (cp & 1);
      const int sv = swz(tv);
      auto vread = [&](int m) {
        const uint32_t a = vb + 128 * (m >> 2) + 16 * ((2 * (m & 3) + (cp >> 1)) ^ sv);
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a);
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(a + 16 * kRowBytes));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t va = vread(0);
#pragma unroll
      for (int m = 0; m < kDvBlocks; ++m) {
        bf16x8_t vn = va;
        if (m + 1 < kDvBlocks) vn = vread(m + 1);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[m], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        va = vn;
      }
    }

    // ---- end of a piece: finish the sequence or leave a partial ----
    const int nt = s_pref[b + 1] - s_pref[b];
    if (j == nt - 1 || i == n - 1) {
      const bool whole = piece_first == 0 && j == nt - 1;
      if (piece_first == 0 && tid == 0) {
        // the workgroup holding the first tile records which workgroups
        // hold the sequence (for the combine step)
        const int last = owner_of_tile(s_pref[b + 1] - 1, T, W);
        p.seq_meta[2 * b] = w;
        p.seq_meta[2 * b + 1] = last;
      }
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (wave_active && h < p.n_h) {
        if (whole) {
          const float inv = 1.f / l_tot;
          uint16_t* orow = p.out + ((int64_t)b * p.n_h + h) * kDv + 4 * g;
#pragma unroll
          for (int m = 0; m < kDvBlocks; ++m) {
            const uint32_t lo = (uint32_t)dev::f32_to_bf16_rne(acc[m][0] * inv) |
                                ((uint32_t)dev::f32_to_bf16_rne(acc[m][1] * inv) << 16);
            const uint32_t hi = (uint32_t)dev::f32_to_bf16_rne(acc[m][2] * inv) |
                                ((uint32_t)dev::f32_to_bf16_rne(acc[m][3] * inv) << 16);
            *reinterpret_cast<dev::u32x2_t*>(orow + 16 * m) = dev::u32x2_t{lo, hi};
          }
        } else {
          const int64_t prow = (int64_t)(w + b) * p.n_h + h;
          float* po = p.part_o + prow * kDv + 4 * g;
#pragma unroll
          for (int m = 0; m < kDvBlocks; ++m)
            *reinterpret_cast<float4*>(po + 16 * m) = float4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
          if (g == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = float2{m_run, l_tot};
        }
      }
      cur_b = -1;
    }
  }
}

// Merge the pieces of the sequences that were cut across workgroups, and
// zero the output of empty sequences.  One 128-thread workgroup per (b, h);
// thread t owns output columns 4t .. 4t+3.
__global__ void __launch_bounds__(128) mla_combine_kernel(MlaParams p) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  uint16_t* orow = p.out + ((int64_t)b * p.n_h + h) * kDv + 4 * t;
  const int ctx = p.context_lens[b];
  if (ctx <= 0) {
    *reinterpret_cast<dev::u32x2_t*>(orow) = dev::u32x2_t{0u, 0u};
    return;
  }
  const int wf = p.seq_meta[2 * b], wl = p.seq_meta[2 * b + 1];
  if (wf == wl) return;   // finished in place
  float M = -INFINITY;
  for (int s = wf; s <= wl; ++s) M = fmaxf(M, p.part_ml[2 * ((int64_t)(s + b) * p.n_h + h)]);
  float L = 0.f;
  float4 O = {0.f, 0.f, 0.f, 0.f};
  for (int s = wf; s <= wl; ++s) {
    const int64_t prow = (int64_t)(s + b) * p.n_h + h;
    const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + 2 * prow);
    const float f = __builtin_amdgcn_exp2f(ml.x - M);
    L = fmaf(ml.y, f, L);
    const float4 o = *reinterpret_cast<const float4*>(p.part_o + prow * kDv + 4 * t);
    O.x = fmaf(o.x, f, O.x);
    O.y = fmaf(o.y, f, O.y);
    O.z = fmaf(o.z, f, O.z);
    O.w = fmaf(o.w, f, O.w);
  }
  const float inv = 1.f / L;
  const uint32_t lo = (uint32_t)dev::f32_to_bf16_rne(O.x * inv) | ((uint32_t)dev::f32_to_bf16_rne(O.y * inv) << 16);
  const uint32_t hi = (uint32_t)dev::f32_to_bf16_rne(O.z * inv) | ((uint32_t)dev::f32_to_bf16_rne(O.w * inv) << 16);
  *reinterpret_cast<dev::u32x2_t*>(orow) = dev::u32x2_t{lo, hi};
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
  p.part_o = d.part_o;
  p.part_ml = d.part_ml;
  p.seq_meta = d.seq_meta;
  p.scale_log2 = d.scale * kLog2e;
  p.B = d.B;
  p.n_h = d.n_h;
  p.block_shift = d.block_shift;
  p.max_blocks_per_seq = d.max_blocks_per_seq;
  p.W = d.workgroups;
  const dim3 grid((unsigned)p.W, (unsigned)mla_head_groups(p.n_h));
  hipLaunchKernelGGL((decode_mla_kernel<kMlaStages>), grid, dim3(kThreadsM), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)p.B, (unsigned)p.n_h), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
