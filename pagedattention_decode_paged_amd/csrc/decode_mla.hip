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
// every compute unit equally busy.  A workgroup owns 128 heads (4 waves x
// 32) of one head group.  A sequence whose tiles all fall in one range is
// finished in place; a sequence cut by range boundaries leaves one fp32
// partial (running max, sum, unnormalised output) per piece, at slot w + b
// (unique because w + b grows along the staircase of (workgroup, sequence)
// pairs), and mla_combine merges the pieces by log-sum-exp.
//
// Per 32-token tile (one LDS stage, rows swizzled against bank conflicts):
//   S^T = K Q^T        A = K rows from LDS, B = Q^T kept in registers
//   online softmax     on the accumulator layout: head = lane % 32
//   O^T += V^T P^T     A = V^T through the LDS transpose read, B = P taken
//                      straight from the S^T registers
// The K and V operands are the same LDS tile; the tile comes in through the
// LDS DMA path (global_load_lds_dwordx4), NS stages deep, issued and awaited
// with explicit vmcnt counts so that loads of later tiles stay in flight
// while the current one is computed.
#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace {

using dev::kLog2e;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDk * 2;                    // 1152
constexpr int kRowChunks = kRowBytes / 16;            // 72 16-byte chunks per row
constexpr int kTileTok = kMlaTileTokens;              // 32
constexpr int kStageBytes = kTileTok * kRowBytes;     // 36864
constexpr int kWavesM = 4;
constexpr int kThreadsM = 64 * kWavesM;
constexpr int kHeadsPerWave = 32;
constexpr int kHeadsPerGroup = kHeadsPerWave * kWavesM;
constexpr int kDmaPerWave = kTileTok * kRowChunks / 64 / kWavesM;   // 9
constexpr int kKSteps = kDk / 16;                     // 36 score MFMAs per tile
constexpr int kDvTiles = kDv / 32;                    // 16 value MFMA columns
constexpr int kTileCap = 512;                         // tiles whose block ids sit in LDS at once
constexpr float kRescaleSlack = 8.f;                  // log2 units a stale max may lag by

static_assert(kTileTok * kRowChunks % (64 * kWavesM) == 0, "stage must split evenly over the waves");
static_assert(kRowChunks % 8 == 0, "the swizzle permutes chunks within aligned groups of 8");

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

// Chunk permutation of row t inside each aligned group of 8 chunks.  With
// it, the 16-byte K reads (32 rows, one chunk column) and the transposed
// 8-byte V reads (4 rows x 2 chunks per 16 lanes) hit distinct banks.
__device__ __forceinline__ int swz(int t) {
  return ((((t & 3) << 1) | ((t >> 2) & 1)) ^ (((t >> 3) & 1) << 1));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most k tiles of this wave's LDS DMA are still in flight.
template <int NS>
__device__ __forceinline__ void wait_tiles(int k) {
  static_assert(NS >= 2 && NS <= 4, "stage count");
  if constexpr (NS >= 4) {
    if (k >= 2) { wait_vmcnt<2 * kDmaPerWave>(); return; }
  }
  if constexpr (NS >= 3) {
    if (k >= 1) { wait_vmcnt<kDmaPerWave>(); return; }
  }
  wait_vmcnt<0>();
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One tile's block ids and fill, staged in LDS for the DMA issue.
struct TileInfo {
  int32_t blk0, blk1;       // physical blocks of rows [0, 16) and [16, 32) when block_size is 16
  int32_t nvalid_row0;      // valid rows | first row inside blk0 << 8
  int32_t seq;
};

// Issue this wave's share of the LDS DMA for one tile: chunk position P of
// the stage (64 per instruction) holds logical chunk c of row t.  Rows at or
// beyond the context are loaded from the last valid row, so that masked
// tokens multiply finite values by zero.
__device__ __forceinline__ void issue_tile(const MlaParams& p, uint32_t stage_lds, const TileInfo ti,
                                           const uint32_t (&dma_rc)[kDmaPerWave], int wave) {
  const int nvalid = ti.nvalid_row0 & 0xff;
  const int row0 = ti.nvalid_row0 >> 8;
  const int bs_mask = (1 << p.block_shift) - 1;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int t = (int)(dma_rc[i] >> 16);
    const uint32_t cbyte = dma_rc[i] & 0xffffu;
    const int tt = min(t, nvalid - 1);
    const int rf = row0 + tt;
    const uint32_t blk = (uint32_t)(rf > bs_mask ? ti.blk1 : ti.blk0);
    const uint32_t slot = (blk << p.block_shift) | (uint32_t)(rf & bs_mask);
    const uint8_t* src = p.pool + (uint64_t)slot * kRowBytes + cbyte;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)((wave * kDmaPerWave + i) * 1024));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(m0), "v"(src) : "memory", "m0");
  }
}

// Global tile x -> (sequence, tile in sequence) by binary search of the
// tile prefix (s_pref[b] <= x < s_pref[b + 1]; sequence b then has a tile).
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
  __shared__ int32_t s_ctx[kMlaMaxBatch];
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
    for (int b = lo; b < hi; ++b) {
      const int c = p.context_lens[b];
      s_ctx[b] = c;
      sum += (c + kTileTok - 1) / kTileTok;
    }
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
      run += (s_ctx[b] + kTileTok - 1) / kTileTok;
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

  // ---- per-lane constants ----
  const int hi32 = lane >> 5, l32 = lane & 31;
  uint32_t dma_rc[kDmaPerWave];            // row << 16 | byte offset of the chunk in the row
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int P = (wave * kDmaPerWave + i) * 64 + lane;
    const int t = P / kRowChunks, pc = P - t * kRowChunks;
    const int c = (pc & ~7) | ((pc & 7) ^ swz(t));
    dma_rc[i] = ((uint32_t)t << 16) | (uint32_t)(c * 16);
  }
  // K operand: row l32, logical chunk 2*ks + hi32.
  uint32_t koff[4];
  {
    const int x = hi32 ^ swz(l32);
#pragma unroll
    for (int k = 0; k < 4; ++k) koff[k] = l32 * kRowBytes + 16 * (x ^ (2 * k));
  }
  // V^T operand (transposed 8-byte reads): 16-lane group g reads rows
  // 16j + 8p + 4(g/2) + r/4, elements 32n + 16(g%2) + 4(r%4) .. +3.
  uint32_t voff[4];
  {
    const int g = lane >> 4, r = lane & 15;
    const int row = 4 * (g >> 1) + (r >> 2);
    const int y = (2 * (g & 1)) ^ ((r & 3) >> 1) ^ ((r >> 2) << 1) ^ (g >> 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) voff[k] = row * kRowBytes + 8 * (r & 1) + 16 * (y ^ (2 * k));
  }
  const uint32_t stage0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)s_stage;

  // ---- block ids of the next tiles, staged in LDS ----
  int c0 = start;
  auto fill_tiles = [&](int first) {
    const int cnt = min(kTileCap + NS, end - first);
    for (int k = tid; k < cnt; k += kThreadsM) {
      const int x = first + k;
      const int b = seq_of_tile(s_pref, B, x);
      const int tok0 = (x - s_pref[b]) * kTileTok;
      const int nvalid = min(kTileTok, s_ctx[b] - tok0);
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
    if (s < n) issue_tile(p, stage0 + s * kStageBytes, s_tile[s], dma_rc, wave);

  bf16x8_t qf[kKSteps];
  f32x16_t acc[kDvTiles];
  float m_run = -INFINITY, l_run = 0.f;
  int piece_first = 0;        // tile index in the sequence where this piece began
  int cur_b = -1;

  for (int i = 0; i < n; ++i) {
    const int x = start + i;
    wait_tiles<NS>(min(NS - 2, n - 1 - i));
    block_barrier();
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

    if (b != cur_b) {           // a new piece: load this sequence's queries
      cur_b = b;
      piece_first = j;
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int n2 = 0; n2 < kDvTiles; ++n2) acc[n2] = f32x16_t{};
      const int h = hbase + l32;
      if (h < p.n_h) {
        const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(
            p.q + ((int64_t)b * p.n_h + h) * kDk + 8 * hi32);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = qp[2 * ks];
      } else {
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = bf16x8_t{};
      }
    }

    f32x16_t s = {};
    if (wave_active) {
      // S^T = K Q^T over the 36 k-steps of the 576-wide row.
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8_t kf = *(const lds_bf16x8_t*)(uintptr_t)(stage + koff[ks & 3] + 128 * (ks >> 2));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
      }
    }

    // Stage (i - 1) % NS is free once every wave passed this tile's barrier.
    if (i + NS - 1 < n)
      issue_tile(p, stage0 + (uint32_t)(((i + NS - 1) % NS) * kStageBytes),
                 s_tile[x + NS - 1 - c0], dma_rc, wave);

    if (wave_active) {
      // ---- online softmax on the accumulator layout (base 2) ----
      float xv[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = 8 * (r >> 2) + 4 * hi32 + (r & 3);
        const float v = tok < nvalid ? s[r] * p.scale_log2 : -INFINITY;
        xv[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (m_run == -INFINITY) {
        m_run = mx;             // first tile of the piece: nothing accumulated yet
      } else if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int n2 = 0; n2 < kDvTiles; ++n2) {
          acc[n2] *= alpha;
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run *= alpha;
        m_run = m_new;
      }
      bf16x8_t pb[2];
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(xv[r] - m_run);
        pb[r >> 3][r & 7] = pr;
        lsum += (float)pr;
      }
      l_run += lsum;

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int n2 = 0; n2 < kDvTiles; ++n2) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t a0 = stage + voff[2 * (n2 & 1)] + (16 * jj) * kRowBytes + 128 * (n2 >> 1);
          const uint32_t a1 = stage + voff[2 * (n2 & 1) + 1] + (16 * jj + 8) * kRowBytes + 128 * (n2 >> 1);
          const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a0);
          const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a1);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[n2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[jj], acc[n2], 0, 0, 0);
        }
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
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const int h = hbase + l32;
      if (wave_active && h < p.n_h) {
        if (whole) {
          const float inv = 1.f / l_tot;
          uint16_t* orow = p.out + ((int64_t)b * p.n_h + h) * kDv + 4 * hi32;
#pragma unroll
          for (int n2 = 0; n2 < kDvTiles; ++n2) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const uint32_t lo = (uint32_t)dev::f32_to_bf16_rne(acc[n2][4 * q4] * inv) |
                                  ((uint32_t)dev::f32_to_bf16_rne(acc[n2][4 * q4 + 1] * inv) << 16);
              const uint32_t hi = (uint32_t)dev::f32_to_bf16_rne(acc[n2][4 * q4 + 2] * inv) |
                                  ((uint32_t)dev::f32_to_bf16_rne(acc[n2][4 * q4 + 3] * inv) << 16);
              *reinterpret_cast<dev::u32x2_t*>(orow + 32 * n2 + 8 * q4) = dev::u32x2_t{lo, hi};
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          const int64_t prow = (int64_t)(w + b) * p.n_h + h;
          float* po = p.part_o + prow * kDv + 4 * hi32;
#pragma unroll
          for (int n2 = 0; n2 < kDvTiles; ++n2) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              *reinterpret_cast<float4*>(po + 32 * n2 + 8 * q4) =
                  float4{acc[n2][4 * q4], acc[n2][4 * q4 + 1], acc[n2][4 * q4 + 2], acc[n2][4 * q4 + 3]};
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if (hi32 == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * prow) = float2{m_run, l_tot};
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
