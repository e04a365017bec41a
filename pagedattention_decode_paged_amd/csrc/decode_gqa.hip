// Paged decode attention for GQA / MQA / MHA on float (bf16, f32) pools.
//
// What is computed: for each sequence b and query head h,
//   out[b][h] = sum_j softmax_j(scale * q[b][h] . K_j) V_j ,  j < context_lens[b],
// where K_j, V_j are reached through the block table (faulkner, first section
// and the logical/physical block mapping; qwbw 3.4) and the g = n_h / n_kv
// query heads of a group share KV head h / g (faulkner's MHA/GQA/MLA table).
//
// How (gfx950, wave64):
// * One workgroup of 4 wavefronts per (context split, KV head, sequence).
//   Every K/V row it reads is used by all g query heads of the group, so the
//   cache is streamed from HBM once per decode step.
// * Score phase: lane i of a wave owns token i of a 64-token tile and holds
//   its whole K row in registers (16 x 16-byte loads for a 256-byte row); q is
//   uniform and read through the scalar path, so the g dot products need no
//   cross-lane reduction (v_dot2 on bf16 pairs, fp32 accumulation).
// * Online softmax per tile in base 2 (scale * log2 e folded into the score):
//   wave max by DPP, running max m and per-lane partial sums l.
// * Value phase: 16 lanes cover one 256-byte V row (fully coalesced 16-byte
//   loads, 4 rows per instruction); the tile's probabilities go through a
//   wave-private LDS slice; fp32 accumulators, g heads x 8 columns per lane.
// * The 4 waves of a workgroup merge their (m, l, acc) in LDS.  With one split
//   per sequence the workgroup writes the output; otherwise it writes a
//   normalised partial (m, l, o) and decode_reduce merges them by log-sum-exp.
// * Tokens at or past the context length are never loaded: their scores are
//   -inf and their V registers are zero, so NaN in unused slots cannot leak.
#include "internal.h"
#include "device_common.h"
#include "decode_epilogue.h"

namespace pkv {
namespace {

using namespace dev;

template <int D, bool BF16>
struct Geo {
  static constexpr int kRowBytes = D * (BF16 ? 2 : 4);
  static constexpr int kRowDw = kRowBytes / 4;       // dwords per row
  static constexpr int kRowQ = kRowBytes / 16;       // 16-byte pieces per row
  static constexpr int kLpr = kRowBytes / 16;        // lanes per row, value phase
  static constexpr int kTpi = kWave / kLpr;          // rows per value load
  static constexpr int kEpl = BF16 ? 8 : 4;          // elements per lane, value phase
  static constexpr int kSteps = kTile / kTpi;        // value loads per tile
  static_assert(kRowBytes == 128 || kRowBytes == 256, "row must be 128 or 256 bytes");
};

// PAIR (bf16 rows, blocks of at least kWave / kRowQ slots): K and V are read
// row-coalesced with one uniform block base per load, K reaches the
// lane-per-token score phase through a swizzled LDS tile, and the value phase
// multiplies token pairs with v_dot2 against bf16 probability pairs.
template <int D, int G, bool BF16, bool PAIR>
__global__ __launch_bounds__(kThreads, 2) void decode_gqa_kernel(const DecodeParams p) {
  using Gm = Geo<D, BF16>;
  static_assert(!PAIR || BF16, "pair mode is for bf16 rows");
  constexpr int kPairs = kTile / 2;                 // token pairs per tile
  constexpr int kGh = (G + 1) / 2;                  // pair dwords written by first lanes
  // value phase: PAIR reads V in 8-byte pieces (kAccLpr lanes per row,
  // kAccTpi rows per load) and pairs token t with t + kAccTpi in one lane
  constexpr int kAccE = PAIR ? 4 : Gm::kEpl;                       // accumulator columns per lane
  constexpr int kAccLpr = PAIR ? Gm::kRowBytes / 8 : Gm::kLpr;     // lanes per V row
  constexpr int kAccTpi = kWave / kAccLpr;                         // V rows per load
  constexpr int kVL = PAIR ? kTile / kAccTpi : Gm::kSteps;         // V loads per tile
  __shared__ __align__(16) int32_t s_bt[kBtSlots];
  __shared__ __align__(16) float s_p[kWaves][PAIR ? 1 : kTile * G];
  __shared__ __align__(16) uint32_t s_pp[kWaves][PAIR ? kPairs * G : 1];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  // PAIR: each wave's K tile (kTile rows) is staged here by direct-to-LDS
  // loads; after the tile loop the same bytes hold the waves' accumulators.
  constexpr int kKBytes = PAIR ? kWaves * kTile * Gm::kRowBytes : 16;
  constexpr int kAccBytes = kWaves * G * D * 4;
  __shared__ __align__(16) uint8_t s_kbuf[kKBytes > kAccBytes ? kKBytes : kAccBytes];
  float (&s_acc)[kWaves][G * D] = *reinterpret_cast<float (*)[kWaves][G * D]>(s_kbuf);

  // grid (KV head, sequence, split), KV head fastest: workgroups are dealt
  // to the 8 XCDs round-robin by linear index, so each XCD serves whole KV
  // heads (identical work) whatever the context lengths and split count
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int split = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ctx = p.context_lens[b];
  const int t_begin = split * p.split_tokens;
  const int n_h = p.n_h;

  if (t_begin >= ctx) {
    if (split == 0) write_zero_rows<G, D>(p, b, kvh);   // empty sequence
    return;
  }
  const int t_end = min(ctx, t_begin + p.split_tokens);
  const int shift = p.block_shift;
  const int bmask = (1 << shift) - 1;

  // Stage this split's slice of the block table (only entries it will use).
  const int lb0 = t_begin >> shift;
  {
    const int nblk = ((t_end - 1) >> shift) - lb0 + 1;
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq + lb0;
    for (int i = tid; i < nblk; i += kThreads) s_bt[i] = row[i];
  }
  __syncthreads();

  const int64_t slot_stride = (int64_t)p.n_kv * Gm::kRowBytes;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)kvh * Gm::kRowBytes;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)kvh * Gm::kRowBytes;
  const float qscale = p.scale * kLog2e;

  auto row_addr = [&](const uint8_t* base, int t) -> const uint8_t* {
    const int32_t phys = s_bt[(t >> shift) - lb0];
    const int64_t slot = ((int64_t)phys << shift) + (t & bmask);
    return base + slot * slot_stride;
  };

  // First dword of the group's q rows (q rows are contiguous per sequence).
  const int64_t q_dw0 = ((int64_t)b * n_h + (int64_t)kvh * G) * Gm::kRowDw;

  float m_run[G], l_run[G];
  float acc[G][kAccE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < kAccE; ++e) acc[h][e] = 0.f;
  }

  const int vj = lane / kAccLpr;       // row within a value load
  const int ve = lane % kAccLpr;       // piece within the row

  u32x4_t kreg[Gm::kRowQ];
  int tile_start = t_begin + wave * kTile;

  // PAIR: K rows are loaded row-coalesced (kRpi rows of kPr 16-byte pieces
  // per instruction, one block per instruction) into kreg, stored to this
  // wave's LDS tile with row r's piece P in slot P ^ swz(r), and read back
  // one token row per lane; both LDS passes touch every bank once per 16
  // lanes.  Rows past the context re-read the last valid row (finite data
  // that gets a masked score and probability 0).
  constexpr int kPr = Gm::kRowQ;                    // 16-byte pieces per row
  constexpr int kRpi = kWave / kPr;                 // rows per load instruction
  constexpr int kRows256 = 256 / Gm::kRowBytes;     // rows per 256 bytes of LDS
  uint8_t* const kl = s_kbuf + (PAIR ? wave * kTile * Gm::kRowBytes : 0);
  const int lj = lane / kPr, le = lane % kPr;
  auto swz = [](int r) { return (r / kRows256) % kPr; };
  const int t_last = t_end - 1;
  auto load_k_rows = [&](int ts) {
#pragma unroll
    for (int k = 0; k < kPr; ++k) {
      const int tg = min(ts + k * kRpi, t_last);    // first (valid) token of the instruction
      const int32_t phys = __builtin_amdgcn_readfirstlane(s_bt[(tg >> shift) - lb0]);
      const uint8_t* gb = kbase + ((int64_t)phys << shift) * slot_stride;
      const int tr = min(ts + k * kRpi + lj, t_last);
      kreg[k] = *reinterpret_cast<const u32x4_t*>(gb + (uint32_t)(tr & bmask) * (uint32_t)slot_stride + (uint32_t)le * 16u);
    }
  };

  if constexpr (PAIR) {
    if (tile_start < t_end) load_k_rows(tile_start);
  } else if (tile_start < t_end) {
    const int t = tile_start + lane;
    if (t < t_end) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(row_addr(kbase, t));
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
    }
  }

  for (; tile_start < t_end; tile_start += kWaves * kTile) {
    if constexpr (PAIR) {
      // rows -> swizzled LDS tile -> this lane's token row
#pragma unroll
      for (int k = 0; k < kPr; ++k) {
        const int r = k * kRpi + lj;
        *reinterpret_cast<u32x4_t*>(kl + r * Gm::kRowBytes + ((le ^ swz(r)) * 16)) = kreg[k];
      }
      wave_sync_lds();
      int sw = swz(lane);
      asm volatile("" : "+v"(sw));          // keep the 16 addresses out of the loop preheader
      const uint8_t* krow = kl + lane * Gm::kRowBytes;
#pragma unroll
      for (int i = 0; i < kPr; ++i)
        kreg[i] = *reinterpret_cast<const u32x4_t*>(krow + ((i ^ sw) * 16));
    }

    // ---- issue the value loads of this tile (they fly during the scores)
    uint4 vreg[PAIR ? 1 : Gm::kSteps];
    u32x2_t vreg2[PAIR ? kVL : 1];
    if constexpr (PAIR) {
      // load k covers rows k*kAccTpi .. +kAccTpi-1 of the tile (one block)
#pragma unroll
      for (int k = 0; k < kVL; ++k) {
        const int t_grp = min(tile_start + k * kAccTpi, t_last);
        const int32_t phys = __builtin_amdgcn_readfirstlane(s_bt[(t_grp >> shift) - lb0]);
        const uint8_t* gbase = vbase + ((int64_t)phys << shift) * slot_stride;
        const int t = min(tile_start + k * kAccTpi + vj, t_last);
        vreg2[k] = *reinterpret_cast<const u32x2_t*>(gbase + (uint32_t)(t & bmask) * (uint32_t)slot_stride + (uint32_t)ve * 8u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < Gm::kSteps; ++k) {
        const int t = tile_start + k * Gm::kTpi + vj;
        if (t < t_end) vreg[k] = reinterpret_cast<const uint4*>(row_addr(vbase, t))[ve];
        else vreg[k] = make_uint4(0, 0, 0, 0);
      }
    }


    // ---- scores of this lane's token for the G heads
    // q is uniform and never written here, so it is read with scalar loads
    // through the constant address space, in 16-dword chunks, one chunk ahead
    // of its use.  The base address is made opaque and tied to the running
    // dot products (below): otherwise every q value of the group (G * D / 2
    // dwords) is hoisted into SGPRs and spilled.  Chunk offsets are constants
    // folded into the scalar loads.
    const int my_t = tile_start + lane;
    const bool valid = my_t < t_end;
    float s[G];
    {
      using QPtr = const __attribute__((address_space(4))) uint32_t*;
      constexpr int kQch = 16;
      constexpr int kCph = Gm::kRowDw / kQch;       // chunks per head
      constexpr int kNch = G * kCph;
      float ax[G], ay[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { ax[h] = 0.f; ay[h] = 0.f; }
      uintptr_t qaddr = (uintptr_t)p.q + (uintptr_t)q_dw0 * 4u;
      asm volatile("" : "+s"(qaddr));
      uint32_t qa[kQch], qb[kQch];
      auto load_chunk = [&](uint32_t (&dst)[kQch], int c) {
        const QPtr qp = (QPtr)qaddr;
        const int off = (c / kCph) * Gm::kRowDw + (c % kCph) * kQch;   // immediate offset
#pragma unroll
        for (int i = 0; i < kQch; ++i) dst[i] = qp[off + i];
      };
      load_chunk(qa, 0);
#pragma unroll
      for (int c = 0; c < kNch; ++c) {
        // The address of chunk c + 1 depends on the accumulator finished by
        // chunk c - 1, so at most two chunks of q are live in SGPRs.
        if (c > 0) {
          const int hp = (c - 1) / kCph;
          asm volatile("" : "+s"(qaddr) : "v"(ax[hp]), "v"(ay[hp]));
        }
        if (c + 1 < kNch) load_chunk(qb, c + 1);
        const int h = c / kCph;
        const int w0 = (c % kCph) * kQch;
#pragma unroll
        for (int i = 0; i < kQch; i += 2) {
          const uint32_t k0 = kdw(kreg, w0 + i);
          const uint32_t k1 = kdw(kreg, w0 + i + 1);
          if constexpr (BF16) {
            ax[h] = dot2_bf16(qa[i], k0, ax[h]);
            ay[h] = dot2_bf16(qa[i + 1], k1, ay[h]);
          } else {
            ax[h] = fmaf(__uint_as_float(qa[i]), __uint_as_float(k0), ax[h]);
            ay[h] = fmaf(__uint_as_float(qa[i + 1]), __uint_as_float(k1), ay[h]);
          }
        }
#pragma unroll
        for (int i = 0; i < kQch; ++i) qa[i] = qb[i];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = valid ? (ax[h] + ay[h]) * qscale : -INFINITY;
    }

    // ---- prefetch the next tile's K rows (the registers are free now)
    const int next = tile_start + kWaves * kTile;
    if constexpr (PAIR) {
      if (next < t_end) load_k_rows(next);
    } else if (next < t_end) {
      const int t = next + lane;
      if (t < t_end) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(row_addr(kbase, t));
#pragma unroll
        for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = src[i];
      } else {
#pragma unroll
        for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }

    // ---- online softmax update (base 2); the rescale is skipped while the
    // running maximum of a head does not move
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tmax = wave_max(s[h]);           // finite: token tile_start is valid
      if (tmax > m_run[h]) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - tmax);
        l_run[h] *= alpha;
#pragma unroll
        for (int e = 0; e < kAccE; ++e) acc[h][e] *= alpha;
        m_run[h] = tmax;
      }
      const float pr = __builtin_amdgcn_exp2f(s[h] - m_run[h]);
      l_run[h] += pr;
      s[h] = pr;
    }

    if constexpr (PAIR) {
      // bf16 probability pairs of tokens (t, t + kAccTpi): the first lane of a
      // pair packs heads [0, kGh), the second heads [kGh, G), exchanging
      // values with its partner lane t ^ kAccTpi; pair id of token t is
      // (t / (2 kAccTpi)) * kAccTpi + t % kAccTpi
      const bool first = ((lane / kAccTpi) & 1) == 0;
      uint32_t packed[kGh];
#pragma unroll
      for (int j = 0; j < kGh; ++j) {
        const int ho = kGh + j;
        const float mine_e = s[j];
        const float mine_o = ho < G ? s[ho < G ? ho : 0] : 0.f;
        const float send = first ? mine_o : mine_e;
        float recv;
        if constexpr (kAccTpi == 2) recv = dpp<0x4E>(send);                 // quad_perm [2,3,0,1]
        else recv = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x101F));  // lane ^ 4
        const float keep = first ? mine_e : mine_o;
        typedef float f2_t __attribute__((ext_vector_type(2)));
        const f2_t v2 = {first ? keep : recv, first ? recv : keep};
        packed[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2_t));
      }
      const int pid = (lane / (2 * kAccTpi)) * kAccTpi + lane % kAccTpi;
      uint32_t* dst = &s_pp[wave][pid * G + (first ? 0 : kGh)];
      const int nw = first ? kGh : G - kGh;
#pragma unroll
      for (int j = 0; j < kGh; ++j)
        if (j < nw) dst[j] = packed[j];
      wave_sync_lds();

      // ---- acc += p * V over token pairs: (p_t0, p_t1) . (V_t0[e], V_t1[e])
#pragma unroll
      for (int m = 0; m < kVL / 2; ++m) {
        const int i = m * kAccTpi + vj;            // pair id of tokens 2m*kAccTpi + vj, +kAccTpi
        uint32_t pp[G];
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h = 0; h < G; h += 4) {
            const uint4 v4 = *reinterpret_cast<const uint4*>(&s_pp[wave][i * G + h]);
            pp[h] = v4.x; pp[h + 1] = v4.y; pp[h + 2] = v4.z; pp[h + 3] = v4.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pp[h] = s_pp[wave][i * G + h];
        }
        const u32x2_t a = vreg2[2 * m], c = vreg2[2 * m + 1];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t lo = __builtin_amdgcn_perm(c[x], a[x], 0x05040100u);   // (V_t0[2x], V_t1[2x])
          const uint32_t hi = __builtin_amdgcn_perm(c[x], a[x], 0x07060302u);   // (V_t0[2x+1], V_t1[2x+1])
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][2 * x] = dot2_bf16(pp[h], lo, acc[h][2 * x]);
            acc[h][2 * x + 1] = dot2_bf16(pp[h], hi, acc[h][2 * x + 1]);
          }
        }
      }
      wave_sync_lds();   // s_pp is rewritten by the next tile
    } else {
      if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h = 0; h < G; h += 4)
          *reinterpret_cast<float4*>(&s_p[wave][lane * G + h]) = make_float4(s[h], s[h + 1], s[h + 2], s[h + 3]);
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) s_p[wave][lane * G + h] = s[h];
      }
      wave_sync_lds();

      // ---- acc += p * V
#pragma unroll
      for (int k = 0; k < Gm::kSteps; ++k) {
        const int i = k * Gm::kTpi + vj;
        float pr[G];
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h = 0; h < G; h += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(&s_p[wave][i * G + h]);
            pr[h] = v4.x; pr[h + 1] = v4.y; pr[h + 2] = v4.z; pr[h + 3] = v4.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pr[h] = s_p[wave][i * G + h];
        }
        float v[Gm::kEpl];
        if constexpr (BF16) {
          const uint32_t w[4] = {vreg[k].x, vreg[k].y, vreg[k].z, vreg[k].w};
#pragma unroll
          for (int x = 0; x < 4; ++x) { v[2 * x] = bf_lo(w[x]); v[2 * x + 1] = bf_hi(w[x]); }
        } else {
          v[0] = __uint_as_float(vreg[k].x); v[1] = __uint_as_float(vreg[k].y);
          v[2] = __uint_as_float(vreg[k].z); v[3] = __uint_as_float(vreg[k].w);
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < Gm::kEpl; ++e) acc[h][e] = fmaf(pr[h], v[e], acc[h][e]);
      }
      wave_sync_lds();   // s_p is rewritten by the next tile
    }
  }

  // every wave has left the tile loop before s_acc (aliasing the K staging
  // area) is written
  __syncthreads();

  // ---- merge within the wave: rows sharing a 16-byte piece, and the sums
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = wave_sum(l_run[h]);
#pragma unroll
    for (int e = 0; e < kAccE; ++e) {
#pragma unroll
      for (int off = kAccLpr; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_m[wave][h] = m_run[h]; s_l[wave][h] = l_run[h]; }
  }
  if (vj == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < kAccE; ++e) s_acc[wave][h * D + ve * kAccE + e] = acc[h][e];
  }
  __syncthreads();
  finish_split<G, D>(p, b, kvh, split, ctx, s_m, s_l, s_acc);
}

// Log-sum-exp merge of split partials (the split-context reduction that
// qwbw 8 Q2/Q3 name FlashDecoding): with M the largest split maximum (scores
// in base 2), out = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per (sequence, query head), kReduceWaves of them per
// workgroup.  The first batch of partials is loaded before the context
// length arrives (every split the launch has is inside the workspace, and
// splits past the sequence's own count are discarded by selects, never
// multiplied), so the kernel costs about one memory round trip.
constexpr int kReduceThreads = 64;
constexpr int kReduceWaves = 4;
constexpr int kMaxSplits = 1024;
constexpr int kFewSplits = 8;       // splits whose loads are issued together (d_v <= 128)

__global__ __launch_bounds__(kReduceThreads * kReduceWaves) void decode_reduce_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ context_lens, void* __restrict__ out, int rows, int n_h, int d_v,
    int num_splits, int split_tokens, int out_bf16, int window) {
  const int bh = blockIdx.x * kReduceWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kReduceThreads);
  if (bh >= rows) return;
  const int b = bh / n_h;
  const int lane = threadIdx.x % kReduceThreads;
  const int64_t base = (int64_t)bh * num_splits;
  const float* ml = part_ml + 2 * base;
  const float* po = part_o + base * d_v + lane;
  const bool c0 = lane < d_v, c1 = lane + kReduceThreads < d_v;
  // split s of this row into slot k of the batch (defaults past lim)
#define PKV_REDUCE_LOAD(s, k, lim)                                    \
  do {                                                                \
    if ((s) < (lim)) {                                                \
      m[k] = ml[2 * (s)];                                             \
      l[k] = ml[2 * (s) + 1];                                         \
      v0[k] = c0 ? po[(int64_t)(s) * d_v] : 0.f;                      \
      v1[k] = c1 ? po[(int64_t)(s) * d_v + kReduceThreads] : 0.f;     \
    } else {                                                          \
      m[k] = -INFINITY;                                               \
      l[k] = 0.f;                                                     \
      v0[k] = v1[k] = 0.f;                                            \
    }                                                                 \
  } while (0)
  float m[kFewSplits], l[kFewSplits], v0[kFewSplits], v1[kFewSplits];
#pragma unroll
  for (int k = 0; k < kFewSplits; ++k) PKV_REDUCE_LOAD(k, k, num_splits);   // in flight with ctx
  const int ctx = context_lens[b];
  const int a0 = window > 0 ? max(ctx - window, 0) & ~15 : 0;   // first position read (sliding window)
  const int nsp = min(num_splits, (ctx - a0 + split_tokens - 1) / split_tokens);
  if (nsp <= 1) return;                 // written by the decode kernel itself
  // batches of kFewSplits splits merged online (running max M, sum L, outputs o)
  float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += kFewSplits) {
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < kFewSplits; ++k) PKV_REDUCE_LOAD(s0 + k, k, nsp);
    }
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
      const bool in = s0 + k < nsp;
      m[k] = in ? m[k] : -INFINITY;
      l[k] = in ? l[k] : 0.f;
      v0[k] = in ? v0[k] : 0.f;
      v1[k] = in ? v1[k] : 0.f;
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) Mb = fmaxf(Mb, m[k]);
    const float f = __builtin_amdgcn_exp2f(M - Mb);   // 0 for the first batch
    L *= f;
    o0 *= f;
    o1 *= f;
    M = Mb;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
      const float w = l[k] * __builtin_amdgcn_exp2f(m[k] - M);   // 0 past the last split
      L += w;
      o0 = fmaf(v0[k], w, o0);
      o1 = fmaf(v1[k], w, o1);
    }
  }
#undef PKV_REDUCE_LOAD
  const float inv = 1.0f / L;
  const int64_t o = (int64_t)bh * d_v + lane;
  if (out_bf16) {
    if (c0) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(o0 * inv);
    if (c1) reinterpret_cast<uint16_t*>(out)[o + kReduceThreads] = f32_to_bf16_rne(o1 * inv);
  } else {
    if (c0) reinterpret_cast<float*>(out)[o] = o0 * inv;
    if (c1) reinterpret_cast<float*>(out)[o + kReduceThreads] = o1 * inv;
  }
}

// The same merge for the LDS-ring kernel's stream grid: row (b, h) takes the
// pieces j + b of workgroups j = jf .. jl, [jf, jl] = seq_meta[b].  Without
// a shared prefix, jf == jl means nothing to merge (the sequence was written
// whole, or is empty).  With one (prefix_tokens > 0) every sequence with
// tokens is merged: first its prefix pieces stream_wgs + B + c * B + b for
// the chunks c < ceil(min(ctx, prefix_tokens) / prefix_chunk), then its
// stream pieces [jf, jl] (none when jl < jf).  Piece p's partials sit at row
// p * n_h + h.
__global__ __launch_bounds__(kReduceThreads * kReduceWaves) void decode_reduce_stream_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_meta, const int32_t* __restrict__ context_lens, void* __restrict__ out,
    int rows, int n_h, int d_v, int out_bf16, int B, int stream_wgs, int prefix_tokens, int prefix_chunk,
    int block_shift) {
  const int bh = blockIdx.x * kReduceWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kReduceThreads);
  if (bh >= rows) return;
  const int b = bh / n_h, h = bh % n_h;
  const int lane = threadIdx.x % kReduceThreads;
  const int jf = seq_meta[2 * b], jl = seq_meta[2 * b + 1];
  int npre = 0;
  if (prefix_tokens > 0) {
    const int ctx = context_lens[b];
    if (ctx <= 0) return;                       // zeroed by the decode kernel
    npre = (prefix_end(ctx, prefix_tokens, block_shift) + prefix_chunk - 1) / prefix_chunk;
  } else if (jl <= jf) {
    return;
  }
  const int n = npre + (jl >= jf ? jl - jf + 1 : 0);
  const int64_t pre0 = (int64_t)stream_wgs + B;
  const bool c0 = lane < d_v, c1 = lane + kReduceThreads < d_v;
  float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int k0 = 0; k0 < n; k0 += kFewSplits) {
    float m[kFewSplits], l[kFewSplits], v0[kFewSplits], v1[kFewSplits];
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
      const int kk = k0 + k;
      const bool in = kk < n;
      const int64_t piece = kk < npre ? pre0 + (int64_t)kk * B + b : (int64_t)(jf + kk - npre + b);
      const int64_t pi = piece * n_h + h;
      m[k] = in ? part_ml[2 * pi] : -INFINITY;
      l[k] = in ? part_ml[2 * pi + 1] : 0.f;
      v0[k] = in && c0 ? part_o[pi * d_v + lane] : 0.f;
      v1[k] = in && c1 ? part_o[pi * d_v + lane + kReduceThreads] : 0.f;
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) Mb = fmaxf(Mb, m[k]);
    const float f = __builtin_amdgcn_exp2f(M - Mb);   // 0 for the first batch
    L *= f;
    o0 *= f;
    o1 *= f;
    M = Mb;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
      const float w = l[k] * __builtin_amdgcn_exp2f(m[k] - M);   // 0 past the last piece
      L += w;
      o0 = fmaf(v0[k], w, o0);
      o1 = fmaf(v1[k], w, o1);
    }
  }
  const float inv = 1.0f / L;
  const int64_t o = (int64_t)bh * d_v + lane;
  if (out_bf16) {
    if (c0) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(o0 * inv);
    if (c1) reinterpret_cast<uint16_t*>(out)[o + kReduceThreads] = f32_to_bf16_rne(o1 * inv);
  } else {
    if (c0) reinterpret_cast<float*>(out)[o] = o0 * inv;
    if (c1) reinterpret_cast<float*>(out)[o + kReduceThreads] = o1 * inv;
  }
}

template <int D, int G, bool BF16, bool PAIR>
hipError_t launch_inst(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.n_kv, (unsigned)p.B, (unsigned)p.num_splits);
  hipLaunchKernelGGL((decode_gqa_kernel<D, G, BF16, PAIR>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool BF16, bool PAIR>
hipError_t dispatch_g(const DecodeParams& p, int g, hipStream_t stream) {
  switch (g) {
    case 1: return launch_inst<D, 1, BF16, PAIR>(p, stream);
    case 2: return launch_inst<D, 2, BF16, PAIR>(p, stream);
    case 4: return launch_inst<D, 4, BF16, PAIR>(p, stream);
    case 8: return launch_inst<D, 8, BF16, PAIR>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// Pair mode needs the rows of every K load (kWave / kRowQ of them) inside
// one block (the V loads cover fewer rows).
template <int D>
bool pair_ok(const DecodeParams& p) {
  return (1 << p.block_shift) >= kWave / Geo<D, true>::kRowQ;
}

}  // namespace

bool gqa_supported(KV kv, bool q_bf16, int d_k, int d_v, int g) {
  if (d_k != d_v) return false;
  if (g == 16) return gqa_ring_supported(kv, q_bf16, d_k, d_v, g);   // the LDS-ring kernel only
  if (!(g == 1 || g == 2 || g == 4 || g == 8)) return false;
  if (kv == KV::BF16) return q_bf16 && (d_k == 64 || d_k == 128);
  if (kv == KV::F32) return !q_bf16 && (d_k == 32 || d_k == 64);
  if (kv == KV::INT8) return int8_supported(q_bf16, d_k, d_v, g);
  if (kv == KV::INT4) return gqa_ring_supported(kv, q_bf16, d_k, d_v, g);
  return false;
}

hipError_t launch_decode_gqa(const DecodeParams& p, hipStream_t stream) {
  if (p.split_tokens > kMaxSplitTokens || p.split_tokens % kGqaSplitGranule ||
      (p.split_tokens >> p.block_shift) > kBtSlots)
    return hipErrorInvalidValue;
  const int g = p.n_h / p.n_kv;
  // only the bf16 and INT8 LDS-ring kernels write appended rows themselves
  if (p.k_new && !((p.kv == KV::BF16 || (p.kv == KV::INT8 && p.q_bf16)) &&
                   gqa_ring_supported(p.kv, p.q_bf16, p.d_k, p.d_v, g)))
    return hipErrorInvalidValue;
  // the stream grid and the sliding window exist on the LDS-ring kernel only
  if ((p.stream_wgs != 0 || p.window != 0) && !gqa_ring_supported(p.kv, p.q_bf16, p.d_k, p.d_v, g))
    return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  if (gqa_ring_supported(p.kv, p.q_bf16, p.d_k, p.d_v, g)) {
    e = launch_decode_gqa_ring(p, stream);
  } else if (p.kv == KV::BF16) {
    if (p.d_k == 128) e = pair_ok<128>(p) ? dispatch_g<128, true, true>(p, g, stream)
                                          : dispatch_g<128, true, false>(p, g, stream);
    else if (p.d_k == 64) e = pair_ok<64>(p) ? dispatch_g<64, true, true>(p, g, stream)
                                             : dispatch_g<64, true, false>(p, g, stream);
  } else if (p.kv == KV::F32) {
    if (p.d_k == 64) e = dispatch_g<64, false, false>(p, g, stream);
    else if (p.d_k == 32) e = dispatch_g<32, false, false>(p, g, stream);
  } else if (p.kv == KV::INT8) {
    e = launch_decode_int8(p, g, stream);
  }
  const int rows = p.B * p.n_h;
  if (e == hipSuccess && p.stream_wgs != 0) {
    hipLaunchKernelGGL(decode_reduce_stream_kernel, dim3((unsigned)((rows + kReduceWaves - 1) / kReduceWaves)),
                       dim3(kReduceThreads * kReduceWaves), 0, stream, (const float*)p.part_o,
                       (const float*)p.part_ml, (const int32_t*)p.seq_meta, p.context_lens, p.out, rows,
                       p.n_h, p.d_v, p.q_bf16 ? 1 : 0, p.B, p.stream_wgs, p.prefix_tokens, p.prefix_chunk,
                       p.block_shift);
    return hipGetLastError();
  }
  if (e != hipSuccess || p.num_splits == 1) return e;
  if (p.num_splits > kMaxSplits) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((rows + kReduceWaves - 1) / kReduceWaves)),
                     dim3(kReduceThreads * kReduceWaves), 0, stream, (const float*)p.part_o,
                     (const float*)p.part_ml, p.context_lens, p.out, rows, p.n_h, p.d_v, p.num_splits,
                     p.split_tokens, p.q_bf16 ? 1 : 0, p.window);
  return hipGetLastError();
}

}  // namespace pkv
