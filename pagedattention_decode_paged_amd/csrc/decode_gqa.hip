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

template <int D, int G, bool BF16>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(const DecodeParams p) {
  using Gm = Geo<D, BF16>;
  __shared__ __align__(16) int32_t s_bt[kMaxSplitTokens];
  __shared__ __align__(16) float s_p[kWaves][kTile * G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ __align__(16) float s_acc[kWaves][G * D];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ctx = p.context_lens[b];
  const int t_begin = split * p.split_tokens;
  const int n_h = p.n_h;

  if (t_begin >= ctx) {
    // Only the first split of an empty sequence has anything to write.
    if (split == 0 && p.num_splits == 1) {
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        const int64_t o = ((int64_t)b * n_h + kvh * G + h) * D + d;
        if (p.q_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = 0;
        else reinterpret_cast<float*>(p.out)[o] = 0.f;
      }
    }
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
  float acc[G][Gm::kEpl];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < Gm::kEpl; ++e) acc[h][e] = 0.f;
  }

  const int vj = lane / Gm::kLpr;      // row within a value load
  const int ve = lane % Gm::kLpr;      // 16-byte piece within the row

  uint4 kreg[Gm::kRowQ];
  int tile_start = t_begin + wave * kTile;
  if (tile_start < t_end) {
    const int t = tile_start + lane;
    if (t < t_end) {
      const uint4* src = reinterpret_cast<const uint4*>(row_addr(kbase, t));
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = make_uint4(0, 0, 0, 0);
    }
  }

  for (; tile_start < t_end; tile_start += kWaves * kTile) {
    // ---- issue the value loads of this tile
    uint4 vreg[Gm::kSteps];
#pragma unroll
    for (int k = 0; k < Gm::kSteps; ++k) {
      const int t = tile_start + k * Gm::kTpi + vj;
      if (t < t_end) vreg[k] = reinterpret_cast<const uint4*>(row_addr(vbase, t))[ve];
      else vreg[k] = make_uint4(0, 0, 0, 0);
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
    if (next < t_end) {
      const int t = next + lane;
      if (t < t_end) {
        const uint4* src = reinterpret_cast<const uint4*>(row_addr(kbase, t));
#pragma unroll
        for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = src[i];
      } else {
#pragma unroll
        for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = make_uint4(0, 0, 0, 0);
      }
    }

    // ---- online softmax update (base 2)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tmax = wave_max(s[h]);           // finite: token tile_start is valid
      const float m_new = fmaxf(m_run[h], tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      const float pr = __builtin_amdgcn_exp2f(s[h] - m_new);
      l_run[h] = l_run[h] * alpha + pr;
      m_run[h] = m_new;
#pragma unroll
      for (int e = 0; e < Gm::kEpl; ++e) acc[h][e] *= alpha;
      s[h] = pr;
    }
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

  // ---- merge within the wave: rows sharing a 16-byte piece, and the sums
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = wave_sum(l_run[h]);
#pragma unroll
    for (int e = 0; e < Gm::kEpl; ++e) {
#pragma unroll
      for (int off = Gm::kLpr; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
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
      for (int e = 0; e < Gm::kEpl; ++e) s_acc[wave][h * D + ve * Gm::kEpl + e] = acc[h][e];
  }
  __syncthreads();

  // ---- merge the 4 waves and write
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (s_m[w][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
      L = fmaf(s_l[w][h], f, L);
      O = fmaf(s_acc[w][idx], f, O);
    }
    const int hq = kvh * G + h;
    if (p.num_splits == 1) {
      const float r = O / L;
      const int64_t o = ((int64_t)b * n_h + hq) * D + d;
      if (p.q_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(r);
      else reinterpret_cast<float*>(p.out)[o] = r;
    } else {
      const int64_t pi = ((int64_t)b * n_h + hq) * p.num_splits + split;
      p.part_o[pi * D + d] = O / L;
      if (d == 0) { p.part_ml[2 * pi] = M; p.part_ml[2 * pi + 1] = L; }
    }
  }
}

// Log-sum-exp merge of split partials (FlashDecoding-style, qwbw 8 Q2/Q3
// name the idea): with M the largest split maximum (base-2 scores),
// out = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s.
__global__ void decode_reduce_kernel(const float* __restrict__ part_o,
                                     const float* __restrict__ part_ml,
                                     const int32_t* __restrict__ context_lens, void* out,
                                     int n_h, int d_v, int num_splits, int split_tokens,
                                     int out_bf16) {
  const int bh = blockIdx.x;
  const int b = bh / n_h;
  const int ctx = context_lens[b];
  const int nsp = min(num_splits, (ctx + split_tokens - 1) / split_tokens);
  const int64_t pbase = (int64_t)bh * num_splits;
  float M = -INFINITY;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, part_ml[2 * (pbase + s)]);
  float L = 0.f;
  for (int s = 0; s < nsp; ++s) L += part_ml[2 * (pbase + s) + 1] * __builtin_amdgcn_exp2f(part_ml[2 * (pbase + s)] - M);
  for (int d = threadIdx.x; d < d_v; d += blockDim.x) {
    float O = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const float w = part_ml[2 * (pbase + s) + 1] * __builtin_amdgcn_exp2f(part_ml[2 * (pbase + s)] - M);
      O = fmaf(part_o[(pbase + s) * d_v + d], w, O);
    }
    const float r = nsp > 0 ? O / L : 0.f;
    const int64_t o = (int64_t)bh * d_v + d;
    if (out_bf16) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(r);
    else reinterpret_cast<float*>(out)[o] = r;
  }
}

template <int D, int G, bool BF16>
hipError_t launch_inst(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)p.n_kv, (unsigned)p.B);
  hipLaunchKernelGGL((decode_gqa_kernel<D, G, BF16>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t dispatch_g(const DecodeParams& p, int g, hipStream_t stream) {
  switch (g) {
    case 1: return launch_inst<D, 1, BF16>(p, stream);
    case 2: return launch_inst<D, 2, BF16>(p, stream);
    case 4: return launch_inst<D, 4, BF16>(p, stream);
    case 8: return launch_inst<D, 8, BF16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gqa_supported(KV kv, bool q_bf16, int d_k, int d_v, int g) {
  if (d_k != d_v) return false;
  if (!(g == 1 || g == 2 || g == 4 || g == 8)) return false;
  if (kv == KV::BF16) return q_bf16 && (d_k == 64 || d_k == 128);
  if (kv == KV::F32) return !q_bf16 && (d_k == 32 || d_k == 64);
  return false;
}

hipError_t launch_decode_gqa(const DecodeParams& p, hipStream_t stream) {
  if (p.split_tokens > kMaxSplitTokens || p.split_tokens % kGqaSplitGranule) return hipErrorInvalidValue;
  const int g = p.n_h / p.n_kv;
  hipError_t e = hipErrorInvalidValue;
  if (p.kv == KV::BF16) {
    if (p.d_k == 128) e = dispatch_g<128, true>(p, g, stream);
    else if (p.d_k == 64) e = dispatch_g<64, true>(p, g, stream);
  } else if (p.kv == KV::F32) {
    if (p.d_k == 64) e = dispatch_g<64, false>(p, g, stream);
    else if (p.d_k == 32) e = dispatch_g<32, false>(p, g, stream);
  }
  if (e != hipSuccess || p.num_splits == 1) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)(p.B * p.n_h)), dim3(64), 0, stream,
                     (const float*)p.part_o, (const float*)p.part_ml, p.context_lens, p.out,
                     p.n_h, p.d_v, p.num_splits, p.split_tokens, p.q_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace pkv
