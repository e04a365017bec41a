// Paged decode attention over an INT8 KV cache with the dequantization fused
// into the loads (guijiagi 4.2: value = code * scale, one fp32 scale per
// token and KV head).
//
// Same decomposition as the float kernel (one workgroup of 4 wavefronts per
// (context split, KV head, sequence); lane-per-token scores; online softmax
// in base 2; a wave-private LDS slice for probabilities; 4-wave merge), with
// the scales folded out of the inner loops:
//   score_j = scale * sK_j * (q . code_j)        (codes widened to bf16 exactly:
//                                                every int8 value is a bf16)
//   acc    += (p_j * sV_j) * code_j               (p_j * sV_j formed once per
//                                                token, in the score phase)
// while the softmax denominator sums p_j itself.
#include "internal.h"
#include "device_common.h"
#include "decode_epilogue.h"

namespace pkv {
namespace {

using namespace dev;

// Four int8 codes -> two dwords of bf16 pairs (exact).
__device__ __forceinline__ void codes_to_bf16x2(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const float c0 = (float)(int8_t)(w & 0xffu);
  const float c1 = (float)(int8_t)((w >> 8) & 0xffu);
  const float c2 = (float)(int8_t)((w >> 16) & 0xffu);
  const float c3 = (float)(int8_t)(w >> 24);
  // the low 16 bits of a small integer's binary32 are zero: keep the high halves
  lo = __builtin_amdgcn_perm(__float_as_uint(c1), __float_as_uint(c0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(c3), __float_as_uint(c2), 0x07060302u);
}

template <int D>
struct Geo8 {
  static constexpr int kRowBytes = D;                 // one byte per code
  static constexpr int kRowQ = D / 16;                // 16-byte pieces per K row
  static constexpr int kQdw = D / 2;                  // q dwords (bf16 pairs) per head
  static constexpr int kLpr = D / 8;                  // lanes per V row (8 codes each)
  static constexpr int kTpi = kWave / kLpr;           // rows per value load
  static constexpr int kSteps = kTile / kTpi;
};

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_int8_kernel(const DecodeParams p) {
  using Gm = Geo8<D>;
  __shared__ __align__(16) int32_t s_bt[kBtSlots];
  __shared__ __align__(16) float s_p[kWaves][kTile * G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ __align__(16) float s_acc[kWaves][G * D];

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
  const int lb0 = t_begin >> shift;
  {
    const int nblk = ((t_end - 1) >> shift) - lb0 + 1;
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq + lb0;
    for (int i = tid; i < nblk; i += kThreads) s_bt[i] = row[i];
  }
  __syncthreads();

  const int n_kv = p.n_kv;
  const int8_t* kcodes = reinterpret_cast<const int8_t*>(p.k);
  const int8_t* vcodes = reinterpret_cast<const int8_t*>(p.v);
  const float qscale = p.scale * kLog2e;
  // slot * n_kv + kvh: row index into the codes (x D bytes); the scales are
  // [num_blocks, n_kv, block_size]
  auto row_of = [&](int t) -> int64_t {
    const int32_t phys = s_bt[(t >> shift) - lb0];
    return (((int64_t)phys << shift) + (t & bmask)) * n_kv + kvh;
  };
  auto scale_of = [&](int t) -> int64_t {
    const int32_t phys = s_bt[(t >> shift) - lb0];
    return (((int64_t)phys * n_kv + kvh) << shift) + (t & bmask);
  };
  const int64_t q_dw0 = ((int64_t)b * n_h + (int64_t)kvh * G) * Gm::kQdw;

  float m_run[G], l_run[G];
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const int vj = lane / Gm::kLpr;
  const int ve = lane % Gm::kLpr;

  for (int tile_start = t_begin + wave * kTile; tile_start < t_end; tile_start += kWaves * kTile) {
    // ---- value codes of this tile (8 per lane), issued first
    uint2 vreg[Gm::kSteps];
#pragma unroll
    for (int k = 0; k < Gm::kSteps; ++k) {
      const int t = tile_start + k * Gm::kTpi + vj;
      if (t < t_end) vreg[k] = reinterpret_cast<const uint2*>(vcodes + row_of(t) * D)[ve];
      else vreg[k] = make_uint2(0, 0);
    }
    // ---- this lane's token: K codes, K scale, V scale
    const int my_t = tile_start + lane;
    const bool valid = my_t < t_end;
    uint4 kreg[Gm::kRowQ];
    float ks = 0.f, vs = 0.f;
    if (valid) {
      const int64_t r = row_of(my_t);
      const uint4* src = reinterpret_cast<const uint4*>(kcodes + r * D);
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = src[i];
      const int64_t si = scale_of(my_t);
      ks = p.k_scale[si];
      vs = p.v_scale[si];
    } else {
#pragma unroll
      for (int i = 0; i < Gm::kRowQ; ++i) kreg[i] = make_uint4(0, 0, 0, 0);
    }

    // ---- scores: q (bf16 pairs, scalar loads in chunks, see the float
    // kernel) against the codes widened to bf16 pairs
    float s[G];
    {
      using QPtr = const __attribute__((address_space(4))) uint32_t*;
      constexpr int kQch = 16;
      constexpr int kCph = Gm::kQdw / kQch;
      constexpr int kNch = G * kCph;
      uintptr_t qaddr = (uintptr_t)p.q + (uintptr_t)q_dw0 * 4u;
      asm volatile("" : "+s"(qaddr));
      // widen the codes once: kQdw dwords of bf16 pairs
      uint32_t kw[Gm::kQdw];
#pragma unroll
      for (int i = 0; i < Gm::kRowQ * 4; ++i) codes_to_bf16x2(kdw(kreg, i), kw[2 * i], kw[2 * i + 1]);
      float ax[G], ay[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { ax[h] = 0.f; ay[h] = 0.f; }
      uint32_t qa[kQch], qb[kQch];
      auto load_chunk = [&](uint32_t (&dst)[kQch], int c) {
        const QPtr qp = (QPtr)qaddr;
        const int off = (c / kCph) * Gm::kQdw + (c % kCph) * kQch;
#pragma unroll
        for (int i = 0; i < kQch; ++i) dst[i] = qp[off + i];
      };
      load_chunk(qa, 0);
#pragma unroll
      for (int c = 0; c < kNch; ++c) {
        if (c > 0) {
          const int hp = (c - 1) / kCph;
          asm volatile("" : "+s"(qaddr) : "v"(ax[hp]), "v"(ay[hp]));
        }
        if (c + 1 < kNch) load_chunk(qb, c + 1);
        const int h = c / kCph;
        const int w0 = (c % kCph) * kQch;
#pragma unroll
        for (int i = 0; i < kQch; i += 2) {
          ax[h] = dot2_bf16(qa[i], kw[w0 + i], ax[h]);
          ay[h] = dot2_bf16(qa[i + 1], kw[w0 + i + 1], ay[h]);
        }
#pragma unroll
        for (int i = 0; i < kQch; ++i) qa[i] = qb[i];
      }
      const float f = ks * qscale;
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = valid ? (ax[h] + ay[h]) * f : -INFINITY;
    }

    // ---- online softmax; LDS gets p * sV
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tmax = wave_max(s[h]);
      const float m_new = fmaxf(m_run[h], tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      const float pr = __builtin_amdgcn_exp2f(s[h] - m_new);
      l_run[h] = l_run[h] * alpha + pr;
      m_run[h] = m_new;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      s[h] = pr * vs;
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

    // ---- acc += (p * sV) * code
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
      float v[8];
      const uint32_t w0 = vreg[k].x, w1 = vreg[k].y;
      v[0] = (float)(int8_t)(w0 & 0xffu); v[1] = (float)(int8_t)((w0 >> 8) & 0xffu);
      v[2] = (float)(int8_t)((w0 >> 16) & 0xffu); v[3] = (float)(int8_t)(w0 >> 24);
      v[4] = (float)(int8_t)(w1 & 0xffu); v[5] = (float)(int8_t)((w1 >> 8) & 0xffu);
      v[6] = (float)(int8_t)((w1 >> 16) & 0xffu); v[7] = (float)(int8_t)(w1 >> 24);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr[h], v[e], acc[h][e]);
    }
    wave_sync_lds();
  }

  // ---- merge inside the wave, then across the 4 waves
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = wave_sum(l_run[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
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
      for (int e = 0; e < 8; ++e) s_acc[wave][h * D + ve * 8 + e] = acc[h][e];
  }
  __syncthreads();
  finish_split<G, D>(p, b, kvh, split, ctx, s_m, s_l, s_acc);
}

template <int D, int G>
hipError_t launch8(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.n_kv, (unsigned)p.B, (unsigned)p.num_splits);
  hipLaunchKernelGGL((decode_int8_kernel<D, G>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch8(const DecodeParams& p, int g, hipStream_t stream) {
  switch (g) {
    case 1: return launch8<D, 1>(p, stream);
    case 2: return launch8<D, 2>(p, stream);
    case 4: return launch8<D, 4>(p, stream);
    case 8: return launch8<D, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool int8_supported(bool q_bf16, int d_k, int d_v, int g) {
  return q_bf16 && d_k == d_v && (d_k == 64 || d_k == 128) && (g == 1 || g == 2 || g == 4 || g == 8);
}

hipError_t launch_decode_int8(const DecodeParams& p, int g, hipStream_t stream) {
  if (p.d_k == 128) return dispatch8<128>(p, g, stream);
  if (p.d_k == 64) return dispatch8<64>(p, g, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
