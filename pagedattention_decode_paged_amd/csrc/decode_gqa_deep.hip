// Deep-pipelined paged decode attention for bf16 pools with 256-byte rows
// (d_h = 128) and blocks of at least 8 slots: the 70B- and 8B-shaped layers.
//
// Same arithmetic as decode_gqa.hip (lane-per-token scores with v_dot2 and
// scalar q loads, base-2 online softmax, value phase on token pairs with
// bf16 probability pairs, 4-wave merge, split partials + decode_reduce), but
// the memory pipeline is built to keep HBM busy:
// * one 4-wave workgroup per compute unit (one wave per SIMD, up to 512
//   VGPRs each);
// * K and V tiles are loaded row-coalesced (16 lanes per 256-byte row, 4 rows
//   per instruction) into registers: K one tile ahead, V two tiles ahead
//   (double-buffered), so while tile j is computed K(j+1), V(j+1) and V(j+2)
//   are in flight (up to 48 KiB per wave);
// * the lane-per-token score phase gets its K row through a per-wave LDS
//   tile: row r's 16-byte piece P is stored in slot P ^ (r % 16), so both the
//   row-wise writes and the token-wise reads touch every bank once per 16
//   lanes;
// * rows past the context re-read the last valid row (finite data that gets
//   a masked score and probability 0), so loads never depend on validity.
#include "internal.h"
#include "device_common.h"
#include "decode_epilogue.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kD = 128;
constexpr int kRowBytes = 256;
constexpr int kRowDw = kRowBytes / 4;
constexpr int kPr = 16;                     // 16-byte pieces per row
constexpr int kRpi = kWave / kPr;           // rows per load instruction (4)
constexpr int kVSteps = kTile / kRpi;       // V loads per tile (16)
constexpr int kKBuf = kTile * kRowBytes;    // one K tile in LDS (16 KiB)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int G>
__global__ __launch_bounds__(kThreads, 1) void decode_gqa_deep_kernel(const DecodeParams p) {
  constexpr int kPairs = kTile / 2;
  constexpr int kGh = (G + 1) / 2;
  __shared__ __align__(16) int32_t s_bt[kBtSlots];
  __shared__ __align__(16) uint32_t s_pp[kWaves][kPairs * G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ __align__(16) uint8_t s_kbuf[kWaves * kKBuf];
  float (&s_acc)[kWaves][G * kD] = *reinterpret_cast<float (*)[kWaves][G * kD]>(s_kbuf);
  static_assert(kWaves * G * kD * 4 <= kWaves * kKBuf, "accumulators fit the K staging area");

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
    if (split == 0) write_zero_rows<G, kD>(p, b, kvh);   // empty sequence
    return;
  }
  const int t_end = min(ctx, t_begin + p.split_tokens);
  const int t_last = t_end - 1;
  const int shift = p.block_shift;
  const int bmask = (1 << shift) - 1;
  const int lb0 = t_begin >> shift;
  {
    const int nblk = ((t_end - 1) >> shift) - lb0 + 1;
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq + lb0;
    for (int i = tid; i < nblk; i += kThreads) s_bt[i] = row[i];
  }
  __syncthreads();

  const int64_t slot_stride = (int64_t)p.n_kv * kRowBytes;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)kvh * kRowBytes;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)kvh * kRowBytes;
  const float qscale = p.scale * kLog2e;
  const int64_t q_dw0 = ((int64_t)b * n_h + (int64_t)kvh * G) * kRowDw;

  // tiles of this wave: j = 0 .. n_w-1 start at t_begin + (wave + 4 j) * 64
  const int first = t_begin + wave * kTile;
  const int n_w = first < t_end ? (t_last - first) / (kWaves * kTile) + 1 : 0;
  auto tile_start = [&](int j) { return first + j * (kWaves * kTile); };

  uint8_t* const kb = s_kbuf + wave * kKBuf;
  const int lj = lane / kPr, le = lane % kPr;       // load role: row lj of 4, piece le
  const int vj = lj, ve = le;                       // value role: same split

  // K rows of tile j, row-coalesced: load k covers rows 4k .. 4k+3
  auto load_k = [&](int j, u32x4_t (&kr)[kPr]) __attribute__((always_inline)) {
    const int ts = tile_start(j);
#pragma unroll
    for (int k = 0; k < kPr; ++k) {
      const int tg = min(ts + k * kRpi, t_last);
      const int32_t phys = __builtin_amdgcn_readfirstlane(s_bt[(tg >> shift) - lb0]);
      const uint8_t* gb = kbase + ((int64_t)phys << shift) * slot_stride;
      const int tr = min(ts + k * kRpi + lj, t_last);
      kr[k] = *reinterpret_cast<const u32x4_t*>(gb + (uint32_t)(tr & bmask) * (uint32_t)slot_stride + (uint32_t)le * 16u);
    }
  };
  // ... and their swizzled home in this wave's LDS tile
  auto store_k = [&](const u32x4_t (&kr)[kPr], uint8_t* kb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kPr; ++k) {
      const int r = k * kRpi + lj;
      *reinterpret_cast<u32x4_t*>(kb + r * kRowBytes + ((le ^ (r & 15)) * 16)) = kr[k];
    }
  };
  // pair-ordered V: load 2m covers tokens 8m + 2 vj, load 2m+1 tokens 8m + 2 vj + 1
  auto load_v = [&](int j, uint4 (&vr)[kVSteps]) __attribute__((always_inline)) {
    const int ts = tile_start(j);
#pragma unroll
    for (int m = 0; m < kVSteps / 2; ++m) {
      const int t_grp = min(ts + 2 * kRpi * m, t_last);
      const int32_t phys = __builtin_amdgcn_readfirstlane(s_bt[(t_grp >> shift) - lb0]);
      const uint8_t* gbase = vbase + ((int64_t)phys << shift) * slot_stride;
      const int t0 = min(ts + 2 * kRpi * m + 2 * vj, t_last);
      const int t1 = min(ts + 2 * kRpi * m + 2 * vj + 1, t_last);
      vr[2 * m] = *reinterpret_cast<const uint4*>(gbase + (uint32_t)(t0 & bmask) * (uint32_t)slot_stride + (uint32_t)ve * 16u);
      vr[2 * m + 1] = *reinterpret_cast<const uint4*>(gbase + (uint32_t)(t1 & bmask) * (uint32_t)slot_stride + (uint32_t)ve * 16u);
    }
  };

  float m_run[G], l_run[G];
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  u32x4_t kload[kPr];        // K rows of the next tile, in flight
  auto process = [&](int j, uint4 (&vr)[kVSteps]) __attribute__((always_inline)) {
    const int ts = tile_start(j);
    const bool has1 = j + 1 < n_w, has2 = j + 2 < n_w;
    // K(j): registers -> swizzled LDS tile -> this lane's token row
    store_k(kload, kb);
    if (has1) load_k(j + 1, kload);
    wave_sync_lds();
    uint4 kreg[kPr];
    {
      int sw = lane & 15;
      asm volatile("" : "+v"(sw));
      const uint8_t* krow = kb + lane * kRowBytes;
#pragma unroll
      for (int i = 0; i < kPr; ++i) kreg[i] = *reinterpret_cast<const uint4*>(krow + ((i ^ sw) * 16));
    }

    // ---- scores (see decode_gqa.hip for the scalar q chunking)
    const bool valid = ts + lane < t_end;
    float s[G];
    {
      using QPtr = const __attribute__((address_space(4))) uint32_t*;
      constexpr int kQch = 16;
      constexpr int kCph = kRowDw / kQch;
      constexpr int kNch = G * kCph;
      float ax[G], ay[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { ax[h] = 0.f; ay[h] = 0.f; }
      uintptr_t qaddr = (uintptr_t)p.q + (uintptr_t)q_dw0 * 4u;
      asm volatile("" : "+s"(qaddr));
      uint32_t qa[kQch], qb[kQch];
      auto load_chunk = [&](uint32_t (&dst)[kQch], int c) {
        const QPtr qp = (QPtr)qaddr;
        const int off = (c / kCph) * kRowDw + (c % kCph) * kQch;
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
          ax[h] = dot2_bf16(qa[i], kdw(kreg, w0 + i), ax[h]);
          ay[h] = dot2_bf16(qa[i + 1], kdw(kreg, w0 + i + 1), ay[h]);
        }
#pragma unroll
        for (int i = 0; i < kQch; ++i) qa[i] = qb[i];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = valid ? (ax[h] + ay[h]) * qscale : -INFINITY;
    }


    // ---- online softmax (base 2), rescale only when a maximum moves
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tmax = wave_max(s[h]);
      if (tmax > m_run[h]) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - tmax);
        l_run[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m_run[h] = tmax;
      }
      const float pr = __builtin_amdgcn_exp2f(s[h] - m_run[h]);
      l_run[h] += pr;
      s[h] = pr;
    }
    // bf16 probability pairs of tokens (2i, 2i+1)
    {
      const bool even = (lane & 1) == 0;
      uint32_t packed[kGh];
#pragma unroll
      for (int jj = 0; jj < kGh; ++jj) {
        const int ho = kGh + jj;
        const float mine_e = s[jj];
        const float mine_o = ho < G ? s[ho < G ? ho : 0] : 0.f;
        const float send = even ? mine_o : mine_e;
        const float recv = dpp<0xB1>(send);
        const float keep = even ? mine_e : mine_o;
        typedef float f2_t __attribute__((ext_vector_type(2)));
        const f2_t v2 = {even ? keep : recv, even ? recv : keep};
        packed[jj] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2_t));
      }
      uint32_t* dst = &s_pp[wave][(lane >> 1) * G + (even ? 0 : kGh)];
      const int nw = even ? kGh : G - kGh;
#pragma unroll
      for (int jj = 0; jj < kGh; ++jj)
        if (jj < nw) dst[jj] = packed[jj];
    }
    wave_sync_lds();

    // ---- acc += p * V over token pairs
#pragma unroll
    for (int m = 0; m < kVSteps / 2; ++m) {
      const int i = m * kRpi + vj;
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
      const uint4 a = vr[2 * m], c = vr[2 * m + 1];
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t lo = __builtin_amdgcn_perm(cw[x], aw[x], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(cw[x], aw[x], 0x07060302u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * x] = dot2_bf16(pp[h], lo, acc[h][2 * x]);
          acc[h][2 * x + 1] = dot2_bf16(pp[h], hi, acc[h][2 * x + 1]);
        }
      }
    }
    wave_sync_lds();
    if (has2) load_v(j + 2, vr);
  };

  uint4 va[kVSteps], vb[kVSteps];
  if (n_w > 0) { load_k(0, kload); load_v(0, va); }
  if (n_w > 1) load_v(1, vb);
  for (int j = 0; j < n_w; j += 2) {
    process(j, va);
    if (j + 1 < n_w) process(j + 1, vb);
  }

  // every wave has left the loop before s_acc (aliasing the K buffers) is written
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = wave_sum(l_run[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int off = kPr; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
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
      for (int e = 0; e < 8; ++e) s_acc[wave][h * kD + ve * 8 + e] = acc[h][e];
  }
  __syncthreads();
  finish_split<G, kD>(p, b, kvh, split, ctx, s_m, s_l, s_acc);
}

template <int G>
hipError_t launch_deep(const DecodeParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)p.n_kv, (unsigned)p.B);
  hipLaunchKernelGGL(decode_gqa_deep_kernel<G>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool deep_supported(const DecodeParams& p) {
  const int g = p.n_h / p.n_kv;
  return p.kv == KV::BF16 && p.q_bf16 && p.d_k == kD && p.d_v == kD && p.block_shift >= 3 &&
         (g == 1 || g == 2 || g == 4 || g == 8);
}

hipError_t launch_decode_deep(const DecodeParams& p, hipStream_t stream) {
  switch (p.n_h / p.n_kv) {
    case 1: return launch_deep<1>(p, stream);
    case 2: return launch_deep<2>(p, stream);
    case 4: return launch_deep<4>(p, stream);
    case 8: return launch_deep<8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
