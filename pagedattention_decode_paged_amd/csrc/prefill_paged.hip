// Chunked-prefill attention over the paged cache (faulkner, continuous
// batching section: a long prompt is processed a fixed number of tokens per
// step, each chunk attending causally to everything cached before it plus
// itself).  Sequence b's chunk holds chunk_lens[b] query tokens at positions
// start_pos[b] + i, whose K/V rows are already in the cache; query i sees
// positions 0 .. start_pos[b] + i, through the block table (faulkner's
// logical/physical mapping; qwbw 3.4), the g query heads of a group sharing
// KV head h / g.
//
// How (gfx950, bf16, d = 128): one workgroup of four waves per (KV head,
// tile of query tokens, sequence).  The query columns of a tile, g heads per
// token, fill two 16-column matrix-core blocks per wave (32 / g tokens per
// wave); the workgroup walks the sequence's K/V rows up to its last query's
// position in 64-token stages staged by LDS DMA (two stages in flight), and
// every wave runs S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16
// over each stage, with one online softmax step per stage and column whose
// mask is that column's causal limit.  Rows past 511 blocks of
// the table are taken in chunks (the softmax state carries over).
#include "internal.h"
#include "device_common.h"
#include "lds_dma.h"

namespace pkv {
namespace {

using namespace dev;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;             // one head's bf16 row
constexpr int kStage = 64;                    // tokens per stage
constexpr int kStageBytes = kStage * kRowBytes;
constexpr int kRing = 2;
constexpr int kNW = 4;
constexpr int kDmaPerWave = 2 * (kStage / 4) / kNW;   // 4 rows of 256 B per instruction, K and V
constexpr int kKs = kD / 32;                  // k-steps of the score product
constexpr int kCb = kD / 16;                  // 16-column blocks of the value product
constexpr int kChunkBlocks = kBtSlots - 1;    // table entries staged per chunk of the context

// Piece permutations of the LDS tiles (the decode kernel's one-head layout):
// K row r's logical 16-byte piece p sits at p ^ (r % 16), so 16 lanes
// reading one piece of 16 rows hit 16 bank groups; V rows take p ^ 2(r % 8),
// so the 8 rows of a transposed read phase differ.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 7); }

template <int G>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_paged_kernel(const PrefillParams p) {
  constexpr int kTpw = 32 / G;                // query tokens per wave
  constexpr int kTpc = 16 / G;                // query tokens per column block
  constexpr int kQt = kNW * kTpw;             // query tokens per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t s_dma[2][kRing][kStageBytes];
  __shared__ __align__(16) int32_t s_bt[kBtSlots];

  const int kvh = blockIdx.x, tile = blockIdx.y, b = blockIdx.z;
  // a chunk longer than the q rows, a negative start or one that runs past
  // the table is outside the contract: nothing is read or written for it
  const int n = p.chunk_lens[b], p0 = p.start_pos[b];
  const int i0 = tile * kQt;
  if (i0 >= n || n <= 0 || n > p.max_chunk || p0 < 0 ||
      (int64_t)p0 + n > ((int64_t)p.max_blocks_per_seq << p.block_shift))
    return;
  const int t_end = p0 + min(i0 + kQt, n);   // positions the workgroup reads: [0, t_end)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ml16 = lane & 15, mg = lane >> 4;
  const int shift = p.block_shift, bmask = (1 << shift) - 1;
  const int n_h = p.n_h;

  // the lane's two columns: query token i, head kvh * G + ml16 % G
  int lim[2], qi[2];
  u32x4_t qf[2][kKs];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    qi[cb] = i0 + wave * kTpw + cb * kTpc + ml16 / G;
    const bool valid = qi[cb] < n;
    lim[cb] = valid ? p0 + qi[cb] + 1 : 0;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) +
                          (((int64_t)b * p.max_chunk + min(qi[cb], n - 1)) * n_h + (int64_t)kvh * G + ml16 % G) *
                              kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + (32 * ks + 8 * mg) * 2);
      qf[cb][ks] = valid ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  f32x4_t acc[2][kCb];
  float mm[2] = {-INFINITY, -INFINITY}, ml[2] = {0.f, 0.f};
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int db = 0; db < kCb; ++db) acc[cb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // DMA share: waves 0-1 move K rows, 2-3 V rows, 8 instructions of 4 rows
  const int j0 = wave * kDmaPerWave;
  const bool dma_v = j0 >= kStage / 4;
  const int jbase = j0 % (kStage / 4);
  const int64_t slot_stride = (int64_t)p.n_kv * kRowBytes;
  const uint8_t* mat = reinterpret_cast<const uint8_t*>(dma_v ? p.v : p.k) + (int64_t)kvh * kRowBytes;
  const uint32_t lds_mat =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_dma[dma_v ? 1 : 0][0][0];
  const int lrow = lane / 16, lpiece = lane % 16;
  auto spiece = [&](int r) { return lpiece ^ (dma_v ? swz_v(r) : swz_k(r)); };
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)(lrow * slot_stride) + (uint32_t)spiece((jbase + i) * 4 + lrow) * 16u;
  const bool fast_ok = (1 << shift) >= 4;
  const float qscale = p.scale * kLog2e;

  int cb0 = 0, ce = 0, lb0 = 0;
  auto issue = [&](int s, int slot) {
    const int tile0 = cb0 + s * kStage;
    const uint32_t dst0 = lds_mat + (uint32_t)(slot * kStageBytes);
    if (fast_ok && tile0 + kStage <= ce) {
#pragma unroll
      for (int jj = 0; jj < kDmaPerWave; ++jj) {
        const int jm = jbase + jj;
        const int t0 = tile0 + jm * 4;
        const int32_t phys = __builtin_amdgcn_readfirstlane(s_bt[(t0 >> shift) - lb0]);
        const uint8_t* sb = mat + (((int64_t)phys << shift) + (t0 & bmask)) * slot_stride;
        dma16(sb, voff[jj % 4], dst0 + (uint32_t)(jm * 1024));
      }
    } else {
      int32_t ph[kDmaPerWave];
#pragma unroll
      for (int jj = 0; jj < kDmaPerWave; ++jj) {
        const int r = (jbase + jj) * 4 + lrow;
        ph[jj] = s_bt[(min(tile0 + r, ce - 1) >> shift) - lb0];
      }
#pragma unroll
      for (int jj = 0; jj < kDmaPerWave; ++jj) {
        const int jm = jbase + jj;
        const int r = jm * 4 + lrow;
        const int t = min(tile0 + r, ce - 1);
        const int64_t sl = ((int64_t)ph[jj] << shift) + (t & bmask);
        dma16(mat + sl * slot_stride + spiece(r) * 16, dst0 + (uint32_t)(jm * 1024));
      }
    }
  };
  int n_st = 0;
  auto stage = [&](int s, int slot) {
    wait_vm_imm<0>();                         // this wave's DMA of stage s has landed
    lds_barrier();                            // ... and every wave's; stage s - 1 is free
    if (s + 1 < n_st) issue(s + 1, (slot + 1) % kRing);
    const uint8_t* kst = &s_dma[0][slot][0];
    const uint32_t vbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_dma[1][slot][0];
    const int tile0 = cb0 + s * kStage;
    const int cp = ml16 & 3;
    // The whole stage per step: the scores of its four 16-token blocks, one
    // online softmax step over them, then O^T += V^T P^T on
    // v_mfma_f32_16x16x32_bf16 over pairs of blocks (k = 32 tokens; lane
    // group mg holds tokens 4 mg .. + 3 of each block of the pair, in both
    // operands): half the matrix instructions of 16x16x16 steps, which take
    // as long as one 16x16x32 each on gfx950 (70B-heads chunk leg: 526.7 us
    // with 16x16x16 steps per block, 420 with pairs, 403 with whole stages).
    constexpr int kNB = 4;                            // 16-token blocks per softmax step
#pragma unroll 1
    for (int tp = 0; tp < 4 / kNB; ++tp) {
      const int base = 16 * kNB * tp;
      f32x4_t sacc[kNB][2];
#pragma unroll
      for (int h = 0; h < kNB; ++h)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) sacc[h][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
        for (int h = 0; h < kNB; ++h) {
          const int row = base + 16 * h + ml16;
          const u32x4_t ka =
              *reinterpret_cast<const u32x4_t*>(kst + row * kRowBytes + (((4 * ks + mg) ^ swz_k(row)) * 16));
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            sacc[h][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                                  __builtin_bit_cast(bf16x8_t, qf[cb][ks]), sacc[h][cb], 0, 0, 0);
        }
      }
      bf16x8_t pb[kNB / 2][2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float sc[4 * kNB];
#pragma unroll
        for (int h = 0; h < kNB; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[4 * h + i] = tile0 + base + 16 * h + 4 * mg + i < lim[cb] ? sacc[h][cb][i] * qscale : -INFINITY;
        float smax = sc[0];
#pragma unroll
        for (int e = 1; e < 4 * kNB; ++e) smax = fmaxf(smax, sc[e]);
        {
          const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
          smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
          const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
          smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
        }
        // lazy rescale: the running maximum moves only when a score exceeds
        // it by more than 2^8 (weights stay below 2^8, inside bf16)
        constexpr float kSlack = 8.f;
        if (mm[cb] == -INFINITY) {
          mm[cb] = smax;
        } else if (__builtin_amdgcn_ballot_w64(smax > mm[cb] + kSlack)) {
          const float m_new = fmaxf(mm[cb], smax);
          const float alpha = __builtin_amdgcn_exp2f(mm[cb] - m_new);
          ml[cb] *= alpha;
#pragma unroll
          for (int db = 0; db < kCb; ++db) acc[cb][db] *= alpha;
          mm[cb] = m_new;
        }
        // weights rounded to bf16 (the running sum adds the rounded values);
        // pair q: elements 0-3 block 2 q, 4-7 block 2 q + 1
        float rs = 0.f;
#pragma unroll
        for (int q = 0; q < kNB / 2; ++q) {
          u32x4_t pw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = sc[8 * q + 2 * e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[8 * q + 2 * e] - mm[cb]);
            const float c = sc[8 * q + 2 * e + 1] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[8 * q + 2 * e + 1] - mm[cb]);
            pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, c}), bf16x2_t));
          }
          rs += ((bf_lo(pw[0]) + bf_hi(pw[0])) + (bf_lo(pw[1]) + bf_hi(pw[1]))) +
                ((bf_lo(pw[2]) + bf_hi(pw[2])) + (bf_lo(pw[3]) + bf_hi(pw[3])));
          pb[q][cb] = __builtin_bit_cast(bf16x8_t, pw);
        }
        ml[cb] += rs;
      }
      // V^T fragments: rows 4 mg .. + 3 of each block of pair q, column ml16
      // of the 16-column block, by two transposed reads 16 rows apart
#pragma unroll
      for (int q = 0; q < kNB / 2; ++q) {
        const int tv = base + 32 * q + 4 * mg + (ml16 >> 2);
        const uint32_t vrow = vbase + (uint32_t)(tv * kRowBytes + 8 * (cp & 1));
        const int svz = swz_v(tv);                     // = swz_v(tv + 16)
#pragma unroll
        for (int db = 0; db < kCb; ++db) {
          const uint32_t a = vrow + (uint32_t)((((2 * db + (cp >> 1)) ^ svz)) * 16);
          const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a);
          const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)(a + 16 * kRowBytes));
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[q][cb], acc[cb][db], 0, 0, 0);
        }
      }
    }
  };

  // the context in chunks whose blocks fit the staged table
  const int chunk = (kChunkBlocks << shift) & ~(kStage - 1);
  for (cb0 = 0; cb0 < t_end; cb0 += chunk) {
    ce = min(t_end, cb0 + chunk);
    lb0 = cb0 >> shift;
    if (cb0 > 0) __syncthreads();             // the ring and table of the previous chunk are free
    {
      const int nblk = ((ce - 1) >> shift) - lb0 + 1;
      const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq + lb0;
      for (int i = tid; i < nblk; i += 64 * kNW) s_bt[i] = row[i];
    }
    __syncthreads();
    n_st = (ce - cb0 + kStage - 1) / kStage;
    issue(0, 0);
    for (int s0 = 0; s0 < n_st; s0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u)
        if (s0 + u < n_st) stage(s0 + u, u);
    }
  }
  // outputs: column (token qi, head), 4 rows of each 16-column block per lane
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float L = ml[cb];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (qi[cb] < n) {
      const float inv = 1.0f / L;
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) +
                    (((int64_t)b * p.max_chunk + qi[cb]) * n_h + (int64_t)kvh * G + ml16 % G) * kD;
#pragma unroll
      for (int db = 0; db < kCb; ++db) {
        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                             (f32x2_t{acc[cb][db][0] * inv, acc[cb][db][1] * inv}), bf16x2_t));
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                             (f32x2_t{acc[cb][db][2] * inv, acc[cb][db][3] * inv}), bf16x2_t));
        *reinterpret_cast<u32x2_t*>(o + 16 * db + 4 * mg) = u32x2_t{lo, hi};
      }
    }
  }
}

}  // namespace

bool prefill_supported(int d_k, int d_v, int g) {
  return d_k == kD && d_v == kD && (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

int prefill_tokens_per_workgroup(int g) { return kNW * 32 / g; }

hipError_t launch_prefill_paged(const PrefillParams& p, hipStream_t stream) {
  const int g = p.n_h / p.n_kv;
  if (!prefill_supported(p.d_k, p.d_v, g) || p.B <= 0 || p.max_chunk <= 0) return hipErrorInvalidValue;
  const int qt = prefill_tokens_per_workgroup(g);
  const dim3 grid((unsigned)p.n_kv, (unsigned)((p.max_chunk + qt - 1) / qt), (unsigned)p.B);
  switch (g) {
    case 1: hipLaunchKernelGGL(prefill_paged_kernel<1>, grid, dim3(64 * kNW), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(prefill_paged_kernel<2>, grid, dim3(64 * kNW), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(prefill_paged_kernel<4>, grid, dim3(64 * kNW), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(prefill_paged_kernel<8>, grid, dim3(64 * kNW), 0, stream, p); break;
    default: hipLaunchKernelGGL(prefill_paged_kernel<16>, grid, dim3(64 * kNW), 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
