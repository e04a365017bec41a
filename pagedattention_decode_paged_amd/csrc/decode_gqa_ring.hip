// Paged decode attention for GQA with g = n_h / n_kv in {4, 8}: bf16 pools,
// and INT8 pools with the dequantization fused in.  The kernel for the
// bandwidth-bound shapes (8B- and 70B-shaped layers).
//
// What is computed: for each sequence b and query head h,
//   out[b][h] = sum_j softmax_j(scale * q[b][h] . K_j) V_j ,  j < context_lens[b],
// with K_j, V_j reached through the block table (faulkner, first section and
// the logical/physical block mapping; qwbw 3.4) and the g query heads of a
// group sharing KV head h / g (faulkner's MHA/GQA/MLA table).  For an INT8
// pool K_j = code_j * sK_j and V_j = code_j * sV_j with one fp32 scale per
// (token, KV head) (guijiagi 4.2).
//
// How (gfx950, wave64, one workgroup of NW waves per (split, KV head, seq)):
// * K and V rows reach LDS through the LDS DMA path (global_load_lds_dwordx4)
//   in 64-token stages, RING stages deep: while a stage is computed the next
//   RING - 1 are in flight, so the reads outstanding live in LDS, not in
//   registers.  Each DMA instruction moves whole rows, 16 bytes per lane;
//   for a whole stage the block's base address is formed on the scalar unit
//   and each lane adds a loop-invariant 32-bit offset (rows of an
//   instruction share a block); the last, partial stage (and blocks smaller
//   than an instruction's rows) use per-lane addresses.
// * INT8: codes and the per-token scales land in a staging ring, and each
//   wave takes the codes of its own rows from there (no other wave waits for
//   them).  Scores: the K codes go as they are into the 8-bit matrix-core
//   product against the query held as three int8 parts with one scale per
//   head, q ~ s_q (q1 + q2 / 254 + q3 / 254^2) (error at most
//   s_q / (2 * 254^2) per element, about 6e-8 of the head's largest |q|).
//   Values: the wave widens its V codes to a bf16 tile in LDS as
//   u = code + 128 (exact: every integer in [0, 255] is a bf16), read back
//   transposed, and the offset is taken out exactly afterwards:
//   sum_t p'_t code_t = sum_t p'_t u_t - 128 sum_t p'_t with p'_t = p_t * sV_t.
// * Four waves; each takes 16 tokens of a stage for all g heads (padded to
//   16).  Per KV head the work is a dense [g x d] . [d x tokens]
//   contraction: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16
//   (INT8: v_mfma_i32_16x16x64_i8) / 16x16x16bf16_1k, with lane l holding
//   head l % 16 and tokens 4 (l / 16) .. + 3 in both, so the weights feed
//   the second product from the lane's own registers and a head's rescale
//   factor sits in the lanes that hold its outputs.  Online softmax in
//   base 2 (scale * log2 e folded in), with a lazy rescale.  Each wave keeps
//   its own softmax state; the four are merged through LDS at the end.  A
//   K/V byte crosses HBM once and feeds all g heads.
// * K rows (or code rows) are read one per lane (16 lanes per LDS phase) and
//   V transposed (ds_read_b64_tr_b16, 4 rows of 2 pieces per 16 lanes); the
//   tiles and the code ring are stored with their 16-byte pieces permuted by
//   row so that every read phase hits distinct banks of the 64-bank LDS.
// * Tokens at or past the context length re-read the last valid row (finite
//   data): their scores are -inf and weights 0, so unused slots (NaN in the
//   tests) are never read.
#include <utility>

#include "internal.h"
#include "device_common.h"
#include "lds_dma.h"

// Launch shape (measured on the 70B-shaped layer): four waves, two 32 KiB
// stages (two workgroups resident per compute unit).
constexpr int kWaves = 4;
constexpr int kRing = 2;
// INT4 stages are 4 KiB of codes per matrix: four in the ring (three in
// flight), which also leaves room for the four waves' merge buffers
constexpr int kRingQ4 = 4;
constexpr int kGridSplit = 0, kGridCompact = 1, kGridStream = 2, kGridStreamPrefix = 3;
// bf16 with d = 128: two adjacent KV heads per workgroup
// (512 contiguous bytes per token per DMA row), when n_kv is even
#ifndef PKV_GQA_PAIR
#define PKV_GQA_PAIR 1
#endif
// INT8 with d = 128: up to this many adjacent KV heads per
// workgroup (128-byte code rows moved KH at a time; on the skewed 70B-shaped
// INT8 batch 1, 2, 4 heads: 108.5, 88.5, 90.6 us)
#ifndef PKV_Q8_KH
#define PKV_Q8_KH 2
#endif

namespace pkv {
namespace {

using namespace dev;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// A workgroup serves KH adjacent KV heads (1, or 2 / 4 on the matrix-core
// path): a token's rows of those heads are adjacent in the pool, so the DMA
// moves KH rows of 256 (bf16) or 128 (INT8) contiguous bytes per token.  A
// stage holds 64 / KH tokens.
template <int D, int NW, bool Q8, int KH = 1, bool Q4 = false>
struct Ring {
  static constexpr int kStageTok = 64 / KH;                   // tokens per stage
  static constexpr int kHeadRow = Q4 ? D / 2 : (Q8 ? D : D * 2);   // bytes of one head's row in the pool
  static constexpr int kRowBytes = KH * D * 2;                // bf16 row of the LDS tiles (KH heads)
  static constexpr int kPieces = D * 2 / 16;                  // 16-byte pieces per head row (bf16)
  static constexpr int kSrcRow = KH * kHeadRow;               // bytes per token moved by the DMA
  static constexpr int kSrcPieces = kSrcRow / 16;
  static constexpr int kRowsPerDma = kWave / kSrcPieces;      // rows per DMA instruction
  static constexpr int kDmaPerMat = kStageTok / kRowsPerDma;  // per stage, per matrix
  static constexpr int kDmaPerWave = 2 * kDmaPerMat / NW;     // each wave's row share (K or V)
  static constexpr int kMatBytes = kStageTok * kRowBytes;     // one bf16 tile
  static constexpr int kSrcBytes = kStageTok * kSrcRow;       // one matrix of a staged stage
  static constexpr int kRows256 = kRowBytes >= 256 ? 1 : 256 / kRowBytes;   // bf16 rows per 256 bytes (>= 1)
  // INT8 scales: one 4-byte DMA instruction per matrix per stage, issued by
  // waves 0 and 1
  static constexpr int kScaleWaves = Q8 ? 2 : 0;
  static_assert(D == 64 || D == 128, "row must be 64 or 128 elements");
  static_assert(KH == 1 || (D == 128 && (KH == 2 || (Q8 && KH == 4))),
                "KV-head groups: d = 128, two heads (bf16, INT8) or four (INT8)");
  static_assert(!Q4 || (Q8 && D == 128 && KH == 2), "INT4: d = 128, two KV heads per workgroup");
  static_assert(kDmaPerMat % kDmaPerWave == 0, "a wave issues K or V instructions only");
  // Piece permutations of the bf16 tiles (row r's logical piece p of a head
  // sits at position p ^ swz(r) of that head's pieces; every swz is below
  // the pieces per head row): K rows are read one row per lane, 16 lanes
  // per LDS phase; V is read transposed, 4 rows x 2 pieces per 16 lanes, 32
  // lanes per phase.
  static __device__ __forceinline__ int swz_k(int r) { return (r / kRows256) % kPieces; }
  // V: the two 16-lane groups of a transposed read phase are on rows 4
  // apart, so the 8 rows of a phase need distinct piece pairs (swz >> 1
  // distinct over 8 aligned rows).  INT8 (d = 128): the waves also store
  // their widened rows, one row per lane, and a 16-byte store is served 8
  // lanes (128 bytes) at a time, so swz & 7 must be distinct over 8 aligned
  // rows as well, and all of swz over 16 (r & 7 with bit 3 = bit 0 of
  // r ^ (r >> 3) does all three; 2 (r & 7) | bit 3 of r, distinct over 16
  // rows only, cost the INT8 call 2.7e6 conflict cycles).
  static __device__ __forceinline__ int swz_v(int r) {
    if constexpr (D == 128 && Q8) return (r & 7) | (((r ^ (r >> 3)) & 1) << 3);
    return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
  }
  // INT8 code rows in the staging ring: 16-byte piece p of row r sits at
  // position p ^ swz_c(r).  A wave reads one piece of 16 consecutive rows
  // per phase, which then fall on the 16 distinct 16-byte bank groups.
  static constexpr int kCodeRows256 = kSrcPieces >= 16 ? 1 : 16 / kSrcPieces;   // code rows per 256 bytes
  static constexpr int kCodeSwzMask = (kSrcPieces >= 16 ? 16 : kSrcPieces) - 1;
  static __device__ __forceinline__ int swz_c(int r) { return (r / kCodeRows256) & kCodeSwzMask; }
};

// Sixteen int8 codes (a 16-byte piece) -> sixteen bf16 values code + 128
// (exact), as two 16-byte pieces.
__device__ __forceinline__ void widen_codes(const u32x4_t c, u32x4_t& lo, u32x4_t& hi) {
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t u = c[w] ^ 0x80808080u;        // code + 128 as unsigned bytes
    // (byte -> float conversions: v_cvt_f32_ubyte0..3)
    const f32x2_t a = {(float)(u & 0xffu), (float)((u >> 8) & 0xffu)};
    const f32x2_t b = {(float)((u >> 16) & 0xffu), (float)(u >> 24)};
    o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_t));
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_t));
  }
  lo = u32x4_t{o[0], o[1], o[2], o[3]};
  hi = u32x4_t{o[4], o[5], o[6], o[7]};
}

// Thirty-two int4 codes (a 16-byte piece, element 2i in the low and 2i + 1
// in the high nibble of byte i) -> thirty-two bf16 values 136 + code, as four
// 16-byte pieces in element order.  With n = code + 8 in [0, 15], the bf16
// bits of 128 + n are 0x4300 | n (exponent 7, mantissa n), so each byte
// becomes one bf16 pair by a byte permute and an or.
__device__ __forceinline__ void widen_int4(const u32x4_t c, u32x4_t (&out)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t u = c[w] ^ 0x88888888u;             // every nibble + 8 (mod 16)
    const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)                        // byte k of lo to byte 0, of hi to byte 2
      o[k] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | (uint32_t)k | ((uint32_t)(4 + k) << 16)) | 0x43004300u;
    out[w] = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

// INT8: registers for three waves per SIMD (at most 168, no AGPR copies;
// on the skewed INT8 batch 81.4 against 84.7 us with 136 + 40 AGPRs).  The
// shared-prefix instance: at most 256 registers, so that two workgroups stay
// resident per compute unit (the prefix pass alone would take 357).  INT4:
// its LDS (four stages, ~54 KB) allows two workgroups per compute unit, so
// up to 256 registers (at 168 the compact grid spilled).
// GRID: kGridSplit (KV head group, sequence, split), kGridCompact (KV head
// group, unit: the splits that exist), kGridStream (KV head group, equal
// token ranges) or kGridStreamPrefix (the stream grid after a shared prefix,
// plus the prefix workgroups).
// APP: the INT8 instance that also quantizes and writes the appended rows
// (a separate instance, so that the plain INT8 kernels keep their code).
template <int D, int G, int NW, int RING, bool Q8, int GRID, int KH, bool Q4 = false, bool APP = false>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(Q4 ? 2 : (Q8 ? 3 : (GRID == kGridStreamPrefix ? 2 : 1)))))
void decode_gqa_ring_kernel(const DecodeParams p) {
  using R = Ring<D, NW, Q8, KH, Q4>;
  constexpr bool kStreamLike = GRID == kGridStream || GRID == kGridStreamPrefix;
  static_assert(GRID != kGridStreamPrefix || (!Q8 && KH == 2 && D == 128), "shared prefix: bf16, two KV heads");
  constexpr int kStageTok = R::kStageTok;
  constexpr int kThr = 64 * NW;
  static_assert(NW == 4 && G <= 16, "four waves of 16 tokens per stage, g <= 16");
  // k-steps of the score product (32 dims each) and 16-column blocks of
  // the value product
  constexpr int kKs = D / 32;
  constexpr int kCb = D / 16;
  // bf16: the DMA ring holds the K and V tiles themselves.  INT8: it holds
  // codes and scales, and one pair of bf16 tiles receives each stage.
  constexpr int kRingBytes = Q8 ? R::kSrcBytes : R::kMatBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t s_dma[2][RING][kRingBytes];
  // INT8: the bf16 V tile (each wave widens its own rows into it)
  __shared__ __attribute__((aligned(1024))) uint8_t s_tile[Q8 ? R::kMatBytes : 16];
  __shared__ __align__(16) float s_scl[2][Q8 ? RING : 1][Q8 ? KH * kStageTok : 1];   // [K, V][slot][head][token]
  __shared__ __align__(16) int32_t s_bt[Q8 ? kBtSlotsInt8 : kBtSlots];
  // compact grid: units before each sequence; stream grid: padded tokens
  // before each sequence; then the total
  __shared__ int32_t s_upre[GRID != kGridSplit ? kCompactMaxB + 1 : 1];
  __shared__ int32_t s_t16;                         // stream grid: the piece bound (0: equal ranges)

  // KV head (group of KH heads) fastest in the grid: workgroups are dealt to
  // the 8 XCDs round-robin by linear index, so each XCD serves whole KV
  // heads (identical work) whatever the context lengths and split count
  const int kvh = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

  // Zero output for an empty sequence (this workgroup's heads).
  auto zero_out = [&](const int b) {
    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)b * p.n_h + (int64_t)kvh * KH * G) * D;
    for (int i = threadIdx.x; i < KH * G * D; i += kThr) o[i] = 0;
  };

  // ---- one unit of work: tokens [t_begin, t_end) of sequence b (ctx > 0
  // tokens).  Its per-head result is the output itself when the unit is the
  // whole sequence and direct_ok, else a partial at row pmul * row + padd of
  // the workspace (row = b * n_h + head).  In the compact and stream grids the
  // thread index is an opaque copy, so that the lane-dependent offsets below
  // are formed per unit rather than hoisted out of the loop over units and
  // kept live across it.
  auto unit = [&](const int b, const int t_begin, const int t_end, const int ctx, const int64_t pmul,
                  const int64_t padd, const bool direct_ok) __attribute__((always_inline)) {
  int tid = threadIdx.x;
  if constexpr (GRID != kGridSplit) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int n_h = p.n_h;
  const int lo = window_lo(p, ctx);                  // positions below it are masked (sliding window)
  // INT4: the first n_sink positions come from the sink rows, not the codes
  const int mlo = Q4 ? max(lo, p.n_sink) : lo;
  const int shift = p.block_shift;
  const int bmask = (1 << shift) - 1;
  // The tokens go in chunks [cb, ce) whose blocks fit the staged block table
  // (one chunk unless the unit is longer than that); the softmax state runs
  // on across chunks.
  int cb = t_begin, ce = t_end, lb0 = 0, n_stages = 0;
  const int64_t slot_stride = (int64_t)p.n_kv * R::kHeadRow;   // bytes per token slot

  // tokens per chunk: every chunk spans at most kBtN blocks, and chunk
  // starts stay at multiples of 16 tokens (the DMA's whole-stage path takes
  // rows of one instruction from one block).  On the split and compact grids
  // the launch bounds a split to kBtN blocks, so a split is a single chunk.
  constexpr int kBtN = Q8 ? kBtSlotsInt8 : kBtSlots;
  const int chunk = (int)min((int64_t)(kBtN - 1) << shift, (int64_t)1 << 30) & ~(kStageTok - 1);
  // a chunk's block-table entries into LDS (and, for the chunk that holds
  // the sequence's last token, the appended rows), ready for its DMA
  auto begin_chunk = [&]() {
    ce = !kStreamLike ? t_end : min(t_end, cb + chunk);   // a split is one chunk
    lb0 = cb >> shift;
    {
      const int nblk = ((ce - 1) >> shift) - lb0 + 1;
      const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq + lb0;
      for (int i = tid; i < nblk; i += kThr) s_bt[i] = row[i];
    }
    __syncthreads();
    if constexpr (!Q8) {
      if (p.k_new != nullptr && ce == ctx) {
        // Append: the workgroup holding the sequence's last token writes that
        // token's new K and V rows (its KV heads) into its slot, and the store
        // completes before any of the workgroup's DMA can read the slot.
        // With a ring of two stages every wave waits for all of its memory
        // operations before the barrier that precedes each stage's DMA issue,
        // so only a token in the stage issued ahead of the loop needs a wait
        // here (70B-shaped layer 95.1 -> 94.7 us).
        static_assert(RING == 2, "the stage loop's waits cover the append store");
        const bool wait_now = ce - 1 < cb + (RING - 1) * kStageTok;
        if (wave == 0) {
          const int t_last = ce - 1;
          constexpr int kLanesPerRow = R::kSrcRow / 16;     // 16-byte pieces per row
          const int m = lane / kLanesPerRow, piece = lane % kLanesPerRow;
          const int32_t phys = s_bt[(t_last >> shift) - lb0];
          if (m < 2 && phys >= 0) {                          // an unmapped block is skipped
            const int64_t sl = ((int64_t)phys << shift) + (t_last & bmask);
            const int64_t off = (int64_t)kvh * R::kSrcRow + piece * 16;
            const uint8_t* src = reinterpret_cast<const uint8_t*>(m ? p.v_new : p.k_new) +
                                 ((int64_t)b * p.n_kv) * R::kHeadRow + off;
            uint8_t* dst = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(m ? p.v : p.k)) +
                           sl * slot_stride + off;
            *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
          }
          if (wait_now) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        }
        if (wait_now) __syncthreads();
      }
    } else if constexpr (!Q4 && APP) {
      if (p.k_new != nullptr && ce == ctx) {
        // Append (INT8): the new token's K and V rows of this workgroup's KV
        // heads (bf16), quantized as reshape_and_cache quantizes them
        // (guijiagi 4.2: scale = absmax / 127 by IEEE division, codes
        // rint(x / scale) clamped to [-128, 127]; a zero row has scale 0 and
        // codes 0), so codes and scales are the same bits; eight elements
        // per thread, a row's absolute maximum reduced over its threads.
        // The same ordering as the bf16 rows: the stores complete before any
        // DMA of the workgroup reads the slot.
        static_assert(RING == 2, "the stage loop's waits cover the append stores");
        const bool wait_now = ce - 1 < cb + (RING - 1) * kStageTok;
        constexpr int kLpr = D / 8;                          // threads per row
        constexpr int kAppThr = 2 * KH * kLpr;               // the K and V rows of the group
        static_assert(kAppThr <= kThr && kWave % kLpr == 0, "eight elements per thread, rows inside a wave");
        if (tid < kAppThr) {
          const int t_last = ce - 1;
          const int r = tid / kLpr, sub = tid % kLpr;
          const int m = r / KH, h = kvh * KH + r % KH;       // K or V, KV head
          const int32_t phys = s_bt[(t_last >> shift) - lb0];
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(
              reinterpret_cast<const uint16_t*>(m ? p.v_new : p.k_new) + ((int64_t)b * p.n_kv + h) * D + sub * 8);
          float x[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[2 * k] = bf_lo(w[k]);
            x[2 * k + 1] = bf_hi(w[k]);
          }
          float amax = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
          for (int off = 1; off < kLpr; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
          if (phys >= 0) {                                   // an unmapped block is skipped
            const float qs = amax / 127.0f;
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              int c = 0;
              if (qs > 0.f) c = (int)fminf(fmaxf(rintf(x[k] / qs), -128.f), 127.f);
              if (k < 4) lo |= (uint32_t)(c & 0xFF) << (8 * k);
              else hi |= (uint32_t)(c & 0xFF) << (8 * (k - 4));
            }
            const int64_t sl = ((int64_t)phys << shift) + (t_last & bmask);
            uint8_t* dst = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(m ? p.v : p.k)) +
                           (sl * p.n_kv + h) * D + sub * 8;
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{lo, hi};
            if (sub == 0)
              const_cast<float*>(m ? p.v_scale : p.k_scale)[(((int64_t)phys * p.n_kv + h) << shift) + (t_last & bmask)] = qs;
          }
          if (wait_now) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        }
        if (wait_now) __syncthreads();
      }
    }
  };
  begin_chunk();                                    // the first chunk (cb = t_begin)

  // ---- this wave's DMA share: instructions j0 .. j0 + kDmaPerWave - 1 of a
  // stage, all on K (first half of the waves) or all on V.  Lane l moves
  // piece l % kSrcPieces of row l / kSrcPieces of the instruction's rows.
  const int j0 = wave * R::kDmaPerWave;
  const bool dma_v = j0 >= R::kDmaPerMat;
  const int jbase = j0 % R::kDmaPerMat;
  const uint8_t* mat = reinterpret_cast<const uint8_t*>(dma_v ? p.v : p.k) + (int64_t)kvh * R::kSrcRow;
  const uint32_t lds_mat =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_dma[dma_v ? 1 : 0][0][0];
  const int lrow = lane / R::kSrcPieces, lpiece = lane % R::kSrcPieces;
  // source piece a lane moves for row r: bf16 rows go straight to the tile,
  // INT8 codes to the staging ring, both permuted by row
  auto src_piece = [&](int r) {
    if constexpr (Q8) return lpiece ^ R::swz_c(r);
    else return lpiece ^ (dma_v ? R::swz_v(r) : R::swz_k(r));
  };
  // per-lane offsets inside a block for the fast path, for instructions
  // jbase + i; the permutation depends on the row only through the
  // instruction index mod kSwzPeriod
  constexpr int kSwzPeriod = Q8 ? 16 / R::kRowsPerDma : (KH == 2 ? 8 : (D == 128 ? 4 : 2));
  constexpr int kVoffN = kSwzPeriod < R::kDmaPerWave ? kSwzPeriod : R::kDmaPerWave;
  static_assert(kVoffN == R::kDmaPerWave || R::kDmaPerWave % kSwzPeriod == 0, "offset table period");
  uint32_t voff[kVoffN];
#pragma unroll
  for (int i = 0; i < kVoffN; ++i)
    voff[i] = (uint32_t)(lrow * slot_stride) + (uint32_t)src_piece((jbase + i) * R::kRowsPerDma + lrow) * 16u;
  const bool fast_ok = (1 << shift) >= R::kRowsPerDma;
  // INT8 / INT4 scales of a stage: wave 0 moves the K scales, wave 1 the V
  // scales, one fp32 per lane and token, into [K, V][slot][head][token]
  // (INT4 batch 86.0 us, against 90.2 us with [slot][K, V]).
  // (Scales fetched as 16-byte pieces, four tokens per lane in one DMA of
  // wave 0, ran slower: 85.1 against 81.7 us on the INT8 batch.)
  const int scl_m = wave == 0 ? 0 : 1;                           // K or V
  const uint32_t lds_scl = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_scl[scl_m][0][0];
  const float* scl_src = scl_m == 0 ? p.k_scale : p.v_scale;
  const int scl_h = lane / kStageTok, scl_t = lane % kStageTok;  // lane -> (head of the group, token)
  const int dma_per_wave = R::kDmaPerWave + (wave < R::kScaleWaves ? 1 : 0);

  auto issue = [&](int s, int slot) {
    const int tile0 = cb + s * kStageTok;
    const int t_last = ce - 1;
    const uint32_t dst0 = lds_mat + (uint32_t)(slot * kRingBytes);
    // The block-table entries of a group of DMAs are read from LDS before
    // the group's first DMA: each DMA is an opaque memory operation to the
    // compiler, so a read placed after one would wait for its own LDS round
    // trip (one per DMA before: INT8 batch 85.1 -> 81.7 us).
    // INT8 / INT4 scales (scales [num_blocks, n_kv, block_size]: a block's
    // scales of the group's heads are adjacent, so the stage's scales are
    // whole runs): the lane's token, clamped to the attended positions.
    // INT8: the scales go before the codes (INT8 batch 79.9 against 80.8 us
    // after them; 83.5 with the codes' table entries also read before this
    // DMA).  INT4 keeps the codes first, each DMA reading its own table entry
    // (INT4 batch 86.1 us, against 90.1 us with the INT8 order).
    auto scale_dma = [&]() {
      if (wave < R::kScaleWaves) {
        const int t = max(min(tile0 + scl_t, t_last), lo);
        const int64_t si =
            (((int64_t)s_bt[(t >> shift) - lb0] * p.n_kv + kvh * KH + scl_h) << shift) + (t & bmask);
        dma4(scl_src + si, lds_scl + (uint32_t)(slot * KH * kStageTok * 4));
      }
    };
    if constexpr (Q8 && !Q4) scale_dma();
    if (fast_ok && tile0 + kStageTok <= ce && tile0 >= lo) {
      // whole stage: one block per instruction, address base on the scalar unit
      int32_t ph[R::kDmaPerWave];
      if constexpr (!Q4) {
#pragma unroll
        for (int jj = 0; jj < R::kDmaPerWave; ++jj)
          ph[jj] = s_bt[((tile0 + (jbase + jj) * R::kRowsPerDma) >> shift) - lb0];
      }
#pragma unroll
      for (int jj = 0; jj < R::kDmaPerWave; ++jj) {
        const int jm = jbase + jj;
        const int t0 = tile0 + jm * R::kRowsPerDma;
        const int32_t phys = __builtin_amdgcn_readfirstlane(Q4 ? s_bt[(t0 >> shift) - lb0] : ph[jj]);
        const uint8_t* sb = mat + (((int64_t)phys << shift) + (t0 & bmask)) * slot_stride;
        dma16(sb, voff[jj % kVoffN], dst0 + (uint32_t)(jm * 1024));
      }
    } else {
      // last (partial) stage, the first stage of a window or tiny blocks:
      // per-lane rows, clamped to the attended positions
      int32_t ph[R::kDmaPerWave];
#pragma unroll
      for (int jj = 0; jj < R::kDmaPerWave; ++jj) {
        const int r = (jbase + jj) * R::kRowsPerDma + lrow;
        ph[jj] = s_bt[(max(min(tile0 + r, t_last), lo) >> shift) - lb0];
      }
#pragma unroll
      for (int jj = 0; jj < R::kDmaPerWave; ++jj) {
        const int jm = jbase + jj;
        const int r = jm * R::kRowsPerDma + lrow;
        const int t = max(min(tile0 + r, t_last), lo);
        const int64_t sl = ((int64_t)ph[jj] << shift) + (t & bmask);
        dma16(mat + sl * slot_stride + src_piece(r) * 16, dst0 + (uint32_t)(jm * 1024));
      }
    }
    if constexpr (Q4) scale_dma();
  };

  const float qscale = p.scale * kLog2e;
  // ---- per stage each wave takes 16 tokens (rows
  // 16 wave .. + 15): S^T = K Q^T (A: K rows from LDS, B: Q^T fragments
  // kept in registers, zero for the padding heads g .. 15), then
  // O^T += V^T P^T (A: V^T by transposed LDS reads, B: the lane's own
  // weights).  In both products lane l holds head l % 16 and tokens
  // 4 (l / 16) .. + 3 of the wave's block, so the weights need no shuffle
  // and a head's rescale factor is in the lanes that hold its outputs.  Each
  // wave keeps its own softmax state; the four are merged at the end.
  const int ml16 = lane & 15, mg = lane >> 4;
  u32x4_t qf[kKs];
  // INT8: the query of the lane's head as three int8 parts with one scale
  // per head, q ~ s_q (q1 + q2 / 254 + q3 / 254^2) with s_q = max |q| / 127:
  // each part is the rounded remainder of the one before times 254, so
  // every part is within [-127, 127] and |q - s_q (...)| <= s_q / (2 254^2),
  // about 6e-8 of max |q| (the rounding of fp32 itself).  The scores then
  // run on the 8-bit matrix cores straight from the codes, each part's
  // q_i . code in exact int32.
  constexpr int kLp = D / 64;                      // 16-byte code pieces per lane and row
  constexpr float kQb = 254.f;
  i32x4_t q1f[kLp], q2f[kLp], q3f[kLp];
  float qk = 0.f;                                  // s_q * scale * log2(e)
  f32x4_t macc[kCb];
  float mm_run = -INFINITY, ml_run = 0.f, mps_run = 0.f;
  {
#pragma unroll
    for (int c = 0; c < kCb; ++c) macc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int kv_w = kvh * KH + wave / (NW / KH);             // this wave's KV head
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) +
                          ((int64_t)b * n_h + (int64_t)kv_w * G + min(ml16, G - 1)) * D * 2;
    // k-step ks of lane group mg covers elements 32 ks + 8 mg .. + 7 (bf16:
    // the K tile's order), or (D / 4) mg + 8 ks .. + 7 (INT8: each lane
    // group takes one contiguous quarter of a code row)
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const int e0 = Q8 ? (D / 4) * mg + 8 * ks : 32 * ks + 8 * mg;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + e0 * 2);
      qf[ks] = ml16 < G ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (Q8) {
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(qf[ks][j])), fabsf(bf_hi(qf[ks][j]))));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float inv = amax > 0.f ? 127.f / amax : 0.f;
      qk = amax * (1.f / 127.f) * qscale;
      // INT8: byte m of piece j pairs with code 16 j + m of the lane's
      // quarter row: element (D / 4) mg + 16 j + m, i.e. k-step 2 j + m / 8.
      // INT4: the quarter's 16 packed bytes unpack to the even elements
      // (piece 0) and the odd ones (piece 1): byte m of piece j pairs with
      // element (D / 4) mg + 2 m + j, the low (j = 0) or high half of
      // dword m % 4 of k-step m / 4.
#pragma unroll
      for (int j = 0; j < kLp; ++j) {
        uint32_t w1[4], w2[4], w3[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t bits = qf[2 * j + d / 2][2 * (d % 2)], bits2 = qf[2 * j + d / 2][2 * (d % 2) + 1];
          float x[4] = {bf_lo(bits) * inv, bf_hi(bits) * inv, bf_lo(bits2) * inv, bf_hi(bits2) * inv};
          if constexpr (Q4) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const uint32_t w = qf[d][m];              // byte 4 d + m: dword m of k-step d
              x[m] = (j == 0 ? bf_lo(w) : bf_hi(w)) * inv;
            }
          }
          uint32_t a = 0u, c = 0u, e = 0u;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float p1 = rintf(x[m]);                          // |x| <= 127
            const float x2 = (x[m] - p1) * kQb;                    // |x2| <= 127
            const float p2 = rintf(x2);
            const float p3 = rintf((x2 - p2) * kQb);               // |.| <= 127
            a |= ((uint32_t)(int)p1 & 0xffu) << (8 * m);
            c |= ((uint32_t)(int)p2 & 0xffu) << (8 * m);
            e |= ((uint32_t)(int)p3 & 0xffu) << (8 * m);
          }
          w1[d] = a;
          w2[d] = c;
          w3[d] = e;
        }
        q1f[j] = i32x4_t{(int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
        q2f[j] = i32x4_t{(int)w2[0], (int)w2[1], (int)w2[2], (int)w2[3]};
        q3f[j] = i32x4_t{(int)w3[0], (int)w3[1], (int)w3[2], (int)w3[3]};
      }
    }
  }
  // INT4 attention sink (guijiagi 4.3): positions [t_begin, min(n_sink,
  // t_end)) come from the unquantized sink rows (bf16 [B, n_sink, n_kv, D]),
  // taken by the first wave of each KV head before the stages: the score of
  // the lane's head on the VALU, folded into its softmax state, and the row's
  // values added to the accumulators in the matrix-core layout (lane (mg,
  // ml16) holds columns 16 c + 4 mg .. + 3 of head ml16).  The stages mask
  // these positions.
  if constexpr (Q4) {
    constexpr int kWphS = NW / KH;
    const int se = min(p.n_sink, t_end);
    if (t_begin < se && wave % kWphS == 0) {
      const int kv_w = kvh * KH + wave / kWphS;
      const uint8_t* qr = reinterpret_cast<const uint8_t*>(p.q) +
                          ((int64_t)b * n_h + (int64_t)kv_w * G + min(ml16, G - 1)) * D * 2;
      for (int j = t_begin; j < se; ++j) {
        const int64_t srow = (((int64_t)b * p.n_sink + j) * p.n_kv + kv_w) * D * 2;
        const uint8_t* kr = reinterpret_cast<const uint8_t*>(p.sink_k) + srow;
        const uint8_t* vr = reinterpret_cast<const uint8_t*>(p.sink_v) + srow;
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(qr + 16 * c);
          const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kr + 16 * c);
#pragma unroll
          for (int w = 0; w < 4; ++w) dot = dot2_bf16(qv[w], kv[w], dot);
        }
        const float sc = dot * qscale;
        const float m_new = fmaxf(mm_run, sc);
        const float alpha = mm_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm_run - m_new);
        const float wgt = __builtin_amdgcn_exp2f(sc - m_new);
        ml_run = ml_run * alpha + (mg == 0 ? wgt : 0.f);     // the four lane groups are summed at the end
        mps_run *= alpha;
#pragma unroll
        for (int c = 0; c < kCb; ++c) {
          const u32x2_t v2 = *reinterpret_cast<const u32x2_t*>(vr + (16 * c + 4 * mg) * 2);
          const f32x4_t vv = {bf_lo(v2[0]), bf_hi(v2[0]), bf_lo(v2[1]), bf_hi(v2[1])};
          macc[c] = macc[c] * alpha + vv * wgt;
        }
        mm_run = m_new;
      }
    }
  }

  auto stage = [&](int s, int slot) {
    // this wave's DMA for stage s has landed (later stages may still fly),
    // then every wave's has, and every wave is done with stage s - 1
    wait_vm(min(RING - 2, n_stages - 1 - s) * dma_per_wave);
    lds_barrier();
    if (s + RING - 1 < n_stages) issue(s + RING - 1, (slot + RING - 1) % RING);

    // bf16: the K and V tiles are the ring slot itself.  INT8: the slot
    // holds codes; each wave widens those of its own rows (below), so no
    // other wave waits for them.
    const uint8_t* kst = &s_dma[0][slot][0];
    const uint8_t* vst = Q8 ? &s_tile[0] : &s_dma[1][slot][0];
    const int tile0 = cb + s * kStageTok;
    {
      // wave -> (KV head of the group, 16-token block of the stage)
      constexpr int kWphS = NW / KH;
      const int khw = wave / kWphS;
      const int tb = 16 * (wave % kWphS);
      const int hoff = khw * (D * 2);
      const int row = tb + ml16;                     // K row of this lane (A operand)
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (Q4) {
        // The lane's codes: the 16 packed bytes of elements (D / 4) mg ..
        // + D / 4 - 1 of row `row` of its KV head, for K and V.
        constexpr int kHeadPieces = D / 32;                 // 16-byte code pieces per head row
        const int cz = R::swz_c(row);
        const int pc = (khw * kHeadPieces + mg) ^ cz;
        const u32x4_t kc = *reinterpret_cast<const u32x4_t*>(&s_dma[0][slot][row * R::kSrcRow + pc * 16]);
        const u32x4_t vc = *reinterpret_cast<const u32x4_t*>(&s_dma[1][slot][row * R::kSrcRow + pc * 16]);
        // V codes -> this wave's rows of the bf16 V tile as 136 + code
        uint8_t* vrow_w = &s_tile[row * R::kRowBytes + hoff];
        const int sv = R::swz_v(row);
        u32x4_t wv[4];
        widen_int4(vc, wv);
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4_t*>(vrow_w + ((4 * mg + k) ^ sv) * 16) = wv[k];
        // K codes as 16 x code in int8 (the low nibbles shifted up: the even
        // elements; the high nibbles in place: the odd ones)
        i32x4_t ke, ko;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ke[w] = (int)((kc[w] << 4) & 0xF0F0F0F0u);
          ko[w] = (int)(kc[w] & 0xF0F0F0F0u);
        }
        i32x4_t a1 = {0, 0, 0, 0}, a2 = {0, 0, 0, 0}, a3 = {0, 0, 0, 0};
        a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ke, q1f[0], a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ke, q2f[0], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ke, q3f[0], a3, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ko, q1f[1], a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ko, q2f[1], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ko, q3f[1], a3, 0, 0, 0);
        // |a_i| <= 128 * 127 * 128 < 2^24: exact in fp32; the 16 comes off exactly
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[i] = (1.f / 16.f) * fmaf((float)a3[i], 1.f / (kQb * kQb), fmaf((float)a2[i], 1.f / kQb, (float)a1[i]));
        asm volatile("" ::: "memory");               // the V tile stores stay before its reads
      } else if constexpr (Q8) {
        // The lane's codes: elements (D / 4) mg .. + D / 4 - 1 of row `row`
        // of its KV head, for K and V (kLp 16-byte pieces each; the k index
        // of the score product is permuted the same way in qf).
        constexpr int kLp = D / 64;
        constexpr int kHeadPieces = D / 16;                 // 16-byte code pieces per head row
        const int cz = R::swz_c(row);
        const uint8_t* ck = &s_dma[0][slot][row * R::kSrcRow];
        const uint8_t* cv = &s_dma[1][slot][row * R::kSrcRow];
        u32x4_t kc[kLp], vc[kLp];
#pragma unroll
        for (int j = 0; j < kLp; ++j) {
          const int pc = (khw * kHeadPieces + kLp * mg + j) ^ cz;
          kc[j] = *reinterpret_cast<const u32x4_t*>(ck + pc * 16);
          vc[j] = *reinterpret_cast<const u32x4_t*>(cv + pc * 16);
        }
        // V codes -> this wave's rows of the bf16 V tile (read back below,
        // transposed, by this wave only: LDS keeps a wave's accesses in order)
        uint8_t* vrow_w = &s_tile[row * R::kRowBytes + hoff];
        const int sv = R::swz_v(row);
#pragma unroll
        for (int j = 0; j < kLp; ++j) {
          u32x4_t lo, hi;
          widen_codes(vc[j], lo, hi);
          const int pb = 2 * (kLp * mg + j);
          *reinterpret_cast<u32x4_t*>(vrow_w + (pb ^ sv) * 16) = lo;
          *reinterpret_cast<u32x4_t*>(vrow_w + ((pb + 1) ^ sv) * 16) = hi;
        }
        // K codes straight into the 8-bit products (no widening)
        i32x4_t a1 = {0, 0, 0, 0}, a2 = {0, 0, 0, 0}, a3 = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kLp; ++j) {
          const i32x4_t kci = __builtin_bit_cast(i32x4_t, kc[j]);
          a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kci, q1f[j], a1, 0, 0, 0);
          a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kci, q2f[j], a2, 0, 0, 0);
          a3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kci, q3f[j], a3, 0, 0, 0);
        }
        // each |a_i| <= 128 * 127 * 127 < 2^24: exact in fp32
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[i] = fmaf((float)a3[i], 1.f / (kQb * kQb), fmaf((float)a2[i], 1.f / kQb, (float)a1[i]));
        asm volatile("" ::: "memory");               // the V tile stores stay before its reads
      } else {
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(
              kst + row * R::kRowBytes + hoff + (((4 * ks + mg) ^ R::swz_k(row)) * 16));
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                         __builtin_bit_cast(bf16x8_t, qf[ks]), sacc, 0, 0, 0);
        }
      }
      const int tl0 = tb + 4 * mg;                   // this lane's first token in the stage
      float sk[4] = {1.f, 1.f, 1.f, 1.f}, svv[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (Q8) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&s_scl[0][slot][khw * kStageTok + tl0]);
        const f32x4_t c = *reinterpret_cast<const f32x4_t*>(&s_scl[1][slot][khw * kStageTok + tl0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { sk[i] = a[i]; svv[i] = c[i]; }
      }
      float sc4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float raw = Q8 ? sacc[i] * (sk[i] * qk) : sacc[i] * qscale;
        sc4[i] = tile0 + tl0 + i < ce && tile0 + tl0 + i >= mlo ? raw : -INFINITY;
      }
      // maximum of the head over the wave's 16 tokens (lanes l16 + 16 j)
      float smax = fmaxf(fmaxf(sc4[0], sc4[1]), fmaxf(sc4[2], sc4[3]));
      {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
        smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
        smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      }
      // lazy rescale: the running maximum moves only when a score exceeds it
      // by more than 2^8 (weights stay below 2^8, well inside bf16)
      constexpr float kSlack = 8.f;
      if (mm_run == -INFINITY) {
        mm_run = smax;                               // still -inf if no token was valid yet
      } else if (__builtin_amdgcn_ballot_w64(smax > mm_run + kSlack)) {
        const float m_new = fmaxf(mm_run, smax);
        const float alpha = __builtin_amdgcn_exp2f(mm_run - m_new);
        ml_run *= alpha;
        mps_run *= alpha;
#pragma unroll
        for (int c = 0; c < kCb; ++c) macc[c] *= alpha;
        mm_run = m_new;
      }
      float pw[4], pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = sc4[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc4[i] - mm_run);
        pw[i] = Q8 ? (Q4 && pr[i] == 0.f ? 0.f : pr[i] * svv[i]) : pr[i];
      }
      const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{pw[0], pw[1]}), bf16x2_t));
      const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{pw[2], pw[3]}), bf16x2_t));
      const float rsum = bf_lo(p01) + bf_hi(p01) + bf_lo(p23) + bf_hi(p23);
      if constexpr (Q8) {
        ml_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        mps_run += rsum;
      } else {
        ml_run += rsum;
      }
      const i16x4_t pb = __builtin_bit_cast(i16x4_t, (u32x2_t{p01, p23}));
      // V^T fragments: lane (mg, ml16) addresses row tl0 + ml16 / 4 and 8
      // bytes of the block's columns; the transposed read hands lane ml16
      // column ml16 of rows tl0 .. tl0 + 3
      const int tv = tl0 + (ml16 >> 2), cp = ml16 & 3;
      const uint32_t vrow = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)vst +
                            (uint32_t)(tv * R::kRowBytes + hoff + 8 * (cp & 1));
      const int svz = R::swz_v(tv);
#pragma unroll
      for (int c = 0; c < kCb; ++c) {
        const uint32_t a = vrow + (uint32_t)((((2 * c + (cp >> 1)) ^ svz)) * 16);
        const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a);
        macc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, macc[c], 0, 0, 0);
      }
    }
  };

  // the chunk [cb, ce): prologue DMA, then its stages
  auto run_chunk = [&]() {
    n_stages = (ce - cb + kStageTok - 1) / kStageTok;
#pragma unroll
    for (int s = 0; s < RING - 1; ++s)
      if (s < n_stages) issue(s, s);
    for (int s0 = 0; s0 < n_stages; s0 += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u)
        if (s0 + u < n_stages) stage(s0 + u, u);
    }
  };
  if constexpr (!kStreamLike) {
    run_chunk();
  } else {
    for (cb = t_begin; cb < t_end; cb += chunk) {
      if (cb != t_begin) begin_chunk();
      run_chunk();
      if (cb + chunk < t_end) __syncthreads();      // ring and block table free for the next chunk
    }
  }
  {
    // ---- finish: per wave and head, the sums over the
    // four lane groups; then the four waves' states are merged through LDS
    // (the ring is free once every wave is past the last stage)
    float L = ml_run;
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    float PS = mps_run;
    if constexpr (Q8) {
      PS += __shfl_xor(PS, 16);
      PS += __shfl_xor(PS, 32);
    }
    __syncthreads();
    // the merge buffers in the ring: the waves' outputs [NW][G][D], then per
    // wave and head the running maximum, sum (and the INT8 weight sum).  At
    // g = 16 the INT8 ring (codes only) holds just the outputs, and the
    // statistics go to the bf16 V tile, free as well by now.
    constexpr bool kStatsInRing = sizeof(s_dma) >= (NW * G * D + 3 * NW * G) * sizeof(float);
    static_assert(sizeof(s_dma) >= NW * G * D * sizeof(float) &&
                      (kStatsInRing || sizeof(s_tile) >= 3 * NW * G * sizeof(float)),
                  "the merge buffers fit the ring (and the V tile)");
    float* s_mo = reinterpret_cast<float*>(&s_dma[0][0][0]);
    float* s_mml = kStatsInRing ? s_mo + NW * G * D : reinterpret_cast<float*>(&s_tile[0]);
    // row (wave, head) of s_mo holds its 16-byte pieces XOR-permuted by the
    // head: the 16 lanes of one store (one piece, heads 0 .. 15) then fall on
    // distinct banks, where the plain layout puts them 512 bytes apart, all
    // on the same ones (70B-shaped layer 95.3 -> 94.8 us, g = 16 100.0 ->
    // 98.4).  INT4 keeps the plain layout: there the permuted one ran 89.4
    // against 87.0 us, with the same occupancy.
    constexpr int kMoSwz = Q4 ? 0 : 15;
    if (ml16 < G) {
#pragma unroll
      for (int c = 0; c < kCb; ++c)
        *reinterpret_cast<f32x4_t*>(&s_mo[(wave * G + ml16) * D + 4 * ((4 * c + mg) ^ (ml16 & kMoSwz))]) = macc[c];
      if (mg == 0) {
        s_mml[wave * G + ml16] = mm_run;
        s_mml[NW * G + wave * G + ml16] = L;
        s_mml[2 * NW * G + wave * G + ml16] = PS;
      }
    }
    __syncthreads();
    // thread -> head h of KV head kh of the group, columns d0 .. d0 + kCpt - 1:
    // the merge factors once per thread, the waves' outputs as vector reads;
    // waves kh * kWph .. + kWph - 1 hold that KV head
    constexpr int kWph = NW / KH;
    constexpr int kCpt = KH * G * D / kThr;
    static_assert(KH * G * D % kThr == 0 && kCpt >= 1 && kCpt <= 16 && (kCpt & (kCpt - 1)) == 0, "merge split");
    const int hh = tid / (D / kCpt), d0 = (tid % (D / kCpt)) * kCpt;
    const int kh = hh / G, h = hh % G;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kWph; ++j) M = fmaxf(M, s_mml[(kh * kWph + j) * G + h]);
    float num[kCpt], den = 0.f;
#pragma unroll
    for (int c = 0; c < kCpt; ++c) num[c] = 0.f;
#pragma unroll
    for (int j = 0; j < kWph; ++j) {
      const int w = kh * kWph + j;
      const float mw = s_mml[w * G + h];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      den = fmaf(f, s_mml[NW * G + w * G + h], den);
      const float off = Q8 ? (Q4 ? 136.f : 128.f) * s_mml[2 * NW * G + w * G + h] : 0.f;
      const float* ow = &s_mo[(w * G + h) * D];
      if constexpr (kCpt >= 4) {
#pragma unroll
        for (int c4 = 0; c4 < kCpt / 4; ++c4) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&ow[4 * (((d0 >> 2) + c4) ^ (h & kMoSwz))]);
#pragma unroll
          for (int i = 0; i < 4; ++i) num[4 * c4 + i] = fmaf(f, x[i] - off, num[4 * c4 + i]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kCpt; ++c) {
          const int dc = d0 + c;
          num[c] = fmaf(f, ow[4 * ((dc >> 2) ^ (h & kMoSwz)) + (dc & 3)] - off, num[c]);
        }
      }
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const int64_t row = (int64_t)b * n_h + (int64_t)(kvh * KH + kh) * G + h;
    if (direct_ok && t_begin <= lo && t_end == ctx) {
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + row * D + d0;
#pragma unroll
      for (int c = 0; c < kCpt; ++c) o[c] = f32_to_bf16_rne(num[c] * inv);
    } else {
      const int64_t pi = row * pmul + padd;
#pragma unroll
      for (int c = 0; c < kCpt; ++c) p.part_o[pi * D + d0 + c] = num[c] * inv;
      if (d0 == 0) { p.part_ml[2 * pi] = M; p.part_ml[2 * pi + 1] = den; }
    }
  }
  };

  // ---- stream grid: workgroup j of nwg.  The tokens [S, ctx) of every
  // sequence (S = 0, or the shared prefix's length), each sequence's part
  // padded to a multiple of 16, are laid end to end and cut into nwg equal
  // ranges of T tokens (a multiple of 16); workgroup j takes range j, i.e.
  // its share of every sequence the range overlaps.  Each share is a unit
  // whose partial goes to piece j + b (distinct for every (j, b) that has a
  // share: the ranges and the sequences are both in order), and the
  // workgroup holding a sequence's first share records its first and last
  // workgroup for the merge.  Wave 0 forms the padded prefix (8 sequences
  // per lane).  With S > 0 no share is a whole sequence (the prefix pieces
  // are merged too), and a sequence with no tokens past S records none.
  auto stream_part = [&](const int j, const int nwg, const int S) {
    if constexpr (kStreamLike) {
    // After a shared prefix (S > 0) each sequence's part [s0, ctx), padded
    // to a multiple of 16, is cut into n_b equal pieces, one workgroup each,
    // so that a workgroup runs one unit: equal ranges of the concatenated
    // parts, which are short there, left the workgroups at sequence
    // boundaries two to four units, and those set the call's length (8B-
    // shaped call 37.9 -> 34.8 us).  The piece bound T (a multiple of 16
    // tokens) is the smallest found by three bisection steps with
    // sum_b ceil(len_b / T) <= nwg, between ceil(total / nwg) and
    // ceil(total / (nwg - nne)) (nne sequences with a part: there the sum is
    // at most total / T + nne <= nwg).  Without a prefix, or with at least as
    // many sequences as workgroups, the parts are cut into equal ranges of
    // the concatenation (without the prefix hint the same call ran 43.4 us
    // with equal ranges, 45.2 with pieces).  Wave 0 forms the counts, 8
    // sequences per lane, and their prefix in s_upre (pieces, or padded
    // tokens for equal ranges).
    if (wave == 0) {
      const int lane = threadIdx.x & 63;
      int len[8];                                   // part lengths in units of 16 tokens
      int sum = 0, nne = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sb = 8 * lane + k;
        const int c = sb < p.B ? p.context_lens[sb] : 0;
        len[k] = (max(c - (S > 0 ? prefix_end(c, S, p.block_shift) : window_a0(p, c)), 0) + 15) >> 4;
        sum += len[k];
        nne += len[k] > 0 ? 1 : 0;
      }
      auto wave_sum = [&](int v) {
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
        return __builtin_amdgcn_readfirstlane(v);
      };
      const int total16 = wave_sum(sum), nne_all = wave_sum(nne);
      int t16 = 0;
      if (S > 0 && nwg > nne_all && total16 > 0) {
        int lo16 = (total16 + nwg - 1) / nwg;
        int hi16 = (total16 + (nwg - nne_all) - 1) / (nwg - nne_all);   // fits
        for (int it = 0; it < 3 && lo16 < hi16; ++it) {
          const int mid = (lo16 + hi16) >> 1;
          int cnt = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) cnt += (len[k] + mid - 1) / mid;
          if (wave_sum(cnt) <= nwg) hi16 = mid; else lo16 = mid + 1;
        }
        t16 = hi16;
      }
      int cnt[8], csum = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        cnt[k] = t16 > 0 ? (len[k] + t16 - 1) / t16 : 16 * len[k];
        csum += cnt[k];
      }
      int incl = csum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      int run = incl - csum;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        s_upre[8 * lane + k] = run;
        run += cnt[k];
      }
      if (lane == kWave - 1) s_upre[kCompactMaxB] = incl;
      if (lane == 0) s_t16 = t16;
    }
    __syncthreads();
    const int t16 = __builtin_amdgcn_readfirstlane(s_t16);
    const int total = __builtin_amdgcn_readfirstlane(s_upre[p.B]);   // pieces, or padded tokens
    // empty sequences: zeroed by workgroup b mod nwg (one piece, done); with
    // a prefix, sequences with no tokens past it record no stream pieces
    for (int b = j; b < p.B; b += nwg) {
      const int cx = p.context_lens[b];
      if (cx <= 0) {
        zero_out(b);
        if (kvh == 0 && threadIdx.x == 0) { p.seq_meta[2 * b] = 0; p.seq_meta[2 * b + 1] = S > 0 ? -1 : 0; }
      } else if (S > 0 && prefix_end(cx, S, p.block_shift) == cx) {
        if (kvh == 0 && threadIdx.x == 0) { p.seq_meta[2 * b] = 0; p.seq_meta[2 * b + 1] = -1; }
      }
    }
    if (t16 > 0) {
      // piece j: the sequence b with s_upre[b] <= j < s_upre[b + 1] (the
      // largest b with s_upre[b] <= j; sequences without pieces repeat the
      // value before them), its piece k = j - s_upre[b] of n_b
      if (j < total) {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_upre[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int b = __builtin_amdgcn_readfirstlane(lo);
        const int first = __builtin_amdgcn_readfirstlane(s_upre[b]);
        const int nb = __builtin_amdgcn_readfirstlane(s_upre[b + 1]) - first;
        const int k = j - first;
        const int ctx = p.context_lens[b];
        const int s0 = S > 0 ? prefix_end(ctx, S, p.block_shift) : window_a0(p, ctx);
        const int L = ctx - s0;
        const int pc16 = ((L + 15) / 16 + nb - 1) / nb;      // piece length, units of 16 tokens
        const int a = 16 * k * pc16, e = min(16 * (k + 1) * pc16, L);
        if (k == 0 && kvh == 0 && threadIdx.x == 0) {
          p.seq_meta[2 * b] = j;
          p.seq_meta[2 * b + 1] = j + nb - 1;
        }
        unit(b, s0 + a, s0 + e, ctx, 1, (int64_t)j * p.n_h, S == 0);
      }
    } else {
      const int T = max(16, ((total + nwg - 1) / nwg + 15) & ~15);
      const int64_t r0 = (int64_t)j * T, r1 = r0 + T;
      // the first sequence that can overlap the range: the largest b with
      // s_upre[b] <= r0
      int lo = 0, hi = p.B;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_upre[mid] <= r0) lo = mid; else hi = mid - 1;
      }
      for (int b = __builtin_amdgcn_readfirstlane(lo); b < p.B; ++b) {
        const int st = __builtin_amdgcn_readfirstlane(s_upre[b]);
        if (st >= r1) break;
        const int ctx = p.context_lens[b];
        const int s0 = S > 0 ? prefix_end(ctx, S, p.block_shift) : window_a0(p, ctx);   // its part starts here
        const int L = ctx - s0;                       // this sequence's tokens in the stream part
        const int a = (int)max(r0 - st, (int64_t)0), e = (int)min(r1 - st, (int64_t)L);
        if (L <= 0 || a >= e) continue;
        if (a == 0 && kvh == 0 && threadIdx.x == 0) {
          p.seq_meta[2 * b] = j;
          p.seq_meta[2 * b + 1] = (st + L - 1) / T;
        }
        unit(b, s0 + a, s0 + e, ctx, 1, (int64_t)j * p.n_h, S == 0);
        __syncthreads();                              // the unit's LDS is free again
      }
    }
    }
  };

  // ---- shared prefix: workgroup y of the prefix ones takes KV head
  // kvh * KH + (y & 1), chunk c = [c * CH, min((c + 1) * CH, S)) of the
  // prefix and sequence group cg (y >> 1 = c * groups + cg).  The chunk's
  // rows come from the longest sequence (the reference); a sequence of the
  // group whose block-table entries over the tokens it has in the chunk are
  // the reference's is a member, and its query columns take part in one
  // pass over those rows: each of the four waves holds two 16-column
  // matrix-core blocks (32 / g sequences x g heads) and walks every token of
  // a 64-token stage, S^T = K Q^T then O^T += V^T P^T, with one online
  // softmax per column (tokens at or past a member's length are masked).
  // Each member's partial goes to piece stream_wgs + B + c * B + b.  A
  // sequence with tokens in the chunk whose entries differ runs the chunk
  // on its own blocks (the workgroup of the pair's first head does it for
  // both heads), into the same piece.
  auto prefix_unit = [&](const int y) {
    if constexpr (GRID == kGridStreamPrefix) {
      using RP = Ring<D, NW, false, 1>;                // one KV head: 64-token stages of 256-byte rows
      static_assert(RP::kMatBytes == kRingBytes && RP::kStageTok == 64, "prefix stages fill the ring slots");
      constexpr int kSpw = 32 / G;                      // sequences per wave (two column blocks)
      constexpr int kSpg = NW * kSpw;                   // sequences per workgroup
      constexpr int kCpb = 16 / G;                      // sequences per column block
      static_assert(kSpg == prefix_seqs_per_wg(G) && 3 * kSpg <= kCompactMaxB, "prefix sequence groups");
      const int lane = threadIdx.x & 63, tid = threadIdx.x;
      const int B = p.B, n_h = p.n_h;
      const int ncg = (B + kSpg - 1) / kSpg;
      const int hp = y & 1, cg = (y >> 1) % ncg, c = (y >> 1) / ncg;
      const int kvh_abs = kvh * KH + hp;
      const int S = p.prefix_tokens, CH = p.prefix_chunk;
      const int c0 = c * CH, c1 = min(S, c0 + CH);
      const int shift = p.block_shift, bmask = (1 << shift) - 1;
      int* s_mis = s_upre;                              // [kSpg]: a block of the chunk is not the reference's
      int* s_cl = s_upre + kSpg;                        // [kSpg]: context lengths of the group
      int* s_ref = s_upre + 2 * kSpg;                   // reference sequence and its length
      if (wave == 0) {
        // the reference: the longest sequence (the first of that length)
        int best = -1, bi = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int sb = 8 * lane + k;
          const int cx = sb < B ? p.context_lens[sb] : -1;
          if (cx > best) { best = cx; bi = sb; }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const int ob = __shfl_xor(best, off), oi = __shfl_xor(bi, off);
          if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        if (lane == 0) { s_ref[0] = bi; s_ref[1] = best; }
      }
      if (tid < kSpg) {
        const int b = cg * kSpg + tid;
        s_mis[tid] = 0;
        s_cl[tid] = b < B ? p.context_lens[b] : 0;
      }
      __syncthreads();
      const int ref = __builtin_amdgcn_readfirstlane(s_ref[0]);
      const int ctx_ref = __builtin_amdgcn_readfirstlane(s_ref[1]);
      const int ce = min(c1, prefix_end(ctx_ref, S, shift));
      if (ce <= c0) return;                             // no sequence reaches this chunk
      const int lb0 = c0 >> shift;
      const int nblk = ((ce - 1) >> shift) - lb0 + 1;
      {
        const int32_t* row = p.block_table + (int64_t)ref * p.max_blocks_per_seq + lb0;
        for (int i = tid; i < nblk; i += kThr) s_bt[i] = row[i];
      }
      __syncthreads();
      // DMA of the first stage(s) and the query loads go out before the
      // membership check (its table reads), so that the three are in
      // flight together
      const int ml16 = lane & 15, mg = lane >> 4;
      const int j0 = wave * RP::kDmaPerWave;             // 8 instructions of 4 rows per wave: waves 0-1 K, 2-3 V
      const bool dma_v = j0 >= RP::kDmaPerMat;
      const int jbase = j0 % RP::kDmaPerMat;
      const int64_t slot_stride = (int64_t)p.n_kv * RP::kHeadRow;
      const uint8_t* mat = reinterpret_cast<const uint8_t*>(dma_v ? p.v : p.k) + (int64_t)kvh_abs * RP::kHeadRow;
      const uint32_t lds_mat =
          (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_dma[dma_v ? 1 : 0][0][0];
      const int lrow = lane / RP::kSrcPieces, lpiece = lane % RP::kSrcPieces;
      auto spiece = [&](int r) { return lpiece ^ (dma_v ? RP::swz_v(r) : RP::swz_k(r)); };
      constexpr int kPer = 4;                            // the permutations repeat every 4 instructions (16 rows)
      static_assert(RP::kDmaPerWave % kPer == 0 && RP::kRowsPerDma * kPer == 16, "offset period");
      uint32_t pvoff[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        pvoff[i] = (uint32_t)(lrow * slot_stride) + (uint32_t)spiece((jbase + i) * RP::kRowsPerDma + lrow) * 16u;
      const bool pfast = (1 << shift) >= RP::kRowsPerDma;
      const int n_st = (ce - c0 + 63) / 64;
      auto pissue = [&](int s, int slot) {
        const int tile0 = c0 + s * 64;
        const uint32_t dst0 = lds_mat + (uint32_t)(slot * kRingBytes);
        if (pfast && tile0 + 64 <= ce) {
          int32_t ph[RP::kDmaPerWave];                 // table entries first (one LDS round trip)
#pragma unroll
          for (int jj = 0; jj < RP::kDmaPerWave; ++jj)
            ph[jj] = s_bt[((tile0 + (jbase + jj) * RP::kRowsPerDma) >> shift) - lb0];
#pragma unroll
          for (int jj = 0; jj < RP::kDmaPerWave; ++jj) {
            const int jm = jbase + jj;
            const int t0 = tile0 + jm * RP::kRowsPerDma;
            const int32_t phys = __builtin_amdgcn_readfirstlane(ph[jj]);
            const uint8_t* sb = mat + (((int64_t)phys << shift) + (t0 & bmask)) * slot_stride;
            dma16(sb, pvoff[jj % kPer], dst0 + (uint32_t)(jm * 1024));
          }
        } else {
          int32_t ph[RP::kDmaPerWave];
#pragma unroll
          for (int jj = 0; jj < RP::kDmaPerWave; ++jj) {
            const int r = (jbase + jj) * RP::kRowsPerDma + lrow;
            ph[jj] = s_bt[(min(tile0 + r, ce - 1) >> shift) - lb0];
          }
#pragma unroll
          for (int jj = 0; jj < RP::kDmaPerWave; ++jj) {
            const int jm = jbase + jj;
            const int r = jm * RP::kRowsPerDma + lrow;
            const int t = min(tile0 + r, ce - 1);
            const int64_t sl = ((int64_t)ph[jj] << shift) + (t & bmask);
            dma16(mat + sl * slot_stride + spiece(r) * 16, dst0 + (uint32_t)(jm * 1024));
          }
        }
      };
#pragma unroll
      for (int s = 0; s < RING - 1; ++s)
        if (s < n_st) pissue(s, s);
      // the lane's two columns (one per block): sequence bl of the group,
      // query head ml16 % g of KV head kvh_abs
      int bcol[2];
      u32x4_t qf2[2][kKs];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        bcol[cb] = cg * kSpg + wave * kSpw + cb * kCpb + ml16 / G;
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) +
                              ((int64_t)min(bcol[cb], B - 1) * n_h + (int64_t)kvh_abs * G + ml16 % G) * D * 2;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
          qf2[cb][ks] = *reinterpret_cast<const u32x4_t*>(qrow + (32 * ks + 8 * mg) * 2);
      }
      for (int i = tid; i < kSpg * nblk; i += kThr) {
        const int bl = i / nblk, jj = i % nblk;
        const int lim = min(prefix_end(s_cl[bl], S, shift), ce);
        if (lim > c0 && jj <= ((lim - 1) >> shift) - lb0) {
          const int b = cg * kSpg + bl;
          if (p.block_table[(int64_t)b * p.max_blocks_per_seq + lb0 + jj] != s_bt[jj]) s_mis[bl] = 1;
        }
      }
      const int any_member =
          __builtin_amdgcn_readfirstlane(__syncthreads_or(tid < kSpg && prefix_end(s_cl[tid], S, shift) > c0 &&
                                                          s_mis[tid] == 0));
      const int64_t piece0 = (int64_t)p.stream_wgs + B + (int64_t)c * B;   // + b: this chunk's piece
      if (!any_member) wait_vm_imm<0>();                  // the first stages' DMA lands before the ring is reused
      if (any_member) {
        int lim[2];
        bool mem[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int bl = bcol[cb] - cg * kSpg;
          const int pe = prefix_end(s_cl[bl], S, shift);
          mem[cb] = pe > c0 && s_mis[bl] == 0;
          lim[cb] = mem[cb] ? min(pe, ce) : 0;
#pragma unroll
          for (int ks = 0; ks < kKs; ++ks)
            if (!mem[cb]) qf2[cb][ks] = u32x4_t{0u, 0u, 0u, 0u};
        }
        f32x4_t acc2[2][kCb];
        float mm2[2] = {-INFINITY, -INFINITY}, ml2[2] = {0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int db = 0; db < kCb; ++db) acc2[cb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        const float qscale = p.scale * kLog2e;
        auto pstage = [&](int s, int slot) {
          wait_vm(min(RING - 2, n_st - 1 - s) * RP::kDmaPerWave);
          lds_barrier();
          if (s + RING - 1 < n_st) pissue(s + RING - 1, (slot + RING - 1) % RING);
          const uint8_t* kst = &s_dma[0][slot][0];
          const uint8_t* vst = &s_dma[1][slot][0];
          const int tile0 = c0 + s * 64;
          const uint32_t vbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)vst;
          const int cp = ml16 & 3;
          // the stage's four 16-token blocks in turn: scores of both column
          // blocks (one K fragment per k-step serves both), the online
          // softmax per column, then the values (a loop, not unrolled: the
          // reads of one block in flight at a time keep the registers within
          // two waves per SIMD)
#pragma unroll 1
          for (int tb = 0; tb < 4; ++tb) {
            f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
            const int row = 16 * tb + ml16;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
              const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(
                  kst + row * RP::kRowBytes + (((4 * ks + mg) ^ RP::swz_k(row)) * 16));
#pragma unroll
              for (int cb = 0; cb < 2; ++cb)
                sacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, ka), __builtin_bit_cast(bf16x8_t, qf2[cb][ks]), sacc[cb], 0, 0, 0);
            }
            i16x4_t pb[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              float sc[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sc[i] = tile0 + 16 * tb + 4 * mg + i < lim[cb] ? sacc[cb][i] * qscale : -INFINITY;
              float smax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
              {
                const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
                smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
                const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
                smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
              }
              constexpr float kSlack = 8.f;
              if (mm2[cb] == -INFINITY) {
                mm2[cb] = smax;
              } else if (__builtin_amdgcn_ballot_w64(smax > mm2[cb] + kSlack)) {
                const float m_new = fmaxf(mm2[cb], smax);
                const float alpha = __builtin_amdgcn_exp2f(mm2[cb] - m_new);
                ml2[cb] *= alpha;
#pragma unroll
                for (int db = 0; db < kCb; ++db) acc2[cb][db] *= alpha;
                mm2[cb] = m_new;
              }
              float pr[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                pr[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - mm2[cb]);
              const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{pr[0], pr[1]}), bf16x2_t));
              const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{pr[2], pr[3]}), bf16x2_t));
              ml2[cb] += (bf_lo(p01) + bf_hi(p01)) + (bf_lo(p23) + bf_hi(p23));
              pb[cb] = __builtin_bit_cast(i16x4_t, (u32x2_t{p01, p23}));
            }
            // V^T fragments by transposed reads, each used for both column blocks
            const int tv = 16 * tb + 4 * mg + (ml16 >> 2);
            const uint32_t vrow = vbase + (uint32_t)(tv * RP::kRowBytes + 8 * (cp & 1));
            const int svz = RP::swz_v(tv);
#pragma unroll
            for (int db = 0; db < kCb; ++db) {
              const uint32_t a = vrow + (uint32_t)((((2 * db + (cp >> 1)) ^ svz)) * 16);
              const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(uintptr_t)a);
#pragma unroll
              for (int cb = 0; cb < 2; ++cb)
                acc2[cb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[cb], acc2[cb][db], 0, 0, 0);
            }
          }
        };
        for (int s0 = 0; s0 < n_st; s0 += RING) {
#pragma unroll
          for (int u = 0; u < RING; ++u)
            if (s0 + u < n_st) pstage(s0 + u, u);
        }
        // each member column's partial: (max, sum) and the output over the sum
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          float L = ml2[cb];
          L += __shfl_xor(L, 16);
          L += __shfl_xor(L, 32);
          if (mem[cb]) {
            const int64_t pr = (piece0 + bcol[cb]) * n_h + (int64_t)kvh_abs * G + ml16 % G;
            const float inv = 1.0f / L;
#pragma unroll
            for (int db = 0; db < kCb; ++db)
              *reinterpret_cast<f32x4_t*>(&p.part_o[pr * D + 16 * db + 4 * mg]) = acc2[cb][db] * inv;
            if (mg == 0) { p.part_ml[2 * pr] = mm2[cb]; p.part_ml[2 * pr + 1] = L; }
          }
        }
      }
      // sequences whose blocks in the chunk are their own
      if (hp == 0) {
#pragma unroll 1
        for (int bl = 0; bl < kSpg; ++bl) {
          const int cx = __builtin_amdgcn_readfirstlane(s_cl[bl]);
          const int pe = prefix_end(cx, S, shift);
          if (pe > c0 && __builtin_amdgcn_readfirstlane(s_mis[bl])) {
            __syncthreads();                            // the ring and block table are free
            unit(cg * kSpg + bl, c0, min(c1, pe), cx, 1, piece0 * n_h, false);
          }
        }
      }
    }
  };

  if constexpr (GRID == kGridSplit) {
    // grid (KV head, sequence, split)
    const int b = blockIdx.y, split = blockIdx.z, ctx = p.context_lens[b];
    const int t_begin = window_a0(p, ctx) + split * p.split_tokens;
    if (t_begin >= ctx) {
      if (split == 0) zero_out(b);
    } else {
      unit(b, t_begin, min(ctx, t_begin + p.split_tokens), ctx, p.num_splits, split, true);
    }
  } else if constexpr (GRID == kGridCompact) {
    // Grid (KV head, unit) for ragged batches, a unit being one split of one
    // sequence; an empty sequence has one unit, which zeros its output.
    // Only units with work are launched, instead of every sequence times the
    // largest split count.  Wave 0 forms the prefix of the units per
    // sequence (B <= kCompactMaxB, 8 sequences per lane), and the workgroup
    // takes units blockIdx.y, blockIdx.y + gridDim.y, ..., so that every
    // unit is covered whatever grid size the host chose.
    if (wave == 0) {
      const int lane = threadIdx.x & 63;
      int cnt[8];
      int sum = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sb = 8 * lane + k;
        const int c = sb < p.B ? p.context_lens[sb] : 0;
        cnt[k] = sb < p.B ? max(1, (c - window_a0(p, c) + p.split_tokens - 1) / p.split_tokens) : 0;
        sum += cnt[k];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      int run = incl - sum;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        s_upre[8 * lane + k] = run;
        run += cnt[k];
      }
      if (lane == kWave - 1) s_upre[kCompactMaxB] = incl;
    }
    __syncthreads();
    const int n_units = __builtin_amdgcn_readfirstlane(s_upre[p.B]);
    for (int u = blockIdx.y; u < n_units; u += gridDim.y) {
      // the sequence whose units hold u: the largest b with s_upre[b] <= u
      int lo = 0, hi = p.B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_upre[mid] <= u) lo = mid; else hi = mid;
      }
      const int b = __builtin_amdgcn_readfirstlane(lo);
      const int split = __builtin_amdgcn_readfirstlane(u - s_upre[b]);
      const int ctx = p.context_lens[b];
      const int t_begin = window_a0(p, ctx) + split * p.split_tokens;
      if (t_begin >= ctx) {
        if (split == 0) zero_out(b);
      } else {
        unit(b, t_begin, min(ctx, t_begin + p.split_tokens), ctx, p.num_splits, split, true);
      }
      __syncthreads();                              // the unit's LDS is free again
    }
  } else {
    if constexpr (GRID == kGridStreamPrefix) {
      if ((int)blockIdx.y < p.prefix_wgs) prefix_unit(blockIdx.y);
      else stream_part(blockIdx.y - p.prefix_wgs, gridDim.y - p.prefix_wgs, p.prefix_tokens);
    } else {
      stream_part(blockIdx.y, gridDim.y, 0);
    }
  }
}

}  // namespace

bool gqa_ring_supported(KV kv, bool q_bf16, int d_k, int d_v, int g) {
  const bool g_ok = g == 4 || g == 8 || g == 16;
  if (kv == KV::INT4) return q_bf16 && d_k == 128 && d_v == 128 && g_ok;
  return (kv == KV::BF16 || kv == KV::INT8) && q_bf16 && d_k == d_v && (d_k == 64 || d_k == 128) && g_ok;
}

int gqa_ring_kv_group(KV kv, bool q_bf16, int d_k, int d_v, int g, int n_kv) {
  if (!q_bf16 || d_k != 128 || d_v != 128 || !(g == 4 || g == 8 || g == 16)) return 1;
  if (kv == KV::BF16) return PKV_GQA_PAIR && n_kv % 2 == 0 ? 2 : 1;
  if (kv == KV::INT4) return n_kv % 2 == 0 ? 2 : 0;      // INT4: pairs of KV heads only
  if (kv == KV::INT8) {
    // g = 16: at most two KV heads (the merge gives each thread 8 KH columns)
    if (PKV_Q8_KH >= 4 && n_kv % 4 == 0 && g < 16) return 4;
    if (PKV_Q8_KH >= 2 && n_kv % 2 == 0) return 2;
  }
  return 1;
}

hipError_t launch_decode_gqa_ring(const DecodeParams& p, hipStream_t stream) {
  if (p.compact_units != 0 && p.stream_wgs != 0) return hipErrorInvalidValue;
  if (p.compact_units != 0 && (p.B > kCompactMaxB || p.compact_units < 0 || p.compact_units > 65535))
    return hipErrorInvalidValue;
  if (p.stream_wgs != 0 && (p.B > kCompactMaxB || p.stream_wgs < 0 || p.stream_wgs > 65535 ||
                            p.seq_meta == nullptr))
    return hipErrorInvalidValue;
  const int g = p.n_h / p.n_kv;
  const int kh = gqa_ring_kv_group(p.kv, p.q_bf16, p.d_k, p.d_v, g, p.n_kv);
  const unsigned groups = (unsigned)(p.n_kv / kh);
  if (kh == 0) return hipErrorInvalidValue;
  const bool q4 = p.kv == KV::INT4;
  const bool q8 = p.kv == KV::INT8 || q4;
  if (q4 && (p.window != 0 || p.n_sink < 0 || p.n_sink > kMaxSink || (p.n_sink > 0 && (!p.sink_k || !p.sink_v))))
    return hipErrorInvalidValue;
  // ragged batches: the compact grid on INT8 pools, the stream grid on bf16
  // ones (each measured the faster there)
  if ((q8 && p.stream_wgs != 0) || (!q8 && p.compact_units != 0)) return hipErrorInvalidValue;
  // a split's blocks must fit the staged block table (one chunk)
  // (a windowed split starts anywhere in a block: one block more)
  if ((p.split_tokens >> p.block_shift) + (p.window ? 1 : 0) > (q8 ? kBtSlotsInt8 : kBtSlots))
    return hipErrorInvalidValue;
  // shared prefix: bf16 with two KV heads per workgroup, on the stream grid,
  // no append, chunks of whole 64-token stages whose blocks fit the table
  if (p.window < 0) return hipErrorInvalidValue;
  if (p.prefix_tokens != 0 &&
      (p.window != 0 || q8 || kh != 2 || p.d_k != 128 || p.stream_wgs <= 0 || p.prefix_wgs <= 0 || p.prefix_tokens < 0 ||
       p.prefix_tokens % 64 || p.prefix_chunk <= 0 || p.prefix_chunk % 64 || p.k_new != nullptr ||
       (p.prefix_chunk >> p.block_shift) + 2 > kBtSlots ||
       (int64_t)p.stream_wgs + p.prefix_wgs > 65535 ||
       p.prefix_wgs != 2 * ((p.prefix_tokens + p.prefix_chunk - 1) / p.prefix_chunk) *
                           ((p.B + prefix_seqs_per_wg(g) - 1) / prefix_seqs_per_wg(g))))
    return hipErrorInvalidValue;
  const dim3 grid = p.stream_wgs != 0     ? dim3(groups, (unsigned)(p.stream_wgs + (p.prefix_tokens ? p.prefix_wgs : 0)), 1u)
                    : p.compact_units != 0 ? dim3(groups, (unsigned)p.compact_units, 1u)
                                           : dim3(groups, (unsigned)p.B, (unsigned)p.num_splits);
  const int mode = p.prefix_tokens != 0 ? kGridStreamPrefix
                   : p.stream_wgs != 0  ? kGridStream
                                        : (p.compact_units != 0 ? kGridCompact : kGridSplit);
#define PKV_RING(D_, G_, Q8_, KH_)                                                                 \
  do {                                                                                              \
    constexpr int kRagged = Q8_ ? kGridCompact : kGridStream;                                       \
    const bool app8 = Q8_ && p.k_new != nullptr;                                                    \
    if (mode != kGridSplit && app8)                                                                 \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<D_, G_, kWaves, kRing, Q8_, kRagged, KH_, false, Q8_>), \
                         grid, dim3(64 * kWaves), 0, stream, p);                                   \
    else if (mode != kGridSplit)                                                                    \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<D_, G_, kWaves, kRing, Q8_, kRagged, KH_>), grid,    \
                         dim3(64 * kWaves), 0, stream, p);                                         \
    else if (app8)                                                                                  \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<D_, G_, kWaves, kRing, Q8_, kGridSplit, KH_, false, Q8_>), \
                         grid, dim3(64 * kWaves), 0, stream, p);                                   \
    else                                                                                           \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<D_, G_, kWaves, kRing, Q8_, kGridSplit, KH_>), grid, \
                         dim3(64 * kWaves), 0, stream, p);                                         \
  } while (0)
  // bf16, two KV heads per workgroup: the grids above plus the shared prefix
#define PKV_RING_PAIR(G_)                                                                           \
  do {                                                                                              \
    if (mode == kGridStreamPrefix)                                                                  \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<128, G_, kWaves, kRing, false, kGridStreamPrefix, 2>), \
                         grid, dim3(64 * kWaves), 0, stream, p);                                   \
    else                                                                                           \
      PKV_RING(128, G_, false, 2);                                                                 \
  } while (0)
  if (p.prefix_tokens != 0 && !(p.d_k == 128 && (g == 4 || g == 8 || g == 16) && !q8 && kh == 2))
    return hipErrorInvalidValue;
  // INT4 (two KV heads per workgroup, d = 128): the split or compact grid
#define PKV_RING_Q4(G_)                                                                             \
  do {                                                                                              \
    if (mode != kGridSplit)                                                                         \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<128, G_, kWaves, kRingQ4, true, kGridCompact, 2, true>), grid, \
                         dim3(64 * kWaves), 0, stream, p);                                         \
    else                                                                                           \
      hipLaunchKernelGGL((decode_gqa_ring_kernel<128, G_, kWaves, kRingQ4, true, kGridSplit, 2, true>), grid, \
                         dim3(64 * kWaves), 0, stream, p);                                         \
  } while (0)
  if (q4) {
    if (p.d_k != 128 || kh != 2) return hipErrorInvalidValue;
    if (g == 8) PKV_RING_Q4(8);
    else if (g == 4) PKV_RING_Q4(4);
    else if (g == 16) PKV_RING_Q4(16);
    else return hipErrorInvalidValue;
#undef PKV_RING_Q4
    return hipGetLastError();
  }
  if (p.d_k == 128 && g == 8) {
    if (q8 && kh == 4) PKV_RING(128, 8, true, 4);
    else if (q8 && kh == 2) PKV_RING(128, 8, true, 2);
    else if (q8) PKV_RING(128, 8, true, 1);
    else if (kh == 2) PKV_RING_PAIR(8);
    else PKV_RING(128, 8, false, 1);
  } else if (p.d_k == 128 && g == 4) {
    if (q8 && kh == 4) PKV_RING(128, 4, true, 4);
    else if (q8 && kh == 2) PKV_RING(128, 4, true, 2);
    else if (q8) PKV_RING(128, 4, true, 1);
    else if (kh == 2) PKV_RING_PAIR(4);
    else PKV_RING(128, 4, false, 1);
  } else if (p.d_k == 128 && g == 16) {
    if (q8 && kh == 2) PKV_RING(128, 16, true, 2);
    else if (q8 && kh == 1) PKV_RING(128, 16, true, 1);
    else if (q8) return hipErrorInvalidValue;
    else if (kh == 2) PKV_RING_PAIR(16);
    else PKV_RING(128, 16, false, 1);
  } else if (p.d_k == 64 && g == 16) {
    if (q8) PKV_RING(64, 16, true, 1);
    else PKV_RING(64, 16, false, 1);
  } else if (p.d_k == 64 && g == 8) {
    if (q8) PKV_RING(64, 8, true, 1);
    else PKV_RING(64, 8, false, 1);
  } else if (p.d_k == 64 && g == 4) {
    if (q8) PKV_RING(64, 4, true, 1);
    else PKV_RING(64, 4, false, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_RING_PAIR
#undef PKV_RING
  return hipGetLastError();
}

}  // namespace pkv
