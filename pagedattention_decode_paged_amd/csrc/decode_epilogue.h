// End of a GQA decode workgroup: merge the 4 wavefronts' (m, l, acc) and
// finish the split.  Shared by the float and INT8 kernels.
//
// A sequence whose context fits one split writes its output directly.
// Otherwise every split writes a normalised partial (m, l, o) to the
// workspace and decode_reduce (decode_gqa.hip) merges them.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace pkv {
namespace dev {

static __device__ __forceinline__ void store_out(const DecodeParams& p, int64_t o, float r) {
  if (p.q_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(r);
  else reinterpret_cast<float*>(p.out)[o] = r;
}

// Zero output of an empty sequence (written by split 0 only).
template <int G, int D>
static __device__ __forceinline__ void write_zero_rows(const DecodeParams& p, int b, int kvh) {
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
    store_out(p, ((int64_t)b * p.n_h + (int64_t)kvh * G) * D + idx, 0.f);
}

template <int G, int D>
static __device__ __forceinline__ void finish_split(const DecodeParams& p, int b, int kvh, int split,
                                                    int ctx, float (&s_m)[kWaves][G],
                                                    float (&s_l)[kWaves][G],
                                                    float (&s_acc)[kWaves][G * D]) {
  const int tid = threadIdx.x;
  const int nsp = (ctx + p.split_tokens - 1) / p.split_tokens;   // splits holding tokens
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
    const int64_t row = (int64_t)b * p.n_h + (int64_t)kvh * G + h;
    if (nsp == 1) {
      store_out(p, row * D + d, O / L);
    } else {
      const int64_t pi = row * p.num_splits + split;
      p.part_o[pi * D + d] = O / L;
      if (d == 0) { p.part_ml[2 * pi] = M; p.part_ml[2 * pi + 1] = L; }
    }
  }
}

}  // namespace dev
}  // namespace pkv
