// Device helpers shared by the decode kernels (wave64 reductions, bf16
// conversions, LDS ordering inside a wavefront).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {
namespace dev {

static constexpr int kWave = 64;
static constexpr int kWaves = 4;
static constexpr int kThreads = kWave * kWaves;
static constexpr int kTile = 64;                   // tokens per wave tile
static constexpr int kMaxSplitTokens = 8192;       // longest context split
static constexpr int kBtSlots = 512;               // block-table entries staged per split
static constexpr int kBtSlotsInt8 = 256;           // the same, INT8 caches (smaller LDS footprint)
static constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

static __device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
static __device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

static __device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
static __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Maximum over the 64 lanes, returned in every lane.
static __device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x124>(x));   // row_ror:4
  x = fmaxf(x, dpp<0x128>(x));   // row_ror:8
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fmaxf(fmaxf(a, b), fmaxf(c, d)))));
}

static __device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (a + b) + (c + d);
}

static __device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

static __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int N>
static __device__ __forceinline__ uint32_t kdw(const u32x4_t (&k)[N], int w) {
  return k[w >> 2][w & 3];
}

// Dword w (compile-time after unrolling) of a K row held as 16-byte pieces.
template <int N>
static __device__ __forceinline__ uint32_t kdw(const uint4 (&k)[N], int w) {
  const uint4 v = k[w >> 2];
  switch (w & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}


}  // namespace dev
}  // namespace pkv
