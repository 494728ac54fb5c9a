// Device helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sv {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// bf16 bit patterns (low / high half of a 32-bit word) -> float, exact.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f2bf_rne(lo) | (f2bf_rne(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wave-wide reductions (all 64 lanes get the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Cross-lane moves by DPP, a modifier of a plain vector move (no LDS round
// trip, unlike __shfl_xor, which becomes ds_bpermute).  Within each row of 16
// lanes: 0xB1 swaps neighbours (lane ^ 1), 0x4E swaps pairs (lane ^ 2), 0x141
// mirrors each half-row (lane i <-> 7 - i), 0x140 mirrors the row
// (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xf, 0xf, false);
}

// All-reduce of an N-word state over the 64 lanes of a wave, every lane
// active: four DPP stages make each row of 16 lanes agree (swap neighbours,
// swap pairs, then mirror halves and rows, so every stage folds two disjoint
// groups), then the four row results are read into scalars and folded.
// combine(a, b) folds b into a and must be associative and commutative (a
// selection by a total order is).  Every lane gets the result.
template <int N, typename Combine>
__device__ __forceinline__ void wave_allreduce(uint32_t (&w)[N], Combine combine) {
  auto stage = [&](auto ctrl) __attribute__((always_inline)) {
    uint32_t o[N];
#pragma unroll
    for (int q = 0; q < N; ++q) o[q] = dpp_u32<decltype(ctrl)::value>(w[q]);
    combine(w, o);
  };
  stage(std::integral_constant<int, 0xB1>{});
  stage(std::integral_constant<int, 0x4E>{});
  stage(std::integral_constant<int, 0x141>{});
  stage(std::integral_constant<int, 0x140>{});
  uint32_t r[N];
#pragma unroll
  for (int q = 0; q < N; ++q) r[q] = (uint32_t)__builtin_amdgcn_readlane((int)w[q], 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    uint32_t o[N];
#pragma unroll
    for (int q = 0; q < N; ++q) o[q] = (uint32_t)__builtin_amdgcn_readlane((int)w[q], 16 * row);
    combine(r, o);
  }
#pragma unroll
  for (int q = 0; q < N; ++q) w[q] = r[q];
}

// 16-byte global load through the vector path.
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// 16-byte load of data read exactly once (streaming: no reuse in the caches)
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace sv
