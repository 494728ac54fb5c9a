// Measured ceilings of the GPU the benchmark runs on, reported next to the
// published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 on MI355X):
//
//   spec_probe_hbm_read  a plain streaming read of a large buffer: every
//                        lane reads 16-byte chunks (non-temporal), four in
//                        flight, a grid-stride loop over the whole buffer.
//   spec_probe_mfma      back-to-back bf16 matrix instructions with no memory
//                        traffic: each wave runs independent accumulator
//                        chains of `iters` instructions -- 16 chains of
//                        16x16x32 or 8 chains of 32x32x16 (measured: with 4
//                        chains the 16x16x32 form reaches only ~1.3 PFLOP/s,
//                        the 32x32x16 form ~2.2 already).
//
// Both only enqueue one launch on `stream`; the caller times it with events.
// Not part of the verification library's ABI: a separate shared object that
// only the benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_hbm_read(const u32x4* __restrict__ buf, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;   // keeps the loads; practically never stores
}

template <int KIND>
__global__ __launch_bounds__(256) void k_mfma(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  float total = 0.f;
  if constexpr (KIND == 0) {
    f32x4 c[16] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) total += c[j][0] + c[j][3];
  } else {
    f32x16 c[8] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) total += c[j][0] + c[j][15];
  }
  if (total == 12345.f) sink[blockIdx.x] = total;   // keeps the chains; practically never stores
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from the device buffer `buf`; `sink` needs
// `nwg` floats' worth of room.  Returns a hipError_t value.
int spec_probe_hbm_read(const void* buf, size_t bytes, void* sink, int nwg, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || nwg < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_hbm_read, dim3(nwg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `nwg` workgroups of 4 waves, each wave running `iters` rounds of its chains:
// kind 0 = 16 chains of 16x16x32 (16384 flops each), kind 1 = 8 chains of
// 32x32x16 (32768 flops each).  `sink` needs `nwg` floats.
int spec_probe_mfma(int kind, int nwg, int iters, float* sink, void* stream) {
  if (sink == nullptr || nwg < 1 || iters < 1 || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(k_mfma<0>, dim3(nwg), dim3(256), 0, s, sink, iters);
  else hipLaunchKernelGGL(k_mfma<1>, dim3(nwg), dim3(256), 0, s, sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
