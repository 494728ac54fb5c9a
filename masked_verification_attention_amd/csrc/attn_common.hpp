// Pieces of the matrix-core attention kernel: the LDS ring geometry and its
// swizzle, the direct-to-LDS load, wave waits and barriers.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

template <int D, int NB>
struct MfmaCfg {
  static constexpr int kThreads = 512;
  static constexpr int kWaves = 8;
  static constexpr int TK = 32;                  // keys per tile
  static constexpr int CH = D / 8;               // 16-byte chunks per key row
  static constexpr int ROWB = D * 2;             // bytes per key row
  static constexpr int TILEB = TK * ROWB;        // bytes of a K (or V) tile
  static constexpr int RPI = 64 / CH;            // key rows per 1 KB wave load
  static constexpr int LPT = TK / RPI;           // wave loads per K (or V) tile
  static constexpr int LPS = 2 * LPT / 4;        // wave loads per wave per step (a group's K + V tile over its 4 waves)
  static constexpr int P = 6;                    // tiles in flight per ring (P / 2 steps ahead)
  static constexpr int NSK = P + 2;              // K slots: P in flight + the 2 being scored
  static constexpr int NSV = P + 2;              // V slots: P in flight + the 2 in P*V
  static constexpr int ROWS = 64 * NB;           // rows per workgroup
  static constexpr int MAXW = (SPEC_MAX_TQ + 31) / 32;
  static_assert(LPS >= 1 && (2 * LPT) % 4 == 0 && LPT % LPS == 0,
                "each wave's loads of a step must fall in one tile");
  // chunk position of 16-byte chunk c of key row r is c ^ swz(r).  For 256-byte
  // rows this is the GF(2)-linear map with columns 3, 10, 4, 12 on the row's low
  // four bits: measured free of bank conflicts both for the 16-byte K reads (16
  // consecutive rows, one chunk) and for the transposing V reads (4 rows of two
  // adjacent chunks per 16 lanes), where plain c ^ (r mod 16) costs the V read
  // 2-way conflicts.  128-byte rows keep c ^ (r mod 8).
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (CH == 16)
      return ((r & 1) ? 3 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 4 : 0) ^ ((r & 8) ? 12 : 0);
    else
      return r & (CH - 1);
  }
};

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

__device__ __forceinline__ lds_char* to_lds(const char* p) { return (lds_char*)(char*)p; }

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] and [15:14]; expcnt [6:4] and lgkmcnt [11:8] left unconstrained
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// 16-byte direct-to-LDS load: lane i's 16 bytes from src land at LDS byte
// address lds + 16 i (lds must be wave-uniform).  Issued through asm so that
// the compiler does not serialise the ring with its own conservative waits;
// completion is tracked explicitly with wait_vmcnt.  The LDS address is an
// input bound to m0, so the compiler itself writes m0 before the load and
// knows the register is in use.
__device__ __forceinline__ void dma16(uint32_t lds, const char* src) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// 4-byte direct-to-LDS load: lane i's word lands at LDS byte address lds + 4 i.
__device__ __forceinline__ void dma4(uint32_t lds, const void* src) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// 1-byte direct-to-LDS load: lane i's byte lands zero-extended as the 4-byte
// word at LDS byte address lds + 4 i (checked on the device).
__device__ __forceinline__ void dma1(uint32_t lds, const void* src) {
  asm volatile("global_load_lds_ubyte %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Wait until every LDS read (and scalar load) of this wave has returned.
__device__ __forceinline__ void wait_lgkm0() {
  // vmcnt and expcnt at their maxima (unconstrained), lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace sv
