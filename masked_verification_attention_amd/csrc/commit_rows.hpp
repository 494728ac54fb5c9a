// Copy of the accepted path's block K/V rows into the cache, shared by the
// commit kernel and the fused acceptance + commit kernel.  Node at depth d+1
// of the path (block row path[d]) goes to cache slot L + d; slots past the
// capacity are neither written nor counted.  The new length is written after
// a barrier, so the length arrays may alias.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

// len_in is cache_len_in[b], read by the caller as early as it can (it does not
// depend on the acceptance).  Each thread issues the loads of up to four of its
// 16-byte chunks before their stores, so the copy costs one memory round trip.
__device__ __forceinline__ void commit_rows(int b, const CommitArgs& c, int A, const int32_t* path,
                                            int64_t len_in) {
  constexpr int kU = 4;
  const int64_t L = min<int64_t>(max<int64_t>(len_in, 0), c.lmax);
  const int nw = (int)min<int64_t>(A, c.lmax - L);
  const int head_chunks = c.D * c.esize / 16;
  const int row_chunks = c.Hkv * head_chunks;
  const int total = nw * row_chunks;
  for (int i0 = threadIdx.x; i0 < total; i0 += kU * blockDim.x) {
    u32x4 kx[kU], vx[kU];
    int64_t dst[kU];
    bool on[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int idx = i0 + u * blockDim.x;
      const int d = idx / row_chunks;
      const int ch = idx % row_chunks;
      const int row = idx < total ? path[d] : -1;
      on[u] = row >= 0 && row < c.Tq;
      dst[u] = 0;
      if (on[u]) {
        const int h = ch / head_chunks;
        const int cc = ch % head_chunks;
        const int64_t src = ((((int64_t)b * c.Tq + row) * c.Hkv + h) * c.D) * c.esize + cc * 16;
        dst[u] = ((int64_t)b * c.sb + (L + d) * c.sl + (int64_t)h * c.sh) * c.esize + cc * 16;
        kx[u] = ldg16(c.k_blk + src);
        vx[u] = ldg16(c.v_blk + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (on[u]) {
        *reinterpret_cast<u32x4*>(c.k_cache + dst[u]) = kx[u];
        if (!c.v_tiled) {
          *reinterpret_cast<u32x4*>(c.v_cache + dst[u]) = vx[u];
        } else {
          // fragment-major 32-key tiles (head-major, sl == D): key l = 32 t + k,
          // dim x at (l - k) * D + (x / 16) * 512 + g * 128 + (x % 16) * 8 + e
          // within the head's range, with g = (k % 16) / 4, e = k % 4 + 4 (k / 16)
          const int idx = i0 + u * blockDim.x;
          const int d = idx / row_chunks;
          const int ch = idx % row_chunks;
          const int h = ch / head_chunks, cc = ch % head_chunks;
          const int64_t l = L + d;
          const int k = (int)(l % 32);
          const int g = (k & 15) >> 2, e = (k & 3) + 4 * (k >> 4);
          const int64_t base = (int64_t)b * c.sb + (int64_t)h * c.sh + (l - k) * c.D + g * 128 + e;
          uint16_t e16[8];
          __builtin_memcpy(e16, &vx[u], 16);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int x = cc * 8 + j;
            reinterpret_cast<uint16_t*>(c.v_cache)[base + (x >> 4) * 512 + (x & 15) * 8] = e16[j];
          }
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) c.cache_len_out[b] = (int32_t)(L + nw);
}

}  // namespace sv
