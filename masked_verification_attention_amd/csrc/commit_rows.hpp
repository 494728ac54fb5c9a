// Copy of the accepted path's block K/V rows into the cache, shared by the
// commit kernel and the fused acceptance + commit kernel.  Node at depth d+1
// of the path (block row path[d]) goes to cache slot L + d; slots past the
// capacity are neither written nor counted.  The new length is written after
// a barrier, so the length arrays may alias.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

__device__ __forceinline__ void commit_rows(int b, const CommitArgs& c, int A, const int32_t* path) {
  const int64_t L = min<int64_t>(max(c.cache_len_in[b], 0), c.lmax);
  const int nw = (int)min<int64_t>(A, c.lmax - L);
  const int head_chunks = c.D * c.esize / 16;
  const int row_chunks = c.Hkv * head_chunks;
  for (int idx = threadIdx.x; idx < nw * row_chunks; idx += blockDim.x) {
    const int d = idx / row_chunks;
    const int ch = idx % row_chunks;
    const int row = path[d];
    if (row < 0 || row >= c.Tq) continue;
    const int h = ch / head_chunks;
    const int cc = ch % head_chunks;
    const int64_t src = ((((int64_t)b * c.Tq + row) * c.Hkv + h) * c.D) * c.esize + cc * 16;
    const int64_t dst = ((int64_t)b * c.sb + (L + d) * c.sl + (int64_t)h * c.sh) * c.esize + cc * 16;
    *reinterpret_cast<u32x4*>(c.k_cache + dst) = ldg16(c.k_blk + src);
    *reinterpret_cast<u32x4*>(c.v_cache + dst) = ldg16(c.v_blk + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) c.cache_len_out[b] = (int32_t)(L + nw);
}

}  // namespace sv
