// KV commit: append the accepted path's block K/V rows to the cache.
//
// "Speculative Streaming" keeps the accepted main-stream tokens' KV and
// garbage-collects the pruned or rejected entries after the step;
// "Lookahead Attention" (3.2) drops the lookahead KV after the pass, so its
// callers simply do not call this.  Node v of the path is block row v; the
// node at depth d+1 goes to cache slot L + d.  One workgroup per request
// copies 16-byte chunks; the new length is written after a barrier, so the
// length arrays may alias (every thread has read the old length by then).
#include "commit_rows.hpp"

namespace sv {

constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void k_commit(CommitArgs c, const int32_t* __restrict__ out_len,
                                                           const int32_t* __restrict__ out_path, int max_depth) {
  const int b = blockIdx.x;
  const int64_t len_in = c.cache_len_in[b];
  const int A = clampi(out_len[b], 0, max_depth);
  commit_rows(b, c, A, out_path + (int64_t)b * max_depth, len_in);
}

hipError_t launch_commit(int B, int Tq, int Hkv, int D, int esize, int64_t lmax, int64_t sb,
                         int64_t sl, int64_t sh, int v_tiled, void* k_cache, void* v_cache,
                         const int32_t* cache_len_in, int32_t* cache_len_out, const void* k_blk,
                         const void* v_blk, const int32_t* out_len, const int32_t* out_path,
                         int max_depth, hipStream_t st) {
  CommitArgs c{1, Tq, Hkv, D, esize, lmax, sb, sl, sh, v_tiled, static_cast<char*>(k_cache), static_cast<char*>(v_cache),
               cache_len_in, cache_len_out, static_cast<const char*>(k_blk), static_cast<const char*>(v_blk)};
  hipLaunchKernelGGL(k_commit, dim3(B), dim3(kCommitThreads), 0, st, c, out_len, out_path, max_depth);
  return hipGetLastError();
}

}  // namespace sv
