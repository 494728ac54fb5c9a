// KV commit: append the accepted path's block K/V rows to the cache.
//
// "Speculative Streaming" keeps the accepted main-stream tokens' KV and
// garbage-collects the pruned or rejected entries after the step;
// "Lookahead Attention" (3.2) drops the lookahead KV after the pass, so its
// callers simply do not call this.  Node v of the path is block row v; the
// node at depth d+1 goes to cache slot L + d.  One workgroup per request
// copies 16-byte chunks; the new length is written after a barrier, so the
// length arrays may alias (every thread has read the old length by then).
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void k_commit(
    int Tq, int Hkv, int row_chunks, int esize, int64_t lmax, int64_t sb, int64_t sl, int64_t sh,
    char* __restrict__ k_cache, char* __restrict__ v_cache, const int32_t* cache_len_in,
    int32_t* cache_len_out, const char* __restrict__ k_blk, const char* __restrict__ v_blk,
    const int32_t* __restrict__ out_len, const int32_t* __restrict__ out_path, int max_depth, int D) {
  const int b = blockIdx.x;
  const int64_t L = min<int64_t>(max(cache_len_in[b], 0), lmax);
  const int A = clampi(out_len[b], 0, max_depth);
  const int nw = (int)min<int64_t>(A, lmax - L);
  const int head_chunks = D * esize / 16;
  for (int idx = threadIdx.x; idx < nw * row_chunks; idx += kCommitThreads) {
    const int d = idx / row_chunks;
    const int c = idx % row_chunks;
    const int row = out_path[(int64_t)b * max_depth + d];
    if (row < 0 || row >= Tq) continue;
    const int h = c / head_chunks;
    const int cc = c % head_chunks;
    const int64_t src = ((((int64_t)b * Tq + row) * Hkv + h) * D) * esize + cc * 16;
    const int64_t dst = ((int64_t)b * sb + (L + d) * sl + (int64_t)h * sh) * esize + cc * 16;
    *reinterpret_cast<u32x4*>(k_cache + dst) = ldg16(k_blk + src);
    *reinterpret_cast<u32x4*>(v_cache + dst) = ldg16(v_blk + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) cache_len_out[b] = (int32_t)(L + nw);
}

hipError_t launch_commit(int B, int Tq, int Hkv, int D, int esize, int64_t lmax, int64_t sb,
                         int64_t sl, int64_t sh, void* k_cache, void* v_cache,
                         const int32_t* cache_len_in, int32_t* cache_len_out, const void* k_blk,
                         const void* v_blk, const int32_t* out_len, const int32_t* out_path,
                         int max_depth, hipStream_t st) {
  const int row_chunks = Hkv * D * esize / 16;
  hipLaunchKernelGGL(k_commit, dim3(B), dim3(kCommitThreads), 0, st, Tq, Hkv, row_chunks, esize, lmax, sb,
                     sl, sh, static_cast<char*>(k_cache), static_cast<char*>(v_cache), cache_len_in,
                     cache_len_out, static_cast<const char*>(k_blk), static_cast<const char*>(v_blk),
                     out_len, out_path, max_depth, D);
  return hipGetLastError();
}

}  // namespace sv
