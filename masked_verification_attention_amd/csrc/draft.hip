// The next tree draft ("Speculative Streaming", tree draft construction and
// parallel new draft generation).
//
// The pass that verifies a draft also drafts the next one: the gamma
// speculative streams of the last accepted node -- the new root -- each give a
// logit row; stream j's k best tokens become the children of every node of
// level j - 1, under the correction token at the root.  The result is a
// complete k-ary tree of depth gamma, flattened level by level (the children
// of node p are k p + 1 .. k p + k, in the rank order of their tokens).
//
// k_topk_streams: one workgroup of 1024 threads per (request, stream), two
// passes over the row with 16-byte loads (eight in flight per thread).  Pass
// 1 takes each wave's largest value; the k-th largest of the 16 wave maxima
// is a lower bound on the row's k-th best, since it is met by k distinct
// elements.  Pass 2 (the row is then resident in L2) keeps, per thread, a
// sorted list of its best k candidates at or above the bound; the lists are
// appended to LDS and each entry's rank is the number of entries that rank
// before it ("larger value, then lower index").  More than 256 entries (long
// runs of equal values) are merged instead by k rounds of a wave-wide
// reduction over the lists.  Ties resolve to the lower token index; -0 equals +0; NaN ranks
// after every number (lowest index first among NaNs).
//
// Each top-k workgroup then writes its stream's level of the next tree
// (tokens and parents); k_draft_tree, one workgroup per request, writes the
// tree only when it is the root alone (gamma = 0).
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kTopThreads = 1024;
constexpr int kTopWaves = kTopThreads / kWave;

// (v, i) ranks before (bv, bi): larger value, then lower index
__device__ __forceinline__ bool ranks_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// First stream row of request b's new root in the multi-stream layout, or -1
// when there is none: no accepted node, a path entry outside the tree, or
// stream rows past the block.
__device__ __forceinline__ int root_stream_row(int b, int R, int gamma, const int32_t* n_nodes,
                                               const int32_t* acc_len, const int32_t* acc_path,
                                               int max_depth) {
  const int A = acc_len[b];
  if (A < 1 || A > max_depth) return -1;
  const int last = acc_path[(int64_t)b * max_depth + A - 1];
  const int n = n_nodes[b];
  if (n < 1 || last < 0 || last >= n || (int64_t)n * (1 + gamma) > R) return -1;
  return n + last * gamma;
}

// Sorted list of the K best pairs held by one lane (slots >= k stay empty).
template <int K>
struct TopList {
  float v[K];
  int i[K];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int s = 0; s < K; ++s) {
      v[s] = -INFINITY;
      i[s] = 0x7fffffff;
    }
  }
  // insertion by a pass of compare-and-swap down the list (static indices keep
  // it in registers); the displaced pair moves on, off the end past slot k-1
  __device__ __forceinline__ void push(float x, int xi, int k) {
#pragma unroll
    for (int s = 0; s < K; ++s) {
      if (s < k && ranks_before(x, xi, v[s], i[s])) {
        const float tv = v[s];
        const int ti = i[s];
        v[s] = x;
        i[s] = xi;
        x = tv;
        xi = ti;
      }
    }
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int s = 0; s + 1 < K; ++s) {
      v[s] = v[s + 1];
      i[s] = i[s + 1];
    }
    v[K - 1] = -INFINITY;
    i[K - 1] = 0x7fffffff;
  }
};

// k rounds over a wave: every lane offers its list head, the wave agrees on
// the best, the owner pops it.  Returns round r's pair in (ov[r], oi[r]) on
// every lane.
template <int K>
__device__ __forceinline__ void wave_topk(TopList<K>& L, int k, float (&ov)[K], int (&oi)[K]) {
#pragma unroll
  for (int r = 0; r < K; ++r) {
    if (r >= k) break;
    float bv = L.v[0];
    int bi = L.i[0];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float xv = __shfl_xor(bv, o);
      const int xi = __shfl_xor(bi, o);
      if (ranks_before(xv, xi, bv, bi)) {
        bv = xv;
        bi = xi;
      }
    }
    ov[r] = bv;
    oi[r] = bi;
    if (L.i[0] == bi && bi != 0x7fffffff) L.pop();
  }
}

template <typename T>
__device__ __forceinline__ float logit_at(const T* p, int i);
template <>
__device__ __forceinline__ float logit_at<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float logit_at<uint16_t>(const uint16_t* p, int i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}

// Visit every (value, index) of a row: scalar head up to 16-byte alignment,
// vector body (U loads in flight per thread), scalar tail.  Each thread sees
// its own elements in any order.
template <typename T, int U, typename F>
__device__ __forceinline__ void for_row(const T* base, int V, int tid, F&& f) {
  constexpr int E = 16 / sizeof(T);
  const int mis = (int)(((uintptr_t)base & 15u) / sizeof(T));
  const int pre = min(V, mis == 0 ? 0 : E - mis);
  for (int i = tid; i < pre; i += kTopThreads) f(logit_at<T>(base, i), i);
  const int nvec = (V - pre) / E;
  const char* vb = reinterpret_cast<const char*>(base + pre);
  constexpr int RV = U * kTopThreads;
  for (int r0 = 0; r0 < nvec; r0 += RV) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * kTopThreads + tid;
      x[u] = c < nvec ? ldg16(vb + (int64_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * kTopThreads + tid;
      if (c >= nvec) continue;
      const int i0 = pre + c * E;
      const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f(bf16lo(w[e]), i0 + 2 * e);
          f(bf16hi(w[e]), i0 + 2 * e + 1);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f(__uint_as_float(w[e]), i0 + e);
      }
    }
  }
  for (int i = pre + nvec * E + tid; i < V; i += kTopThreads) f(logit_at<T>(base, i), i);
}

// The workgroup's k best pairs of the lanes' sorted lists, valid in wave 0
// (every lane); uses the LDS staging arrays.
template <int K>
__device__ __forceinline__ void block_topk(TopList<K>& L, int k, float (&ov)[K], int (&oi)[K],
                                           float (&wv)[kTopWaves][K], int (&wi)[kTopWaves][K]) {
  wave_topk<K>(L, k, ov, oi);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < K; ++r) {
      wv[wave][r] = r < k ? ov[r] : -INFINITY;
      wi[wave][r] = r < k ? oi[r] : 0x7fffffff;
    }
  }
  __syncthreads();
  if (wave == 0) {
    L.clear();
    if (lane < kTopWaves) {
#pragma unroll
      for (int r = 0; r < K; ++r) {
        L.v[r] = wv[lane][r];
        L.i[r] = wi[lane][r];
      }
    }
    wave_topk<K>(L, k, ov, oi);
  }
}

template <typename T>
__global__ __launch_bounds__(kTopThreads) void k_topk_streams(
    const T* __restrict__ logits, int R, int V, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ acc_len, const int32_t* __restrict__ acc_path, int max_depth, int gamma,
    int k, int32_t* __restrict__ out_topk, int N, const int32_t* __restrict__ root_tok,
    int32_t* __restrict__ draft_tok, int32_t* __restrict__ tree_parent, int32_t* __restrict__ n_out) {
  constexpr int K = SPEC_MAX_TOPK;
  constexpr int U = 8;        // loads in flight per thread
  constexpr int kCap = 256;   // candidates ranked directly; more go through the list merge
  __shared__ float wv[kTopWaves][K];
  __shared__ int wi[kTopWaves][K];
  __shared__ float wmax_s[kTopWaves];
  __shared__ float cand_v[kCap];
  __shared__ int cand_i[kCap];
  __shared__ float bound_s;
  __shared__ int cnt_s, nan_s;
  __shared__ int tk_s[K];
  const int b = blockIdx.x / gamma;
  const int j = blockIdx.x % gamma;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  int32_t* dst = out_topk + ((int64_t)b * gamma + j) * k;
  // This workgroup also writes level j + 1 of the next tree, whose k^(j+1)
  // nodes are the children of level j in order: node v is the ((v-1) % k)-th
  // child of node (v-1) / k, and its token is stream j's token of that rank.
  // Stream 0's workgroup writes the root and the node count.
  int first = 1, cnt = k;
  for (int g = 0; g < j; ++g) {
    first += cnt;
    cnt *= k;
  }
  int32_t* const tok_b = draft_tok + (int64_t)b * N;
  int32_t* const par_b = tree_parent + (int64_t)b * N;
  const int row0 = root_stream_row(b, R, gamma, n_nodes, acc_len, acc_path, max_depth);
  if (row0 < 0) {   // uniform over the workgroup: no new root, no tree
    if (tid < k) dst[tid] = -1;
    for (int t = tid; t < cnt; t += kTopThreads) {
      tok_b[first + t] = -1;
      par_b[first + t] = -1;
    }
    if (j == 0 && tid == 0) {
      tok_b[0] = -1;
      par_b[0] = -1;
      n_out[b] = 0;
    }
    return;
  }
  auto put = [&](int r, int tok) __attribute__((always_inline)) {
    dst[r] = tok;
    tk_s[r] = tok;
  };
  const T* base = logits + ((int64_t)b * R + row0 + j) * V;

  // pass 1: the largest value of each wave (NaN ignored).  The k-th largest
  // of the 16 wave maxima bounds the row's k-th best from below: k distinct
  // elements reach it.
  float mv = -INFINITY;
  for_row<T, U>(base, V, tid, [&](float x, int) { mv = fmaxf(mv, x); });
  uint32_t mw[1] = {__float_as_uint(mv)};
  wave_allreduce<1>(mw, [](uint32_t (&x)[1], const uint32_t (&y)[1]) {
    x[0] = __float_as_uint(fmaxf(__uint_as_float(x[0]), __uint_as_float(y[0])));
  });
  mv = __uint_as_float(mw[0]);
  if (lane == 0) wmax_s[wave] = mv;
  if (tid == 0) cnt_s = 0;
  __syncthreads();
  if (tid < kTopWaves) {
    const float m = wmax_s[tid];
    int rank = 0;
    for (int w = 0; w < kTopWaves; ++w) {
      const float o = wmax_s[w];
      rank += (o > m || (o == m && w < tid)) ? 1 : 0;
    }
    if (rank == k - 1) bound_s = m;
  }
  __syncthreads();
  const float tv = bound_s;

  // pass 2 (the row is then resident in L2): each thread's sorted list of
  // its best k candidates, values at or above the bound.  The union of the
  // lists holds the row's top k (no thread contributes more than k of them),
  // and every element ranking before one of those is in the union too.  The
  // lists go to LDS with one append per thread after the pass.
  TopList<K> L;
  L.clear();
  for_row<T, U>(base, V, tid, [&](float x, int xi) {
    if (x >= tv) L.push(x, xi, k);
  });
  int mine = 0;
#pragma unroll
  for (int q = 0; q < K; ++q) mine += (q < k && L.i[q] != 0x7fffffff) ? 1 : 0;
  if (mine > 0) {
    const int at = atomicAdd(&cnt_s, mine);
#pragma unroll
    for (int q = 0; q < K; ++q) {
      if (q < mine && at + q < kCap) {
        cand_v[at + q] = L.v[q];
        cand_i[at + q] = L.i[q];
      }
    }
  }
  __syncthreads();
  const int n = cnt_s;
  if (n <= kCap) {
    // each candidate's rank is the number of candidates ranking before it
    if (tid < n) {
      const float cv = cand_v[tid];
      const int ci = cand_i[tid];
      int rank = 0;
      for (int c = 0; c < n; ++c) rank += ranks_before(cand_v[c], cand_i[c], cv, ci) ? 1 : 0;
      if (rank < k) put(rank, ci);
    }
    // Fewer than k numbers in the row (the bound is then -inf and every
    // number is a candidate): NaN entries follow every number, lowest index
    // first, one block-wide minimum per missing place.
    int prev = -1;
    for (int r = n; r < k; ++r) {
      if (tid == 0) nan_s = 0x7fffffff;
      __syncthreads();
      int mine = 0x7fffffff;
      for_row<T, U>(base, V, tid, [&](float x, int xi) {
        if (x != x && xi > prev && xi < mine) mine = xi;
      });
      if (mine != 0x7fffffff) atomicMin(&nan_s, mine);
      __syncthreads();
      const int got = nan_s;
      __syncthreads();
      if (tid == 0) put(r, got == 0x7fffffff ? -1 : got);
      prev = got;
    }
  } else {
    float ov[K];
    int oi[K];
    block_topk<K>(L, k, ov, oi, wv, wi);
    if (tid == 0) {
#pragma unroll
      for (int r = 0; r < K; ++r)
        if (r < k) put(r, oi[r] == 0x7fffffff ? -1 : oi[r]);
    }
  }
  __syncthreads();
  for (int t = tid; t < cnt; t += kTopThreads) {
    const int v = first + t;
    tok_b[v] = tk_s[(v - 1) % k];
    par_b[v] = (v - 1) / k;
  }
  if (j == 0 && tid == 0) {
    tok_b[0] = root_tok[b];
    par_b[0] = -1;
    n_out[b] = N;
  }
}

__global__ __launch_bounds__(256) void k_draft_tree(int R, int gamma, int k, int N,
                                                    const int32_t* __restrict__ n_nodes,
                                                    const int32_t* __restrict__ acc_len,
                                                    const int32_t* __restrict__ acc_path, int max_depth,
                                                    const int32_t* __restrict__ root_tok,
                                                    const int32_t* __restrict__ topk,
                                                    int32_t* __restrict__ draft_tok,
                                                    int32_t* __restrict__ tree_parent,
                                                    int32_t* __restrict__ n_out) {
  const int b = blockIdx.x;
  const bool ok = root_stream_row(b, R, gamma, n_nodes, acc_len, acc_path, max_depth) >= 0;
  for (int v = threadIdx.x; v < N; v += blockDim.x) {
    int tok = -1, par = -1;
    if (ok) {
      if (v == 0) {
        tok = root_tok[b];
      } else {
        // level g holds nodes [first, first + k^g); node v is the ((v-1) % k)-th
        // child of node (v-1) / k
        int first = 1, cnt = k, g = 1;
        while (v >= first + cnt) {
          first += cnt;
          cnt *= k;
          ++g;
        }
        par = (v - 1) / k;
        tok = topk[((int64_t)b * gamma + (g - 1)) * k + (v - 1) % k];
      }
    }
    draft_tok[(int64_t)b * N + v] = tok;
    tree_parent[(int64_t)b * N + v] = par;
  }
  if (threadIdx.x == 0) n_out[b] = ok ? N : 0;
}

hipError_t launch_draft_tree(const void* logits, int dtype, int B, int R, int V, const int32_t* n_nodes,
                             const int32_t* acc_len, const int32_t* acc_path, int max_depth,
                             const int32_t* root_tok, int gamma, int k, int N, int32_t* out_topk,
                             int32_t* draft_tok, int32_t* tree_parent, int32_t* n_out, hipStream_t st) {
  if (gamma == 0) {   // the tree is the root alone
    hipLaunchKernelGGL(k_draft_tree, dim3(B), dim3(256), 0, st, R, gamma, k, N, n_nodes, acc_len, acc_path,
                       max_depth, root_tok, out_topk, draft_tok, tree_parent, n_out);
    return hipGetLastError();
  }
  // the top-k workgroups write the tree as well (one level each)
  const dim3 grid((unsigned)((int64_t)B * gamma));
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(k_topk_streams<uint16_t>, grid, dim3(kTopThreads), 0, st,
                       static_cast<const uint16_t*>(logits), R, V, n_nodes, acc_len, acc_path, max_depth, gamma, k,
                       out_topk, N, root_tok, draft_tok, tree_parent, n_out);
  else
    hipLaunchKernelGGL(k_topk_streams<float>, grid, dim3(kTopThreads), 0, st, static_cast<const float*>(logits), R,
                       V, n_nodes, acc_len, acc_path, max_depth, gamma, k, out_topk, N, root_tok, draft_tok,
                       tree_parent, n_out);
  return hipGetLastError();
}

}  // namespace sv
