// Block visibility mask from a parent array.
//
// Row r of the speculative block sees block key c iff c == r or c is an
// ancestor of r ("Speculative Streaming", tree draft and Equation 4 read
// through its prose; "Lookahead Attention" section 3.1 when the originals
// form a chain and the lookahead rows hang off the last original; ConFu key
// design 1 for contemplate rows, whose parent is their node).  One workgroup
// per request; each thread walks its row's parent chain and sets bits in an
// LDS copy of the row, then the words are stored with plain vector stores.
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kMaskThreads = 256;
constexpr int kMaxW = (SPEC_MAX_TQ + 31) / 32;

__global__ __launch_bounds__(kMaskThreads) void k_build_mask(
    const int32_t* __restrict__ attn_parent, const uint8_t* __restrict__ sp_flag,
    const int32_t* __restrict__ n_q, int Tq, int W, uint32_t* __restrict__ mask_bits,
    uint32_t* __restrict__ sp_bits) {
  __shared__ int32_t par[SPEC_MAX_TQ];
  __shared__ uint8_t spf[SPEC_MAX_TQ];
  __shared__ uint32_t words[SPEC_MAX_TQ][kMaxW + 1];
  const int b = blockIdx.x;
  const int nq = clampi(n_q[b], 0, Tq);
  // parents and soft-prompt flags in one round trip (coalesced), into LDS
  for (int r = threadIdx.x; r < Tq; r += kMaskThreads) {
    par[r] = attn_parent[(int64_t)b * Tq + r];
    spf[r] = sp_flag != nullptr ? sp_flag[(int64_t)b * Tq + r] : 0;
    for (int w = 0; w < W; ++w) words[r][w] = 0u;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nq; r += kMaskThreads) {
    words[r][r >> 5] |= 1u << (r & 31);
    int cur = r;
    int p = par[r];
    // parents must point strictly upwards; the walk ends at -1 or at the
    // first link that breaks that, so it always terminates within r steps
    while (p >= 0 && p < cur) {
      words[r][p >> 5] |= 1u << (p & 31);
      cur = p;
      p = par[p];
    }
  }
  __syncthreads();
  uint32_t* dst = mask_bits + (int64_t)b * Tq * W;
  for (int i = threadIdx.x; i < Tq * W; i += kMaskThreads) dst[i] = words[i / W][i % W];
  for (int w = threadIdx.x; w < W; w += kMaskThreads) {
    uint32_t bits = 0u;
    for (int i = 0; i < 32; ++i) {
      const int r = w * 32 + i;
      if (r < nq && spf[r] != 0) bits |= 1u << i;
    }
    sp_bits[(int64_t)b * W + w] = bits;
  }
}

// Multi-stream rows ("Speculative Streaming", Multi-Stream Attention,
// Equations 1 and 2, over the tree draft of its Equation 4).  For a request
// with n tree nodes, row v < n is node v's main stream and row
// n + v * gamma + (j - 1) its speculative stream j.  A main row sees the main
// rows on its node's root-to-node path; stream j of node v sees those and
// streams 1..j of v.  One workgroup per request, one thread per row: the
// thread sets its node's own stream bits, then walks the tree parents.
__global__ __launch_bounds__(kMaskThreads) void k_build_msa_mask(
    const int32_t* __restrict__ tree_parent, const int32_t* __restrict__ n_nodes, int N, int gamma,
    int Tq, int W, uint32_t* __restrict__ mask_bits, uint32_t* __restrict__ sp_bits,
    int32_t* __restrict__ n_q) {
  __shared__ int32_t par[SPEC_MAX_TQ];
  __shared__ uint32_t words[SPEC_MAX_TQ][kMaxW + 1];
  const int b = blockIdx.x;
  const int n = clampi(n_nodes[b], 0, N);
  const int nq = n * (1 + gamma);
  for (int v = threadIdx.x; v < N; v += kMaskThreads) par[v] = tree_parent[(int64_t)b * N + v];
  for (int r = threadIdx.x; r < Tq; r += kMaskThreads)
    for (int w = 0; w < W; ++w) words[r][w] = 0u;
  __syncthreads();
  for (int r = threadIdx.x; r < nq; r += kMaskThreads) {
    const int v = r < n ? r : (r - n) / gamma;   // r >= n only when gamma >= 1
    const int j = r < n ? 0 : (r - n) % gamma + 1;
    for (int i = 1; i <= j; ++i) {
      const int c = n + v * gamma + i - 1;
      words[r][c >> 5] |= 1u << (c & 31);
    }
    words[r][v >> 5] |= 1u << (v & 31);
    int cur = v;
    int p = par[v];
    // tree parents must point strictly upwards; the walk ends at -1 or at the
    // first link that breaks that
    while (p >= 0 && p < cur) {
      words[r][p >> 5] |= 1u << (p & 31);
      cur = p;
      p = par[p];
    }
  }
  __syncthreads();
  uint32_t* dst = mask_bits + (int64_t)b * Tq * W;
  for (int i = threadIdx.x; i < Tq * W; i += kMaskThreads) dst[i] = words[i / W][i % W];
  for (int w = threadIdx.x; w < W; w += kMaskThreads) sp_bits[(int64_t)b * W + w] = 0u;
  if (threadIdx.x == 0) n_q[b] = nq;
}

hipError_t launch_build_msa_mask(const int32_t* tree_parent, const int32_t* n_nodes, int B, int N,
                                 int gamma, int Tq, uint32_t* mask_bits, uint32_t* sp_bits,
                                 int32_t* n_q, hipStream_t st) {
  const int W = (Tq + 31) / 32;
  hipLaunchKernelGGL(k_build_msa_mask, dim3(B), dim3(kMaskThreads), 0, st, tree_parent, n_nodes, N,
                     gamma, Tq, W, mask_bits, sp_bits, n_q);
  return hipGetLastError();
}

hipError_t launch_build_mask(const int32_t* attn_parent, const uint8_t* sp_flag, const int32_t* n_q,
                             int B, int Tq, uint32_t* mask_bits, uint32_t* sp_bits, hipStream_t st) {
  const int W = (Tq + 31) / 32;
  hipLaunchKernelGGL(k_build_mask, dim3(B), dim3(kMaskThreads), 0, st, attn_parent, sp_flag, n_q, Tq,
                     W, mask_bits, sp_bits);
  return hipGetLastError();
}

}  // namespace sv
