// Greedy acceptance of a draft tree.
//
// k_argmax: the greedy target token of every node -- the index of its row's
// largest logit ("Speculative Streaming", the verification step: hard
// matching against the target's most likely token; "Lookahead Attention"
// 2.3).  One workgroup per node row streams the vocabulary with 16-byte loads,
// two rounds of eight in flight per thread; each thread keeps its best (value, index) in
// increasing index order, and the workgroup reduces with the rule "larger
// value, then lower index", so ties resolve to the lowest index and -0
// compares equal to +0.
//
// k_accept: one workgroup per request, one thread per node.  A node matches
// when its draft equals the greedy token of its verification row -- its own
// row, or a given row (a real model checks a child against its parent's
// prediction; row -1 accepts an explicit root unchecked).  Each thread
// walks its node's path to the root: the node is accepted iff every node on
// the path matches and the path is no longer than max_depth.  The
// accepted length is the largest accepted depth ("Speculative Streaming":
// the longest accepted path; "Lookahead Attention" 2.4: the longest
// consistent prefix of a chain).  Among the deepest accepted nodes the path a
// depth-first walk meets first (children in increasing index) is the one
// with the lexicographically smallest root-first index sequence; node indices
// are < 256 and paths are <= 16 long, so a path packs into a 128-bit key
// (8 bits per depth, root in the top byte) and a min-reduction finds it.  The
// correction token is the greedy token of the path's last node's row
// ("Speculative Streaming", the verification step: one token from the
// target's logits where the walk stopped).
//
// Acceptance by probability (the same scan, other per-node decisions): the
// target's probability p of a node's draft at its verification row, from
// the row's log-sum-exp (k_argmax_lse), either exceeds a threshold
// ("Lookahead Attention", its verification) or beats a given uniform draw
// scaled by the draft's own probability -- u * p_draft < p, i.e. acceptance
// with probability min(1, p / p_draft) ("Speculative Streaming", soft
// matching after Leviathan et al.).
#include "commit_rows.hpp"
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kArgThreads = 256;

__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <typename T>
__device__ __forceinline__ float elem_at(const T* p, int i);
template <>
__device__ __forceinline__ float elem_at<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float elem_at<uint16_t>(const uint16_t* p, int i) {
  return __uint_as_float(uint32_t(p[i]) << 16);
}

// Within one thread the indices it visits only increase, so a strict ">" keeps
// the first maximum; the full rule is needed only when merging threads.
__device__ __forceinline__ void first_max(float& bv, int& bi, float v, int i) {
  const bool gt = v > bv;
  bv = gt ? v : bv;
  bi = gt ? i : bi;
}

template <typename T>
__device__ __forceinline__ void scan16(float& bv, int& bi, const u32x4& x, int i0) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      first_max(bv, bi, bf16lo(w[e]), i0 + 2 * e);
      first_max(bv, bi, bf16hi(w[e]), i0 + 2 * e + 1);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) first_max(bv, bi, __uint_as_float(w[e]), i0 + e);
  }
}

// First entry of a row that is a number, or 0 for a row of NaN only: the
// greedy token of a row none of whose entries exceeds -inf.  One more pass by
// the whole workgroup (rows like this do not occur in practice); s_min is an
// LDS word.
template <typename T>
__device__ __noinline__ int first_number(const T* __restrict__ base, int V, int* s_min) {
  if (threadIdx.x == 0) *s_min = 0x7fffffff;
  __syncthreads();
  int mine = 0x7fffffff;
  for (int i = threadIdx.x; i < V; i += kArgThreads) {
    const float x = elem_at<T>(base, i);
    if (x == x) {
      mine = i;
      break;
    }
  }
  if (mine != 0x7fffffff) atomicMin(s_min, mine);
  __syncthreads();
  const int r = *s_min;
  return r == 0x7fffffff ? 0 : r;
}

// First maximum of one logit row by the whole workgroup (NaN ranks after every
// number); every thread gets the index.  res is an LDS word.
template <typename T, int U>   // U: 16-byte loads in flight per thread and buffer
__device__ __forceinline__ int row_argmax(const T* __restrict__ base, int V, float* sv_, int* si_, int* res) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
  const int mis = (int)(((uintptr_t)base & 15u) / sizeof(T));
  const int pre = min(V, mis == 0 ? 0 : E - mis);
  // two independent running maxima (even / odd load slots) shorten the dependency chain
  float bv0 = -INFINITY, bv1 = -INFINITY;
  int bi0 = 0x7fffffff, bi1 = 0x7fffffff;
  for (int i = threadIdx.x; i < pre; i += kArgThreads) first_max(bv0, bi0, elem_at<T>(base, i), i);
  const int nvec = (V - pre) / E;
  const char* vb = reinterpret_cast<const char*>(base + pre);
  // Rounds of U loads per thread, double-buffered: round r+1 is in flight while
  // round r is scanned.  Loads past the end return an all -inf vector, which
  // never replaces a maximum.
  constexpr int R = U * kArgThreads;   // vectors per round
  constexpr uint32_t kNegInf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
  const int nround = (nvec + R - 1) / R;
  auto load = [&](u32x4 (&x)[U], int r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = r * R + u * kArgThreads + (int)threadIdx.x;
      x[u] = k < nvec ? ldg16_stream(vb + (int64_t)k * 16) : u32x4{kNegInf, kNegInf, kNegInf, kNegInf};
    }
  };
  auto scan = [&](const u32x4 (&x)[U], int r) {
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      scan16<T>(bv0, bi0, x[u], pre + (r * R + u * kArgThreads + (int)threadIdx.x) * E);
      scan16<T>(bv1, bi1, x[u + 1], pre + (r * R + (u + 1) * kArgThreads + (int)threadIdx.x) * E);
    }
  };
  u32x4 xa[U], xb[U];
  if (nround > 0) load(xa, 0);
  int r = 0;
  for (; r + 1 < nround; r += 2) {
    load(xb, r + 1);
    scan(xa, r);
    if (r + 2 < nround) load(xa, r + 2);
    scan(xb, r + 1);
  }
  if (r < nround) scan(xa, r);
  for (int i = pre + nvec * E + threadIdx.x; i < V; i += kArgThreads) first_max(bv1, bi1, elem_at<T>(base, i), i);
  float bv = bv0;
  int bi = bi0;
  better(bv, bi, bv1, bi1);

  uint32_t pair[2] = {__float_as_uint(bv), (uint32_t)bi};
  wave_allreduce<2>(pair, [](uint32_t (&x)[2], const uint32_t (&y)[2]) {
    float v = __uint_as_float(x[0]);
    int i = (int)x[1];
    better(v, i, __uint_as_float(y[0]), (int)y[1]);
    x[0] = __float_as_uint(v);
    x[1] = (uint32_t)i;
  });
  bv = __uint_as_float(pair[0]);
  bi = (int)pair[1];
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    sv_[wave] = bv;
    si_[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / kWave; ++w) better(bv, bi, sv_[w], si_[w]);
    *res = bi;
  }
  __syncthreads();
  // the scan only takes values above -inf: a row without one gets its first
  // number (a -inf) or 0 in a second pass
  const int top = *res;
  return top == 0x7fffffff ? first_number<T>(base, V, si_) : top;
}

template <typename T, int U>
__global__ __launch_bounds__(kArgThreads) void k_argmax(const T* __restrict__ logits, int T_, int V,
                                                        const int32_t* __restrict__ n_nodes,
                                                        int32_t* __restrict__ out) {
  __shared__ float sv_[kArgThreads / kWave];
  __shared__ int si_[kArgThreads / kWave];
  __shared__ int res;
  const int row = blockIdx.x;
  const int b = row / T_;
  const int v = row % T_;
  const int n = clampi(n_nodes[b], 0, T_);
  if (v >= n) {
    if (threadIdx.x == 0) out[row] = -1;
    return;
  }
  const int bi = row_argmax<T, U>(logits + (int64_t)row * V, V, sv_, si_, &res);
  if (threadIdx.x == 0) out[row] = bi;
}

// k_argmax_lse: the greedy token and the log-sum-exp of every node row, for
// acceptance by probability.  Same stream as k_argmax; each thread also keeps
// a running maximum m and sum s of exp(x - m) (in the log2 domain), moving m
// once per 16-byte vector; the workgroup merges (m, s) pairs.  A row holding a
// NaN entry gets a NaN log-sum-exp (its softmax is undefined), and rows past
// n_nodes get argmax -1 and a NaN log-sum-exp.
template <typename T>
__global__ __launch_bounds__(kArgThreads) void k_argmax_lse(const T* __restrict__ logits, int T_, int V,
                                                            const int32_t* __restrict__ n_nodes,
                                                            int32_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int E = 16 / sizeof(T);
  constexpr int U = 8;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float sv_[kArgThreads / kWave];
  __shared__ int si_[kArgThreads / kWave];
  __shared__ float sm_[kArgThreads / kWave];
  __shared__ float ss_[kArgThreads / kWave];
  __shared__ int sn_[kArgThreads / kWave];
  const int row = blockIdx.x;
  const int b = row / T_;
  const int v = row % T_;
  const int n = clampi(n_nodes[b], 0, T_);
  if (v >= n) {
    if (threadIdx.x == 0) {
      out[row] = -1;
      lse[row] = __builtin_nanf("");
    }
    return;
  }
  const T* base = logits + (int64_t)row * V;
  float bv = -INFINITY, m = -INFINITY, s = 0.f;   // m, s in log2 units
  int bi = 0x7fffffff;
  bool nanf = false;                                // a NaN entry makes the row's log-sum-exp NaN
  auto add = [&](float x, int i) {
    nanf = nanf || x != x;
    better(bv, bi, x, i);
    const float y = x * kLog2e;
    if (y > m) {
      s = m == -INFINITY ? 0.f : s * fast_exp2(m - y);
      m = y;
    }
    if (m != -INFINITY) s += fast_exp2(y - m);
  };
  const int mis = (int)(((uintptr_t)base & 15u) / sizeof(T));
  const int pre = min(V, mis == 0 ? 0 : E - mis);
  for (int i = threadIdx.x; i < pre; i += kArgThreads) add(elem_at<T>(base, i), i);
  const int nvec = (V - pre) / E;
  const char* vb = reinterpret_cast<const char*>(base + pre);
  auto unpack = [&](const u32x4& x, float (&xs)[E]) __attribute__((always_inline)) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xs[2 * e] = bf16lo(w[e]);
        xs[2 * e + 1] = bf16hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[e] = __uint_as_float(w[e]);
    }
  };
  // Vectors: the largest number of each (NaN ignored) and the first vector
  // holding the thread's largest; the entry's index is recovered after the
  // scan from that one vector.
  float vv = -INFINITY;
  int vc = -1;
  constexpr int RV = U * kArgThreads;
  for (int r0 = 0; r0 < nvec; r0 += RV) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * kArgThreads + (int)threadIdx.x;
      x[u] = c < nvec ? ldg16_stream(vb + (int64_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = r0 + u * kArgThreads + (int)threadIdx.x;
      if (c >= nvec) continue;
      float xs[E];
      unpack(x[u], xs);
      float cm = xs[0];
#pragma unroll
      for (int e = 1; e < E; ++e) cm = fmaxf(cm, xs[e]);
      // a strict ">" keeps the first vector; the first vector holding a number
      // is taken even when that number is -inf
      const bool up = cm > vv || (vc < 0 && cm == cm);
      vv = up ? cm : vv;
      vc = up ? c : vc;
      const float ym = cm * kLog2e;
      if (ym > m) {
        s = m == -INFINITY ? 0.f : s * fast_exp2(m - ym);
        m = ym;
      }
      if (m != -INFINITY) {
        // a NaN entry turns s into NaN here
#pragma unroll
        for (int e = 0; e < E; ++e) s += fast_exp2(xs[e] * kLog2e - m);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) nanf = nanf || xs[e] != xs[e];
      }
    }
  }
  if (vc >= 0) {
    float xs[E];
    unpack(ldg16(vb + (int64_t)vc * 16), xs);
    int vi = pre + vc * E;
#pragma unroll
    for (int e = E - 1; e >= 0; --e) vi = xs[e] == vv ? pre + vc * E + e : vi;
    better(bv, bi, vv, vi);
  }
  for (int i = pre + nvec * E + threadIdx.x; i < V; i += kArgThreads) add(elem_at<T>(base, i), i);
  nanf = __any(nanf);

  auto merge = [&](float om, float os) {
    const float M = fmaxf(m, om);
    if (M == -INFINITY) return;
    s = (m == -INFINITY ? 0.f : s * fast_exp2(m - M)) + (om == -INFINITY ? 0.f : os * fast_exp2(om - M));
    m = M;
  };
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    better(bv, bi, ov, oi);
    const float om = __shfl_xor(m, o);
    const float os = __shfl_xor(s, o);
    merge(om, os);
  }
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    sv_[wave] = bv;
    si_[wave] = bi;
    sm_[wave] = m;
    ss_[wave] = s;
    sn_[wave] = nanf ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / kWave; ++w) {
      better(bv, bi, sv_[w], si_[w]);
      merge(sm_[w], ss_[w]);
      nanf = nanf || sn_[w] != 0;
    }
    // a row of NaN only: its first entry
    out[row] = bi == 0x7fffffff ? 0 : bi;
    lse[row] = nanf ? __builtin_nanf("") : (m + fast_log2(s)) * 0.69314718055994531f;
  }
}

constexpr int kAccThreads = 256;   // >= SPEC_MAX_NODES: one thread per node

__device__ __forceinline__ bool key_less(uint64_t ah, uint64_t al, uint64_t bh, uint64_t bl) {
  return ah < bh || (ah == bh && al < bl);
}

// LDS of one request's acceptance scan
struct AcceptSmem {
  int32_t link[SPEC_MAX_NODES];   // the node's parent if it is accepted, else INT_MIN
  int32_t gbon[SPEC_MAX_NODES];   // the greedy token of the node's own row (correction token)
  float row_lse[SPEC_MAX_NODES];
  int32_t path_s[SPEC_MAX_DEPTH];
  int red_i[kAccThreads / kWave];
  uint64_t red_h[kAccThreads / kWave];
  uint64_t red_l[kAccThreads / kWave];
};

// The acceptance scan (and, when enabled, the commit) of request b by one
// workgroup of kAccThreads threads, one per node.
__device__ __forceinline__ void accept_request(AcceptSmem& sm, int b, int T_, const int32_t* n_nodes,
                                               const int32_t* draft_tok, const int32_t* acc_parent,
                                               const int32_t* verify_row, const int32_t* argmax, int max_depth,
                                               int32_t* out_len, int32_t* out_path, int32_t* out_bonus,
                                               const AcceptRule& rule, const CommitArgs& commit) {
  const int v = threadIdx.x;
  const int wave = v / kWave;
  const int lane = v % kWave;
  // Every load that does not depend on another goes out first, in one round
  // trip: the node count, the cache length the commit appends at, and the
  // node's parent, draft and own row's greedy token (the acceptance test, or
  // the correction token should the node end the path).
  const int n = clampi(n_nodes[b], 0, T_);
  const int64_t len_in = commit.enabled ? commit.cache_len_in[b] : 0;
  int par_v = -1, x = -1, u = v, g_own = -1;
  if (v < T_) {
    par_v = acc_parent[(int64_t)b * T_ + v];
    x = draft_tok[(int64_t)b * T_ + v];
    if (verify_row) u = verify_row[(int64_t)b * T_ + v];
    if ((rule.mode == 0 && !verify_row) || out_bonus != nullptr) g_own = argmax[(int64_t)b * T_ + v];
  }
  // probability rules: every row's log-sum-exp is staged before the same
  // buffer receives the nodes' probabilities
  if (rule.mode != 0 && v < n) sm.row_lse[v] = rule.prob[(int64_t)b * T_ + v];
  __syncthreads();
  if (v < n) {
    sm.gbon[v] = g_own;
    // the row that verifies node v: v itself, or the given row (-1 = accepted
    // unchecked; a row outside [0, n) never accepts)
    const bool in_rows = u >= 0 && u < n;
    bool okv;
    if (rule.mode == 0) {
      const int g = verify_row ? (in_rows ? argmax[(int64_t)b * T_ + u] : -1) : g_own;
      okv = u == -1 || (in_rows && x == g);
    } else {
      // target probability of the draft at its row: exp(logit - lse)
      float p = u == -1 ? 1.f : 0.f;
      if (in_rows && x >= 0 && x < rule.V) {
        const int64_t at = ((int64_t)b * T_ + u) * rule.V + x;
        const float l = rule.logits_bf16 ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(rule.logits)[at]) << 16)
                                         : static_cast<const float*>(rule.logits)[at];
        p = fast_exp2((l - sm.row_lse[u]) * 1.4426950408889634f);
      }
      if (u == -1) okv = true;
      else if (!in_rows) okv = false;
      else if (rule.mode == 1) okv = p > rule.threshold;
      else okv = rule.uniform[(int64_t)b * T_ + v] * rule.draft_prob[(int64_t)b * T_ + v] < p;
      rule.prob[(int64_t)b * T_ + v] = p;
    }
    // a rejected node's link is INT_MIN, which ends a walk as a broken link does
    sm.link[v] = okv ? par_v : INT_MIN;
  }
  __syncthreads();

  // Walk to the root, one LDS read per level (the node's link).  The path's
  // nodes go into a 128-bit key, 8 bits each, shifted in from the top as the
  // walk climbs: when it ends at the root, the root is the top byte and the
  // walk's first node the lowest used one -- the root-first path, compared as
  // a number below.  Unused bytes are 0.
  int depth = 0;
  bool acc = false;
  uint64_t ph = 0ull, pl = 0ull;
  if (v < n) {
    int cur = v;
    bool good = true;
    while (cur >= 0) {
      const int l = sm.link[cur];
      if (depth >= max_depth || l < -1 || l >= cur) {   // rejected, or a broken link
        good = false;
        break;
      }
      pl = (pl >> 8) | (ph << 56);
      ph = (ph >> 8) | ((uint64_t)cur << 56);
      ++depth;
      cur = l;
    }
    acc = good;
  }

  // A = deepest accepted node
  uint32_t alw[1] = {(uint32_t)(acc ? depth : 0)};
  wave_allreduce<1>(alw, [](uint32_t (&x)[1], const uint32_t (&y)[1]) { x[0] = max(x[0], y[0]); });
  int a_len = (int)alw[0];
  if (lane == 0) sm.red_i[wave] = a_len;
  __syncthreads();
  a_len = 0;
  for (int w = 0; w < kAccThreads / kWave; ++w) a_len = max(a_len, sm.red_i[w]);

  // lexicographically smallest root-first path among accepted nodes of depth A
  uint64_t kh = ~0ull, kl = ~0ull;
  if (acc && depth == a_len && a_len > 0) {
    kh = ph;
    kl = pl;
  }
  uint32_t kw[4] = {(uint32_t)kh, (uint32_t)(kh >> 32), (uint32_t)kl, (uint32_t)(kl >> 32)};
  wave_allreduce<4>(kw, [](uint32_t (&x)[4], const uint32_t (&y)[4]) {
    const uint64_t xh = x[0] | ((uint64_t)x[1] << 32), xl = x[2] | ((uint64_t)x[3] << 32);
    const uint64_t yh = y[0] | ((uint64_t)y[1] << 32), yl = y[2] | ((uint64_t)y[3] << 32);
    if (key_less(yh, yl, xh, xl)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = y[q];
    }
  });
  kh = kw[0] | ((uint64_t)kw[1] << 32);
  kl = kw[2] | ((uint64_t)kw[3] << 32);
  if (lane == 0) {
    sm.red_h[wave] = kh;
    sm.red_l[wave] = kl;
  }
  __syncthreads();
  if (v == 0) {
    for (int w = 1; w < kAccThreads / kWave; ++w)
      if (key_less(sm.red_h[w], sm.red_l[w], kh, kl)) {
        kh = sm.red_h[w];
        kl = sm.red_l[w];
      }
    out_len[b] = a_len;
  }
  __syncthreads();
  if (v == 0) {
    sm.red_h[0] = kh;
    sm.red_l[0] = kl;
    if (out_bonus != nullptr) {
      // correction token: the greedy token of the last accepted node's row
      int bonus = -1;
      if (a_len > 0) {
        const int d = a_len - 1;
        const uint64_t w = d < 8 ? kh : kl;
        const int last = (int)((w >> (56 - 8 * (d & 7))) & 0xffull);
        bonus = sm.gbon[last];
      }
      out_bonus[b] = bonus;
    }
  }
  __syncthreads();
  if (v < max_depth) {
    int node = -1;
    if (v < a_len) {
      const uint64_t w = v < 8 ? sm.red_h[0] : sm.red_l[0];
      const int sh = 56 - 8 * (v & 7);
      node = (int)((w >> sh) & 0xffull);
    }
    out_path[(int64_t)b * max_depth + v] = node;
    sm.path_s[v] = node;
  }
  // fused form: append the accepted rows to the cache in the same launch
  if (commit.enabled) {
    __syncthreads();
    commit_rows(b, commit, a_len, sm.path_s, len_in);
  }
}

__global__ __launch_bounds__(kAccThreads) void k_accept(int T_, const int32_t* __restrict__ n_nodes,
                                                        const int32_t* __restrict__ draft_tok,
                                                        const int32_t* __restrict__ acc_parent,
                                                        const int32_t* __restrict__ verify_row,
                                                        const int32_t* __restrict__ argmax, int max_depth,
                                                        int32_t* __restrict__ out_len,
                                                        int32_t* __restrict__ out_path,
                                                        int32_t* __restrict__ out_bonus, AcceptRule rule,
                                                        CommitArgs commit) {
  __shared__ AcceptSmem sm;
  accept_request(sm, blockIdx.x, T_, n_nodes, draft_tok, acc_parent, verify_row, argmax, max_depth, out_len,
                 out_path, out_bonus, rule, commit);
}

hipError_t launch_argmax(const void* logits, int dtype, int B, int T, int V, const int32_t* n_nodes,
                         int32_t* out_argmax, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)B * T));
  // Rows of at most 128 KB are latency-bound (a workgroup streams one row):
  // 16 loads in flight per thread bring them in about one round trip.  Longer
  // rows are bandwidth-bound, where 8 measured faster.
  const bool short_row = (int64_t)V * (dtype == SPEC_F32 ? 4 : 2) <= (128 << 10);
  if (dtype == SPEC_F32) {
    const float* lg = static_cast<const float*>(logits);
    if (short_row)
      hipLaunchKernelGGL((k_argmax<float, 16>), grid, dim3(kArgThreads), 0, st, lg, T, V, n_nodes, out_argmax);
    else
      hipLaunchKernelGGL((k_argmax<float, 8>), grid, dim3(kArgThreads), 0, st, lg, T, V, n_nodes, out_argmax);
  } else {
    const uint16_t* lg = static_cast<const uint16_t*>(logits);
    if (short_row)
      hipLaunchKernelGGL((k_argmax<uint16_t, 16>), grid, dim3(kArgThreads), 0, st, lg, T, V, n_nodes, out_argmax);
    else
      hipLaunchKernelGGL((k_argmax<uint16_t, 8>), grid, dim3(kArgThreads), 0, st, lg, T, V, n_nodes, out_argmax);
  }
  return hipGetLastError();
}

hipError_t launch_argmax_lse(const void* logits, int dtype, int B, int T, int V, const int32_t* n_nodes,
                             int32_t* out_argmax, float* out_lse, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)B * T));
  if (dtype == SPEC_F32)
    hipLaunchKernelGGL(k_argmax_lse<float>, grid, dim3(kArgThreads), 0, st, static_cast<const float*>(logits), T,
                       V, n_nodes, out_argmax, out_lse);
  else
    hipLaunchKernelGGL(k_argmax_lse<uint16_t>, grid, dim3(kArgThreads), 0, st,
                       static_cast<const uint16_t*>(logits), T, V, n_nodes, out_argmax, out_lse);
  return hipGetLastError();
}

hipError_t launch_accept(int B, int T, const int32_t* n_nodes, const int32_t* draft_tok,
                         const int32_t* acc_parent, const int32_t* verify_row, const int32_t* argmax,
                         int max_depth, int32_t* out_len, int32_t* out_path, int32_t* out_bonus,
                         const AcceptRule& rule, const CommitArgs& commit, hipStream_t st) {
  hipLaunchKernelGGL(k_accept, dim3(B), dim3(kAccThreads), 0, st, T, n_nodes, draft_tok, acc_parent, verify_row,
                     argmax, max_depth, out_len, out_path, out_bonus, rule, commit);
  return hipGetLastError();
}

}  // namespace sv
