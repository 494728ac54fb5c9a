// Masked verification attention on the vector ALUs.
//
// Used for fp32 inputs (bf16 inputs always run on the matrix cores).
//
// Math ("Speculative Streaming", Equation 1): out = softmax(q k^T * scale) v
// over the keys the row sees -- the soft prompt if its sp bit is set (ConFu
// key design 1), every cached prefix key, and the block keys whose mask bit
// is set.  Scores are kept in the log2 domain (scale * log2 e folded in) and
// reduced with an online softmax (running max and sum), accumulated in fp32.
//
// Work decomposition: one workgroup (4 waves) per (split, request, kv-head).
// Each wave walks its own 64-key tiles with its own softmax state; the four
// states are merged through LDS at the end.  Within a tile:
//   scores:  lane = key; the lane reads its key row straight from global
//            memory (16-byte loads) and the rows' queries from LDS (broadcast).
//   P * V:   lane = (key group of 4, 1/16 of the head dim); the probabilities
//            are passed between lanes with cross-lane permutes, and every V
//            row is read with 16 lanes x contiguous loads.
// Rows are processed in groups of 8; a group re-streams the keys (only the
// large fp32 correctness workloads have more than one group).
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kValuThreads = 256;
constexpr int kValuWaves = kValuThreads / kWave;
constexpr int kRG = 8;        // rows per group
constexpr int kTK = 64;       // keys per wave tile
constexpr int kMaxWords = (SPEC_MAX_TQ + 31) / 32;

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kSize = 4;
  __device__ static float get(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  // 8 consecutive elements
  __device__ static void load8(const void* p, float* x) {
    const u32x4 a = ldg16(p);
    const u32x4 b = ldg16(static_cast<const char*>(p) + 16);
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  }
  __device__ static void load4(const void* p, float* x) {
    const u32x4 a = ldg16(p);
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
  }
};
// Where the key with index t of this workgroup's key list lives.
// List = prefix [ks, ke) ++ soft [0, ns) ++ block rows [0, nbk).
struct KeyList {
  int np, ns, nbk;
  __device__ int total() const { return np + ns + nbk; }
};

template <typename T, int D>
__global__ __launch_bounds__(kValuThreads) void k_attn_valu(AttnArgs a) {
  constexpr int VE = D / 16;   // head-dim elements per lane in P*V
  constexpr int ES = Elem<T>::kSize;
  __shared__ float qs[kRG][D];
  __shared__ int row_ok[kRG];
  __shared__ int row_sp[kRG];
  __shared__ uint32_t row_mw[kRG][kMaxWords];
  __shared__ float wm[kValuWaves][kRG];
  __shared__ float wl[kValuWaves][kRG];
  __shared__ float wo[kValuWaves][kRG][D];

  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv;
  const int h = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  const int L = (int)min<int64_t>(max(a.cache_len[b], 0), a.lmax);
  const int nq = clampi(a.n_q[b], 0, a.Tq);
  const int chunk = (L + a.n_split - 1) / a.n_split;
  const int ks = min(L, split * chunk);
  const int ke = min(L, ks + chunk);
  const bool last = split == a.n_split - 1;
  KeyList kl;
  kl.np = ke - ks;
  kl.ns = last ? a.S : 0;
  kl.nbk = last ? nq : 0;
  const int nkeys = kl.total();
  const int ntiles = (nkeys + kTK - 1) / kTK;

  const char* kc = static_cast<const char*>(a.k_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * ES;
  const char* vc = static_cast<const char*>(a.v_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * ES;
  auto key_ptr = [&](int t, bool is_v) -> const char* {
    if (t < kl.np) return (is_v ? vc : kc) + (int64_t)(ks + t) * a.sl * ES;
    t -= kl.np;
    if (t < kl.ns)
      return static_cast<const char*>(is_v ? a.v_soft : a.k_soft) + ((int64_t)t * a.Hkv + h) * D * ES;
    t -= kl.ns;
    return static_cast<const char*>(is_v ? a.v_blk : a.k_blk) +
           (((int64_t)b * a.Tq + t) * a.Hkv + h) * D * ES;
  };

  for (int rg0 = 0; rg0 < a.R; rg0 += kRG) {
    __syncthreads();
    for (int idx = tid; idx < kRG * D; idx += kValuThreads) {
      const int i = idx / D, d = idx % D;
      const int m = rg0 + i;
      const int r = m / a.G, g = m % a.G;
      float x = 0.f;
      if (m < a.R && r < nq)
        x = Elem<T>::get(a.q, (((int64_t)b * a.Tq + r) * a.Hq + (int64_t)h * a.G + g) * D + d);
      qs[i][d] = x;
    }
    if (tid < kRG) {
      const int m = rg0 + tid;
      const int r = m / a.G;
      const bool ok = m < a.R && r < nq;
      row_ok[tid] = ok;
      row_sp[tid] = (ok && a.S > 0) ? (int)((a.sp_bits[(int64_t)b * a.W + (r >> 5)] >> (r & 31)) & 1u) : 0;
    }
    for (int idx = tid; idx < kRG * a.W; idx += kValuThreads) {
      const int i = idx / a.W, w = idx % a.W;
      const int m = rg0 + i;
      const int r = m / a.G;
      row_mw[i][w] = (m < a.R && r < nq) ? a.mask_bits[((int64_t)b * a.Tq + r) * a.W + w] : 0u;
    }
    __syncthreads();

    float mrow[kRG], lrow[kRG], o[kRG][VE];
#pragma unroll
    for (int i = 0; i < kRG; ++i) {
      mrow[i] = -INFINITY;
      lrow[i] = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) o[i][e] = 0.f;
    }

    for (int tile = wave; tile < ntiles; tile += kValuWaves) {
      // ---- scores: lane = key
      const int t = tile * kTK + lane;
      const bool kvalid = t < nkeys;
      float s[kRG];
#pragma unroll
      for (int i = 0; i < kRG; ++i) s[i] = 0.f;
      if (kvalid) {
        const char* kp = key_ptr(t, false);
#pragma unroll 2
        for (int d0 = 0; d0 < D; d0 += 8) {
          float kx[8];
          Elem<T>::load8(kp + d0 * ES, kx);
#pragma unroll
          for (int i = 0; i < kRG; ++i) {
            const float4 qa = *reinterpret_cast<const float4*>(&qs[i][d0]);
            const float4 qb = *reinterpret_cast<const float4*>(&qs[i][d0 + 4]);
            s[i] = fmaf(qa.x, kx[0], s[i]); s[i] = fmaf(qa.y, kx[1], s[i]);
            s[i] = fmaf(qa.z, kx[2], s[i]); s[i] = fmaf(qa.w, kx[3], s[i]);
            s[i] = fmaf(qb.x, kx[4], s[i]); s[i] = fmaf(qb.y, kx[5], s[i]);
            s[i] = fmaf(qb.z, kx[6], s[i]); s[i] = fmaf(qb.w, kx[7], s[i]);
          }
        }
      }
      // visibility of this lane's key for each row
      float p[kRG];
#pragma unroll
      for (int i = 0; i < kRG; ++i) {
        bool vis = false;
        if (kvalid) {
          if (t < kl.np) {
            vis = row_ok[i] != 0;
          } else if (t < kl.np + kl.ns) {
            vis = row_sp[i] != 0;
          } else {
            const int c = t - kl.np - kl.ns;
            vis = ((row_mw[i][c >> 5] >> (c & 31)) & 1u) != 0;
          }
        }
        const float x = vis ? s[i] * a.c : -INFINITY;
        const float mx = wave_max(x);
        const float mnew = fmaxf(mrow[i], mx);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrow[i] - muse);
        p[i] = fast_exp2(x - muse);
        lrow[i] = lrow[i] * alpha + p[i];
        mrow[i] = mnew;
#pragma unroll
        for (int e = 0; e < VE; ++e) o[i][e] *= alpha;
      }
      // ---- P * V: lane = (key group, head-dim slice)
      const int kg = lane >> 4;
      const int dl = lane & 15;
#pragma unroll 4
      for (int u = 0; u < kTK / 4; ++u) {
        const int j = 4 * u + kg;
        const int tv = tile * kTK + j;
        float vx[VE];
        if (tv < nkeys) {
          const char* vp = key_ptr(tv, true) + dl * VE * ES;
          if constexpr (VE == 8) Elem<T>::load8(vp, vx); else Elem<T>::load4(vp, vx);
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) vx[e] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < kRG; ++i) {
          const float pj = __shfl(p[i], j);
#pragma unroll
          for (int e = 0; e < VE; ++e) o[i][e] = fmaf(pj, vx[e], o[i][e]);
        }
      }
    }

    // ---- merge: lanes of a wave, then the four waves
#pragma unroll
    for (int i = 0; i < kRG; ++i) {
      lrow[i] = wave_sum(lrow[i]);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        o[i][e] += __shfl_xor(o[i][e], 16);
        o[i][e] += __shfl_xor(o[i][e], 32);
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < kRG; ++i)
#pragma unroll
        for (int e = 0; e < VE; ++e) wo[wave][i][lane * VE + e] = o[i][e];
    }
    if (lane < kRG) {
      // every lane holds all rows' values; lane i stores row i
      float mv = 0.f, lv = 0.f;
#pragma unroll
      for (int i = 0; i < kRG; ++i)
        if (lane == i) { mv = mrow[i]; lv = lrow[i]; }
      wm[wave][lane] = mv;
      wl[wave][lane] = lv;
    }
    __syncthreads();
    for (int idx = tid; idx < kRG * D; idx += kValuThreads) {
      const int i = idx / D, d = idx % D;
      const int m = rg0 + i;
      if (m >= a.R) continue;
      const int r = m / a.G, g = m % a.G;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kValuWaves; ++w) M = fmaxf(M, wm[w][i]);
      float lsum = 0.f, osum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kValuWaves; ++w) {
          const float wt = fast_exp2(wm[w][i] - M);
          lsum += wt * wl[w][i];
          osum += wt * wo[w][i][d];
        }
      }
      if (a.n_split == 1) {
        if (r < a.Tq) {
          const int64_t orow = ((int64_t)b * a.Tq + r) * a.Hq + (int64_t)h * a.G + g;
          const bool ok = row_ok[i] != 0;
          static_cast<float*>(a.out)[orow * D + d] = ok ? osum / lsum : 0.f;   // fp32 inputs: fp32 out
          if (d == 0 && a.lse != nullptr)
            a.lse[orow] = ok ? (M + fast_log2(lsum)) * 0.69314718055994531f : -INFINITY;
        }
      } else {
        const int64_t prow = (((int64_t)split * a.B + b) * a.Hkv + h) * a.R + m;
        a.part_o[prow * D + d] = osum;
        if (d == 0) {
          a.part_ml[prow * 2 + 0] = M;
          a.part_ml[prow * 2 + 1] = lsum;
        }
      }
    }
  }
}

// Log-sum-exp merge of split-KV partials: out = sum_s w_s O_s / sum_s w_s l_s,
// w_s = 2^(m_s - max_s m_s).  One thread per (row, 4 head-dim elements).
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  const int DQ = a.D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nrows = (int64_t)a.B * a.Hkv * a.R;
  if (idx >= nrows * DQ) return;
  const int64_t row = idx / DQ;
  const int dq = (int)(idx % DQ);
  const int m = (int)(row % a.R);
  const int h = (int)((row / a.R) % a.Hkv);
  const int b = (int)(row / ((int64_t)a.R * a.Hkv));
  const int r = m / a.G, g = m % a.G;
  if (r >= a.Tq) return;
  // rows of the request (multi-stream rows built in the attention: n_nodes * (1 + gamma))
  const int nq = a.mask_mode == MASK_MSA ? min(clampi(a.n_nodes[b], 0, a.msa_N) * (1 + a.msa_gamma), a.Tq)
                                         : clampi(a.n_q[b], 0, a.Tq);
  const int64_t orow = ((int64_t)b * a.Tq + r) * a.Hq + (int64_t)h * a.G + g;
  float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = -INFINITY;
  if (r < nq) {
    const int64_t stride = (int64_t)a.B * a.Hkv * a.R;
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.part_ml[(s * stride + row) * 2]);
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
      for (int s = 0; s < a.n_split; ++s) {
        const int64_t pr = s * stride + row;
        const float wt = fast_exp2(a.part_ml[pr * 2] - M);
        lsum += wt * a.part_ml[pr * 2 + 1];
        const float4 ov = *reinterpret_cast<const float4*>(a.part_o + pr * a.D + dq * 4);
        acc.x += wt * ov.x; acc.y += wt * ov.y; acc.z += wt * ov.z; acc.w += wt * ov.w;
      }
      const float inv = 1.f / lsum;
      res = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      lse = (M + fast_log2(lsum)) * 0.69314718055994531f;
    }
  }
  if (a.out_bf16) {   // rounded to nearest even
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    bf16x4v w;
    w[0] = (__bf16)res.x;
    w[1] = (__bf16)res.y;
    w[2] = (__bf16)res.z;
    w[3] = (__bf16)res.w;
    *reinterpret_cast<bf16x4v*>(static_cast<__bf16*>(a.out) + orow * a.D + dq * 4) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * a.D + dq * 4) = res;
  }
  if (dq == 0 && a.lse != nullptr) a.lse[orow] = lse;
}

hipError_t launch_attn_valu(const AttnArgs& a, int dtype, hipStream_t st) {
  const dim3 grid(a.n_split, a.B * a.Hkv);
  const dim3 block(kValuThreads);
  if (dtype != SPEC_F32) return hipErrorInvalidValue;   // the planner sends bf16 to the MFMA kernel
  if (a.D == 128) hipLaunchKernelGGL((k_attn_valu<float, 128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_attn_valu<float, 64>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.R * (a.D / 4);
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
