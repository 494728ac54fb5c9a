// Masked verification attention on the bf16 matrix cores (gfx950 MFMA).
//
// Used when a kv-head's query rows -- the GQA group of query heads times the
// speculative block rows, (Hq/Hkv) * Tq -- fill 16-row MFMA tiles: ConFu's
// tree + contemplate rows, large trees, multi-candidate streams.
//
// Math ("Speculative Streaming", Equation 1, masked per its Equation 4 prose
// and ConFu key design 1): out = softmax(q k^T * scale) v over the soft keys
// (rows with the sp bit), the cached prefix (all valid rows) and the block
// keys whose mask bit is set.  Online softmax in the log2 domain, fp32
// accumulation, probabilities rounded to bf16 for the P*V product.
//
// Layout of the work.  Rows of one (request, kv-head) are m = r * G + g
// (block row r, head g of the group), so the G heads of one block row are
// adjacent and share its mask word.  A workgroup of 4 waves owns 64 * NB
// rows; wave w owns NB blocks of 16 rows.  Keys stream in 32-key tiles that
// the whole workgroup stages in LDS (double-buffered, one barrier per tile):
//   K tile row-major [key][d]  -> A operand of S^T = K Q^T
//   V tile transposed [d][key] -> A operand of O^T = V^T P^T
// With S^T and O^T every lane holds one query row (lane % 16) for all its
// values: the row's 8 scores of a tile become the B operand of the P*V MFMA
// directly (the contraction order over keys is permuted identically in V^T),
// and the row's running max / scale apply to its own O^T values.  Only the
// max needs a cross-lane step (the row's 32 keys sit in 4 lanes).
//
// Key list of a workgroup: prefix keys [ks, ke) of its split, then -- for
// the last split only -- the S soft keys and the block rows.  Segments are
// tiled separately, so prefix tiles carry no mask (only the ragged tail is
// cut); soft and block tiles test the sp bit and the row's mask word.
#include "device_common.hpp"
#include "internal.hpp"

namespace sv {

constexpr int kMfmaThreads = 256;
constexpr int kTileK = 32;

template <int D>
struct MfmaLds {
  static constexpr int kKStride = D * 2 + 16;        // bytes per K row (padded)
  static constexpr int kVtStride = kTileK * 2 + 4;   // bytes per transposed V row (one head dim)
  static constexpr int kKBytes = kTileK * kKStride;
  static constexpr int kVtBytes = D * kVtStride;
  static constexpr int kBufBytes = kKBytes + kVtBytes;
  static constexpr int kChunks = kTileK * D / 8;     // 16-byte chunks per K (or V) tile
  static constexpr int kChunksPerThread = (kChunks + kMfmaThreads - 1) / kMfmaThreads;
};

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int D, int NB>
__global__ __launch_bounds__(kMfmaThreads) void k_attn_mfma(AttnArgs a) {
  using Lds = MfmaLds<D>;
  constexpr int DC = D / 32;   // k-chunks of S^T = K Q^T
  constexpr int DB = D / 16;   // 16-wide head-dim blocks of O^T
  constexpr int CPT = Lds::kChunksPerThread;
  __shared__ __attribute__((aligned(16))) char lds[2 * Lds::kBufBytes];

  const int split = blockIdx.x;
  const int chunk_id = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / a.Hkv;
  const int h = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  const int L = (int)min<int64_t>(max(a.cache_len[b], 0), a.lmax);
  const int nq = clampi(a.n_q[b], 0, a.Tq);
  const int keys_per_split = (L + a.n_split - 1) / a.n_split;
  const int ks = min(L, split * keys_per_split);
  const int ke = min(L, ks + keys_per_split);
  const bool last = split == a.n_split - 1;
  const int ntp = (ke - ks + kTileK - 1) / kTileK;
  const int nts = last ? (a.S + kTileK - 1) / kTileK : 0;
  const int ntb = last ? (nq + kTileK - 1) / kTileK : 0;
  const int nt = ntp + nts + ntb;

  // ---- this lane's rows: block nb covers rows rowbase + 16 nb + (0..15)
  const int rowbase = chunk_id * (64 * NB) + wave * (16 * NB);
  int row_r[NB], row_j[NB];
  bool row_ok[NB], row_sp[NB];
  bf16x8 qf[NB][DC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = rowbase + 16 * nb + l16;
    const int r = m / a.G, g = m % a.G;
    row_r[nb] = r;
    row_j[nb] = h * a.G + g;
    row_ok[nb] = (m < a.R) && (r < nq);
    row_sp[nb] = row_ok[nb] && a.S > 0 && ((a.sp_bits[(int64_t)b * a.W + (r >> 5)] >> (r & 31)) & 1u);
    const char* qp = static_cast<const char*>(a.q) +
                     ((((int64_t)b * a.Tq + r) * a.Hq + row_j[nb]) * D + 8 * q4) * 2;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok[nb]) v = ldg16(qp + dc * 64);
      qf[nb][dc] = as_bf16x8(v);
    }
  }

  // ---- tile loader: global -> registers -> LDS
  const char* kc = static_cast<const char*>(a.k_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * 2;
  const char* vc = static_cast<const char*>(a.v_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * 2;
  const char* ksoft = static_cast<const char*>(a.k_soft);
  const char* vsoft = static_cast<const char*>(a.v_soft);
  const char* kblk = static_cast<const char*>(a.k_blk) + ((int64_t)b * a.Tq * a.Hkv + h) * D * 2;
  const char* vblk = static_cast<const char*>(a.v_blk) + ((int64_t)b * a.Tq * a.Hkv + h) * D * 2;

  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int ti) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * kMfmaThreads;
      const int kk = c / (D / 8);
      const int d0 = 8 * (c % (D / 8));
      kreg[u] = u32x4{0u, 0u, 0u, 0u};
      vreg[u] = u32x4{0u, 0u, 0u, 0u};
      if (c >= Lds::kChunks) continue;
      if (ti < ntp) {
        const int key = ks + ti * kTileK + kk;
        if (key < ke) {
          const int64_t off = ((int64_t)key * a.sl + d0) * 2;
          kreg[u] = ldg16(kc + off);
          vreg[u] = ldg16(vc + off);
        }
      } else if (ti < ntp + nts) {
        const int key = (ti - ntp) * kTileK + kk;
        if (key < a.S) {
          const int64_t off = (((int64_t)key * a.Hkv + h) * D + d0) * 2;
          kreg[u] = ldg16(ksoft + off);
          vreg[u] = ldg16(vsoft + off);
        }
      } else {
        const int key = (ti - ntp - nts) * kTileK + kk;
        if (key < nq) {
          const int64_t off = ((int64_t)key * a.Hkv * D + d0) * 2;
          kreg[u] = ldg16(kblk + off);
          vreg[u] = ldg16(vblk + off);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = lds + buf * Lds::kBufBytes;
    char* vt = kb + Lds::kKBytes;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * kMfmaThreads;
      if (c >= Lds::kChunks) continue;
      const int kk = c / (D / 8);
      const int d0 = 8 * (c % (D / 8));
      *reinterpret_cast<u32x4*>(kb + kk * Lds::kKStride + d0 * 2) = kreg[u];
      const uint32_t w[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t x = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
        *reinterpret_cast<uint16_t*>(vt + (d0 + e) * Lds::kVtStride + kk * 2) = x;
      }
    }
  };

  float mrun[NB], lrun[NB];
  f32x4 o[NB][DB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mrun[nb] = -INFINITY;
    lrun[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[nb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int ti = 0; ti < nt; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < nt) load_tile(ti + 1);
    const char* kb = lds + buf * Lds::kBufBytes;
    const char* vt = kb + Lds::kKBytes;

    // K fragments: key = 16 kb + l16, head dims 32 dc + 8 q4 .. +7
    bf16x8 kf[2][DC];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kf[kb2][dc] = as_bf16x8(
            *reinterpret_cast<const u32x4*>(kb + (16 * kb2 + l16) * Lds::kKStride + (32 * dc + 8 * q4) * 2));

    // segment of this tile and its masking rule (uniform over the workgroup)
    const int seg = ti < ntp ? 0 : (ti < ntp + nts ? 1 : 2);
    int lim = kTileK;                  // keys of the tile that exist
    if (seg == 0) lim = min(kTileK, ke - (ks + ti * kTileK));
    else if (seg == 1) lim = min(kTileK, a.S - (ti - ntp) * kTileK);
    else lim = min(kTileK, nq - (ti - ntp - nts) * kTileK);

    bf16x8 pf[NB];
    float alpha[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 st[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) acc = mfma16x16x32(kf[kb2][dc], qf[nb][dc], acc);
        st[kb2] = acc;
      }
      // visibility of the lane's 8 keys (tile keys 16 kb + 4 q4 + i) for its row
      uint32_t vis = 0xffu;
      if (seg == 0) {
        if (lim < kTileK) {
          vis = 0u;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kb2 + 4 * q4 + i < lim) vis |= 1u << (4 * kb2 + i);
        }
        if (!row_ok[nb]) vis = 0u;
      } else if (seg == 1) {
        vis = 0u;
        if (row_sp[nb]) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kb2 + 4 * q4 + i < lim) vis |= 1u << (4 * kb2 + i);
        }
      } else {
        const int word = ti - ntp - nts;
        const uint32_t mw =
            row_ok[nb] ? a.mask_bits[((int64_t)b * a.Tq + row_r[nb]) * a.W + word] : 0u;
        vis = 0u;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((mw >> (16 * kb2 + 4 * q4 + i)) & 1u) vis |= 1u << (4 * kb2 + i);
      }
      float x[8];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[4 * kb2 + i] = ((vis >> (4 * kb2 + i)) & 1u) ? st[kb2][i] * a.c : -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[nb], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      alpha[nb] = fast_exp2(mrun[nb] - muse);
      mrun[nb] = mnew;
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(x[e] - muse);
        ps += p[e];
      }
      lrun[nb] = lrun[nb] * alpha[nb] + ps;
      const u32x4 packed = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      pf[nb] = as_bf16x8(packed);
    }

    // O^T += V^T P^T ; V^T fragment: head dim 16 db + l16, keys {4 q4 .. +3} and {16 + 4 q4 .. +3}
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const char* vrow = vt + (16 * db + l16) * Lds::kVtStride + 8 * q4;
      const u32x4 vv = {*reinterpret_cast<const uint32_t*>(vrow), *reinterpret_cast<const uint32_t*>(vrow + 4),
                        *reinterpret_cast<const uint32_t*>(vrow + 32), *reinterpret_cast<const uint32_t*>(vrow + 36)};
      const bf16x8 vf = as_bf16x8(vv);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 ov = o[nb][db];
        ov *= alpha[nb];
        o[nb][db] = mfma16x16x32(vf, pf[nb], ov);
      }
    }

    if (ti + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[d = 16 db + 4 q4 + i][row l16]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float lsum = lrun[nb];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int m = rowbase + 16 * nb + l16;
    if (m >= a.R) continue;
    const int r = row_r[nb];
    if (a.n_split == 1) {
      const int64_t orow = ((int64_t)b * a.Tq + r) * a.Hq + row_j[nb];
      const float inv = row_ok[nb] ? 1.f / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = o[nb][db] * inv;
        *reinterpret_cast<f32x4*>(a.out + orow * D + 16 * db + 4 * q4) = v;
      }
      if (q4 == 0 && a.lse != nullptr)
        a.lse[orow] = row_ok[nb] ? (mrun[nb] + fast_log2(lsum)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t prow = (((int64_t)split * a.B + b) * a.Hkv + h) * a.R + m;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(a.part_o + prow * D + 16 * db + 4 * q4) = o[nb][db];
      if (q4 == 0) {
        a.part_ml[prow * 2 + 0] = mrun[nb];
        a.part_ml[prow * 2 + 1] = lsum;
      }
    }
  }
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st) {
  const int rows_per_wg = a.rows_per_wg;
  const dim3 grid(a.n_split, a.row_chunks, a.B * a.Hkv);
  const dim3 block(kMfmaThreads);
  if (rows_per_wg == 128) {
    if (a.D == 128) hipLaunchKernelGGL((k_attn_mfma<128, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn_mfma<64, 2>), grid, block, 0, st, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((k_attn_mfma<128, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn_mfma<64, 1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
