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
// Work layout
//   Rows of one (request, kv-head) are m = r * G + g (block row r, head g of
//   the group), so the G heads of a block row are adjacent and share its mask
//   word.  A workgroup owns 64 * NB rows and has 8 waves in two groups of 4;
//   wave w of a group owns NB blocks of 16 rows.  The two groups take
//   alternate 32-key tiles of the same key stream (a split of the keys inside
//   the workgroup) and merge their softmax states through LDS at the end.
//
// Schedule (ping-pong of the two groups)
//   A step of a group is a matrix half -- scores of its tile, P*V of its
//   previous tile -- then a barrier, then a softmax half.  Group 1 passes one
//   extra barrier before its first step, so it runs half a step behind group
//   0: while one group's waves feed the matrix cores the other group's waves
//   (on the same SIMDs) run their exponentials, and the two kinds of work
//   overlap without the compiler having to interleave them.  A wave raises
//   its issue priority for its softmax half, so its vector work is not held
//   behind the matrix wave's instruction stream.
//
// Key stream
//   Keys are the prefix range of this split, then -- last split only -- the S
//   soft keys and the block rows.  Segments are tiled separately, so prefix
//   tiles need no mask except the ragged tail.  Each group copies its own
//   tiles straight from HBM into rings of LDS slots (one for K, one for V) with
//   16-byte direct-to-LDS loads, three steps ahead of the compute (the first
//   three steps' loads go out before the setup loads); a wave issues its share
//   of a step's loads in its matrix half, after its fragment reads and before
//   its matrix instructions.  Row-major tiles (K, and V unless the cache keeps
//   V transposed) sit in a slot with 16-byte chunk c of key row k stored at
//   chunk position c ^ swz(k):
//     S^T = K Q^T : K is the A operand, one 16-byte read per lane;
//     O^T = V^T P^T : V^T is the A operand, built by the transposing 64-bit
//                     LDS read (lane j of a 16-lane group receives element
//                     j % 4 of the 8 bytes addressed by lane 4e + j / 4 of its
//                     group, for e = 0..3).
//   A cache whose V is stored in fragment-major 32-key tiles (SPEC_V_TILE32)
//   is copied to LDS as it is, and each lane reads its V^T operand with one
//   linear 16-byte read (soft and block tiles stay row-major).
//   With S^T and O^T every lane holds one query row (lane % 16) for all its
//   values: the row's 8 scores of a tile become the P operand directly (the
//   contraction order over keys is permuted the same way in V^T), and the
//   row's max and scale apply to its own O^T values.
//
// Softmax: the running max only moves when a tile's max exceeds it by more
// than 8 (in log2 units), so after the first tile rows are almost never
// rescaled; probabilities stay below 2^8, far from fp32 / bf16 limits.  The
// common path does not even compute the tile max: the probabilities against
// the current max are needed anyway, and their sum exceeds 2^8 whenever one of
// them could.  Whether a row rescales is decided by that row alone, so each
// query row's output is bitwise the same whatever the other rows of the
// workgroup are (their K/V, their masks, or whether they exist).
#include "attn_common.hpp"

namespace sv {

template <int D, int NB, bool VT>
__global__ __launch_bounds__(512) void k_attn_mfma(AttnArgs a) {
  using C = MfmaCfg<D, NB>;
  constexpr int DC = D / 32;   // k-chunks of S^T = K Q^T
  constexpr int DB = D / 16;   // 16-wide head-dim blocks of O^T
  __shared__ __attribute__((aligned(1024))) char ring[(C::NSK + C::NSV) * C::TILEB];
  __shared__ uint32_t mask_lds[C::ROWS * C::MAXW];   // row rl's word w at rl * W + w
  __shared__ uint32_t sp_lds[64];                      // the request's soft-prompt words

  // ---- which (split, request, kv-head, row chunk): siblings of a row chunk
  // sit on the same XCD (workgroups are dealt round-robin over 8 XCDs: XCD x
  // runs workgroups x, x + 8, ... in order, each on the first CU that frees)
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int tid = threadIdx.x;
  int chunk_id, split, b, h;
  if (a.balance) {
    // A grid of several rounds finishes when its last workgroup does: the
    // pairs go longest prefix first, pair of rank k to XCD k mod 8, so every
    // XCD gets a share of the long ones and ends on short ones.  The rank of
    // a request: the requests with a longer prefix, or as long and a lower
    // index, before it.  The lengths pass through the start of the ring, which
    // nothing loads into before the barrier that ends this.
    __shared__ int pick;
    const int q = bid / 8;
    const int k = (q / a.row_chunks) * 8 + bid % 8;   // the pair's rank
    chunk_id = q % a.row_chunks;
    split = 0;
    h = k % a.Hkv;
    const int r = k / a.Hkv;
    int* const lens = reinterpret_cast<int*>(ring);
    for (int j = tid; j < a.B; j += C::kThreads) lens[j] = (int)min<int64_t>(max(a.cache_len[j], 0), a.lmax);
    __syncthreads();
    for (int j = tid; j < a.B; j += C::kThreads) {
      const int lj = lens[j];
      int rk = 0;
      for (int i = 0; i < a.B; ++i) {
        const int li = lens[i];
        rk += (li > lj || (li == lj && i < j)) ? 1 : 0;
      }
      if (rk == r) pick = j;
    }
    __syncthreads();
    b = pick;
  } else {
    const int item = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
    chunk_id = item % a.row_chunks;
    const int rest = item / a.row_chunks;
    const int bh = rest % (a.B * a.Hkv);
    split = rest / (a.B * a.Hkv);
    b = bh / a.Hkv;
    h = bh % a.Hkv;
  }
  // uniform values in scalar registers: the request's scalars then come by
  // scalar loads, which no wait for the tile loads below has to cover
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  chunk_id = __builtin_amdgcn_readfirstlane(chunk_id);
  split = __builtin_amdgcn_readfirstlane(split);

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave >> 2;          // key-tile parity this wave computes
  const int wq = wave & 3;            // row slice within the workgroup
  const int lane = tid % kWave;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_char*)ring;
  // The request's prefix length and row count (n_q, or for multi-stream rows
  // the node count): scalar loads issued here, used after the setup loads.
  const bool msa = a.mask_mode == MASK_MSA;
  const int len_raw = a.cache_len[b];
  const int cnt = (msa ? a.n_nodes : a.n_q)[b];
  // ---- setup loads.  They need only the workgroup's request, kv-head and
  // rows, so they go out before the lengths are waited for.  Everything a wave needs before the first step comes
  // through the same direct-to-LDS path as the tiles, ahead of them, so that
  // no compiler-generated wait (which would count the tile loads too) stands
  // between the setup and the first step: the workgroup's query rows (staged
  // in V slots 4..7, which the tile stream first writes at step P/2), the mask
  // words of its rows and the request's soft-prompt words.  Rows past the end
  // or past the request's queries read an in-range row; the values are not used.
  // When the mask is built here (from the parent array, or from the node tree
  // of multi-stream rows), the parents and soft-prompt flags come instead, by
  // the same path (a flag byte lands as a zero-extended word), into a slot that
  // the tile stream first writes at step P/2; after the setup barrier each
  // thread walks one row's chain there (below).
  const bool tree = a.mask_mode != MASK_WORDS;
  const int nchain = msa ? a.msa_N : a.Tq;    // parents: one per tree node or block row
  char* const aux_l = ring + 6 * C::TILEB;                                               // K slot 6
  int32_t* const par_l = reinterpret_cast<int32_t*>(aux_l);                              // [nchain]
  uint32_t* const spf_l = reinterpret_cast<uint32_t*>(aux_l + SPEC_MAX_TQ * 4);            // [Tq]
  static_assert(SPEC_MAX_TQ * 8 <= C::TILEB, "parents and flags fit in one slot");
  static_assert(C::ROWS <= C::kThreads, "one workgroup row per thread");
  const bool has_flags = !msa && a.sp_flag != nullptr;
  const int row0 = chunk_id * C::ROWS;
  constexpr int QOPS = C::ROWS * D * 2 / 1024 / C::kWaves;   // 1 KB query loads per wave
  static_assert(QOPS >= 1 && QOPS * 1024 * C::kWaves == C::ROWS * D * 2, "query staging split");
  static_assert(C::ROWS * D * 2 <= 4 * C::TILEB, "query rows fit in V slots 4..7");
  const char* const qstage = ring + (C::NSK + 4) * C::TILEB;
  {
    // 16-byte chunk c of stage row rr sits at position c ^ (rr mod CH)
#pragma unroll
    for (int jq = 0; jq < QOPS; ++jq) {
      const int n = (wave * QOPS + jq) * 64 + lane;
      const int rr = n / C::CH, c = (n % C::CH) ^ (rr & (C::CH - 1));
      const int m = row0 + rr;
      const int r = min(m / a.G, a.Tq - 1), g = m % a.G;
      dma16(ring_lds + (C::NSK + 4) * C::TILEB + (wave * QOPS + jq) * 1024,
            static_cast<const char*>(a.q) + ((((int64_t)b * a.Tq + r) * a.Hq + h * a.G + g) * D + 8 * c) * 2);
    }
    if (tree) {
      // entries 64 k .. 64 k + 63 by wave k (thread r's entry comes with its own wave's
      // loads); lanes past the end repeat the last entry
      if (wave * 64 < nchain) {
        const int r = min(wave * 64 + lane, nchain - 1);
        const uint32_t aux = (uint32_t)(uintptr_t)(lds_char*)aux_l;   // par_l, then spf_l
        dma4(aux + wave * 256, a.attn_parent + (int64_t)b * nchain + r);
        if (has_flags) dma1(aux + SPEC_MAX_TQ * 4 + wave * 256, a.sp_flag + (int64_t)b * a.Tq + r);
      }
    } else {
      const uint32_t mask_addr = (uint32_t)(uintptr_t)(lds_char*)(char*)mask_lds;
      const int nmw = C::ROWS * a.W / 64;   // ROWS is a multiple of 64: whole wave loads
      for (int k = wave; k < nmw; k += C::kWaves) {
        const int n = k * 64 + lane;
        const int r = min((row0 + n / a.W) / a.G, a.Tq - 1);
        dma4(mask_addr + k * 256, a.mask_bits + ((int64_t)b * a.Tq + r) * a.W + n % a.W);
      }
      if (a.S > 0 && wave == C::kWaves - 1)
        dma4((uint32_t)(uintptr_t)(lds_char*)(char*)sp_lds, a.sp_bits + (int64_t)b * a.W + min(lane, a.W - 1));
    }
  }

  __builtin_amdgcn_sched_barrier(0);

  const int L = (int)min<int64_t>(max(len_raw, 0), a.lmax);
  // multi-stream rows: n nodes, each with its main row and gamma stream rows
  const int msa_n = msa ? clampi(cnt, 0, a.msa_N) : 0;
  const int nq = msa ? min(msa_n * (1 + a.msa_gamma), a.Tq) : clampi(cnt, 0, a.Tq);
  // split boundaries on 32-key multiples, so a split's prefix tiles are the cache's tiles
  const int keys_per_split = (((L + a.n_split - 1) / a.n_split) + C::TK - 1) / C::TK * C::TK;
  const int ks = min(L, split * keys_per_split);
  const int ke = min(L, ks + keys_per_split);
  const bool last = split == a.n_split - 1;
  const int ntp = (ke - ks + C::TK - 1) / C::TK;
  const int nts = last ? (a.S + C::TK - 1) / C::TK : 0;
  const int ntb = last ? (nq + C::TK - 1) / C::TK : 0;
  const int nt = ntp + nts + ntb;

  // ---- direct-to-LDS tile loads.  Group g's "step u loads" are what it reads
  // at step u: K of its tile 2u+g (scored at step u) and V of its tile 2u+g-2
  // (whose P*V runs at step u).  Waves 0..3 and 4..7 of the group split the K
  // and V streams, LPS 1 KB wave loads each.
  const char* kc = static_cast<const char*>(a.k_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * 2;
  const char* vc = static_cast<const char*>(a.v_cache) + ((int64_t)b * a.sb + (int64_t)h * a.sh) * 2;
  const char* kblk = static_cast<const char*>(a.k_blk) + ((int64_t)b * a.Tq * a.Hkv + h) * D * 2;
  const char* vblk = static_cast<const char*>(a.v_blk) + ((int64_t)b * a.Tq * a.Hkv + h) * D * 2;
  const char* ksoft = static_cast<const char*>(a.k_soft) + (int64_t)h * D * 2;
  const char* vsoft = static_cast<const char*>(a.v_soft) + (int64_t)h * D * 2;
  const int gw = wave & 3;                        // wave within its group
  const bool load_v = (gw * C::LPS) / C::LPT >= 1;   // first half of the group loads K, second V
  const int lrow = lane / C::CH;               // key row within the wave's 1 KB load
  const int lpos = lane % C::CH;               // chunk position the lane fills
  const char* const kring = ring;
  const char* const vring = ring + C::NSK * C::TILEB;
  int lane_row[C::LPS], lane_off[C::LPS], lane_dst[C::LPS];
#pragma unroll
  for (int j = 0; j < C::LPS; ++j) {
    const int ii = (gw * C::LPS + j) % C::LPT;
    lane_row[j] = ii * C::RPI + lrow;
    lane_off[j] = (lpos ^ C::swz(lane_row[j])) * 16;
    lane_dst[j] = ii * 1024;
  }
  // A transposed V tile (SPEC_V_TILE32) is stored fragment-major: 1 KB piece
  // db holds head dims 16 db .. +15, and its 16-byte chunk i is the P*V operand
  // of lane i -- head dim 16 db + i % 16, the 8 keys 4 g + (0..3) and
  // 16 + 4 g + (0..3) with g = i / 16, the keys the lane's score accumulators
  // hold.  The tile is copied to LDS as it is (lane i's 16 bytes of a wave load
  // land at byte 16 i, as the hardware places them), and the fragment read is
  // linear: 195 B/clk per CU measured, against 154 for the transposing read of
  // a row-major tile.
  const int lane_vt = lane * 16;
  // Rows past a segment's end are clamped to its last key and masked in the
  // compute.  A tile past the end still issues its loads (the last tile again,
  // into the slot that tile index maps to, which nothing reads): the waits
  // below count loads, and a wait for "all but the newest step's loads" only
  // covers an older step if the newer one really issued its share.  Tiles
  // before the start (V in the first two steps) issue nothing; a non-empty
  // step always follows them.
  struct TileSrc {
    const char* base;
    int stride, nvalid;
    uint32_t slot;
    bool on, vt;      // vt: a transposed V tile of the prefix (read whole, no row clamp)
  };
  auto tile_src = [&](int u) __attribute__((always_inline)) {
    TileSrc r;
    const int tslot = 2 * u + grp - (load_v ? 2 : 0);
    r.on = tslot >= 0;
    r.vt = false;
    const int t = min(max(tslot, 0), nt - 1);
    if (t < ntp) {
      r.vt = VT && load_v;
      const int key0 = ks + t * C::TK;
      r.base = (load_v ? vc : kc) + (int64_t)key0 * a.sl * 2;
      r.stride = (int)(a.sl * 2);
      r.nvalid = ke - key0;
    } else if (t < ntp + nts) {
      const int key0 = (t - ntp) * C::TK;
      r.base = (load_v ? vsoft : ksoft) + (int64_t)key0 * a.Hkv * D * 2;
      r.stride = a.Hkv * D * 2;
      r.nvalid = a.S - key0;
    } else {
      const int key0 = (t - ntp - nts) * C::TK;
      r.base = (load_v ? vblk : kblk) + (int64_t)key0 * a.Hkv * D * 2;
      r.stride = a.Hkv * D * 2;
      r.nvalid = nq - key0;
    }
    r.slot = ring_lds + (load_v ? (C::NSK + max(tslot, 0) % C::NSV) : (max(tslot, 0) % C::NSK)) * C::TILEB;
    return r;
  };
  auto issue_one = [&](const TileSrc& r, int j) __attribute__((always_inline)) {
    if (!r.on) return;
    const int rel = min(lane_row[j], r.nvalid - 1);
    dma16(r.slot + lane_dst[j], r.base + (r.vt ? lane_dst[j] + lane_vt : rel * r.stride + lane_off[j]));
  };
  auto issue_step = [&](int u) __attribute__((always_inline)) {
    const TileSrc r = tile_src(u);
#pragma unroll
    for (int j = 0; j < C::LPS; ++j) issue_one(r, j);
  };

  // The first steps' tiles follow; their HBM latency overlaps the setup's.
  if (nt > 0) {
#pragma unroll
    for (int u = 0; u < C::P / 2; ++u) issue_step(u);
  }
  // The wave's setup loads have landed once no more than its tile loads are in
  // flight (K loaders issued P/2 steps of them, V loaders P/2 - 1: their first
  // step has no tile); after the barrier below every wave's have.
  auto wait_setup = [&]() __attribute__((always_inline)) {
    if (nt == 0)
      wait_vmcnt<0>();
    else if (load_v)
      wait_vmcnt<(C::P / 2 - 1) * C::LPS>();
    else
      wait_vmcnt<(C::P / 2) * C::LPS>();
  };

  // ---- this lane's rows
  int row_r[NB], row_j[NB], row_l[NB];
  bool row_ok[NB], row_sp[NB];
  bf16x8 qf[NB][DC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    row_l[nb] = wq * (16 * NB) + 16 * nb + l16;
    const int m = row0 + row_l[nb];
    const int r = m / a.G, g = m % a.G;
    row_r[nb] = r;
    row_j[nb] = h * a.G + g;
    row_ok[nb] = (m < a.R) && (r < nq);
  }

  float mrun[NB], lrun[NB], negm[NB];
  f32x4 o[NB][DB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mrun[nb] = -INFINITY;   // running max, log2 units
    negm[nb] = 0.f;         // -max used for the exponent (0 while no key is visible)
    lrun[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[nb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int lx16 = ((lane ^ 16) << 2), lx32 = ((lane ^ 32) << 2);   // byte lane addresses for permutes

  wait_setup();
  block_barrier();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rr = row_l[nb];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int pos = (4 * dc + q4) ^ (rr & (C::CH - 1));
      u32x4 v = *reinterpret_cast<const u32x4*>(qstage + rr * C::ROWB + pos * 16);
      if (!row_ok[nb]) v = u32x4{0u, 0u, 0u, 0u};
      qf[nb][dc] = as_bf16x8(v);
    }
    const int r = row_r[nb];
    if (tree)
      row_sp[nb] = row_ok[nb] && a.S > 0 && has_flags && spf_l[min(r, a.Tq - 1)] != 0u;
    else
      row_sp[nb] = row_ok[nb] && a.S > 0 && ((sp_lds[min(r, a.Tq - 1) >> 5] >> (r & 31)) & 1u);
  }
  // ---- the block mask of the workgroup's rows from the parents (only the last
  // split has block tiles), one row per thread, while the first tiles are in
  // flight.  Row r sees block key c iff r < n_q and c is r or an ancestor of r
  // along parent links that point strictly upwards (the first link that does
  // not ends the chain).  Multi-stream rows: the chain runs over the tree
  // nodes from the row's node v, and stream j of v also sees streams 1..j of
  // v (rows n + v gamma .. + j - 1).  The walk of a chain of depth d takes d
  // dependent LDS reads; the bits go straight into the row's words in LDS.
  if (tree && last && tid < C::ROWS) {
    const int rl = tid;
    const int r = min((row0 + rl) / a.G, a.Tq - 1);
    uint32_t* const words = mask_lds + rl * a.W;   // this thread's row alone
    for (int w = 0; w < a.W; ++w) words[w] = 0u;
    // one LDS OR per key, issued without waiting: a chain step costs one
    // dependent LDS read
    auto set_bits = [&](int w, uint32_t bits) __attribute__((always_inline)) { atomicOr(words + w, bits); };
    if (r < nq) {
      int cur = r, j = 0;
      if (msa && r >= msa_n) {
        cur = (r - msa_n) / a.msa_gamma;
        j = (r - msa_n) % a.msa_gamma + 1;
      }
      const int node = cur;
      set_bits(cur >> 5, 1u << (cur & 31));
      for (int pr = par_l[cur]; pr >= 0 && pr < cur; pr = par_l[pr]) {
        set_bits(pr >> 5, 1u << (pr & 31));
        cur = pr;
      }
      if (j > 0) {   // streams 1..j of the node: rows s0 .. s0 + j - 1
        const int s0 = msa_n + node * a.msa_gamma;
        for (int w = s0 >> 5; w <= (s0 + j - 1) >> 5; ++w) {
          const int lo = max(s0, 32 * w), hi = min(s0 + j, 32 * w + 32);
          set_bits(w, (hi - lo == 32 ? ~0u : ((1u << (hi - lo)) - 1u)) << (lo - 32 * w));
        }
      }
    }
  }
  // the staged queries are overwritten by step P/2's V loads, issued only after
  // a barrier that every wave reaches after this; the mask words are read after
  // many barriers
  wait_lgkm0();

  const float P_LIMIT = 256.0f;   // 2^TAU with TAU = 8: bound on any probability between rescales
  if (nt > 0) {
    // Ping-pong of the two wave groups (group g owns tiles 2s+g).  Between any
    // two barriers one group runs its matrix half (scores of one tile, P*V of
    // its previous tile) while the other runs its softmax half, so each SIMD
    // holds one wave on the matrix cores and one on the vector ALUs.
    const int nsteps = (nt + 1) / 2;
    f32x4 st[NB][2];
    bf16x8 pf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      pf[nb] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) st[nb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // step s: wait for step s's loads, free the slots read at step s-1, refill
    auto begin_step = [&](int s) __attribute__((always_inline)) {
      wait_vmcnt<(C::P / 2 - 1) * C::LPS>();
      block_barrier();
    };
    // K fragments of tile t: key 16 kb + l16, head dims 32 dc + 8 q4 .. +7
    auto read_k = [&](int t, bf16x8 (&kf)[2][DC]) __attribute__((always_inline)) {
      const char* slotK = kring + (t % C::NSK) * C::TILEB;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 16 * kb + l16;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const int ch = (4 * dc + q4) ^ C::swz(row);
          kf[kb][dc] = as_bf16x8(*reinterpret_cast<const u32x4*>(slotK + row * C::ROWB + ch * 16));
        }
      }
    };
    // S^T = K Q^T + bias (bias -inf hides a key: the score is -inf, its
    // probability exactly 0, as with an additive -inf mask)
    auto scores_biased = [&](const bf16x8 (&kf)[2][DC], f32x4 (&sc)[NB][2], const f32x4 (&bias)[NB][2])
        __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x4 acc = bias[nb][kb];
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) acc = mfma16x16x32(kf[kb][dc], qf[nb][dc], acc);
          sc[nb][kb] = acc;
        }
    };
    // S^T = K Q^T
    auto scores = [&](const bf16x8 (&kf)[2][DC], f32x4 (&sc)[NB][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) acc = mfma16x16x32(kf[kb][dc], qf[nb][dc], acc);
          sc[nb][kb] = acc;
        }
    };
    // V^T fragments of tile tp: head dims 16 db + l16 and keys {4 q4 .. +3}
    // (read 0) and {16 + 4 q4 .. +3} (read 1)
    auto read_v = [&](int tp, bf16x8 (&vf)[DB]) __attribute__((always_inline)) {
      const char* slotV = vring + (tp % C::NSV) * C::TILEB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint32_t vw[4];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int row = 16 * cc + 4 * q4 + (l16 >> 2);
          const int ch = (2 * db + ((l16 & 3) >> 1)) ^ C::swz(row);
          lds_char* ptr = to_lds(slotV) + row * C::ROWB + ch * 16 + 8 * (l16 & 1);
          const bf16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)ptr);
          uint32_t w2[2];
          __builtin_memcpy(w2, &v4, 8);
          vw[2 * cc] = w2[0];
          vw[2 * cc + 1] = w2[1];
        }
        vf[db] = as_bf16x8(u32x4{vw[0], vw[1], vw[2], vw[3]});
      }
    };
    // V^T fragments of a transposed tile tp: one linear 16-byte read per head-dim block
    auto read_vt = [&](int tp, bf16x8 (&vf)[DB]) __attribute__((always_inline)) {
      const char* slotV = vring + (tp % C::NSV) * C::TILEB + lane * 16;
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[db] = as_bf16x8(*reinterpret_cast<const u32x4*>(slotV + db * 1024));
    };
    // zero the values of keys at or past lim (the ragged last tile of a
    // transposed prefix: cache slots past the length may hold anything, NaN
    // included, and a zero probability does not cancel a NaN in the product).
    // Element e of the lane's fragment is key 4 q4 + e (e < 4) or 16 + 4 q4 + e - 4.
    auto clip_vt = [&](bf16x8 (&vf)[DB], int lim) __attribute__((always_inline)) {
      const int nlo = clampi(lim - 4 * q4, 0, 4), nhi = clampi(lim - 16 - 4 * q4, 0, 4);
      u32x4 keep;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int n = w < 2 ? nlo : nhi, e = 2 * (w & 1);
        keep[w] = (e < n ? 0x0000ffffu : 0u) | (e + 1 < n ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4 v;
        __builtin_memcpy(&v, &vf[db], 16);
        v &= keep;
        vf[db] = as_bf16x8(v);
      }
    };
    // O^T += V^T P^T
    auto pv = [&](const bf16x8 (&vf)[DB]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb][db] = mfma16x16x32(vf[db], pf[nb], o[nb][db]);
    };
    auto pack = [&](int nb, const float (&p)[8]) __attribute__((always_inline)) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2_t v2;
        v2[0] = (__bf16)p[2 * e];
        v2[1] = (__bf16)p[2 * e + 1];
        pk[e] = __builtin_bit_cast(uint32_t, v2);
      }
      pf[nb] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    };
    // Rescale row block nb and recompute p.  The new reference is the max over
    // the lanes of the row that asked for it (need): a lane whose sum is within
    // the bound stays within it against any larger reference.  A row that asked
    // for nothing keeps its reference, so one row's arithmetic never depends on
    // the other rows of its wave (the call is wave-uniform, the decision is not).
    auto rescale = [&](int nb, const float (&xs)[8], float (&p)[8], float& ps, bool need) __attribute__((always_inline)) {
      const float lmax = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])),
                               fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
      float mx = need ? lmax * a.c : -INFINITY;
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(lx16, __float_as_int(mx))));
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_bpermute(lx32, __float_as_int(mx))));
      const float mnew = fmaxf(mrun[nb], mx);
      if (mnew != -INFINITY) {
        const float alpha = (mrun[nb] == -INFINITY) ? 0.f : fast_exp2(mrun[nb] - mnew);
        lrun[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[nb][db] *= alpha;
        mrun[nb] = mnew;
        negm[nb] = -mnew;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(xs[e], a.c, negm[nb]));
      ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    };
    // softmax of a complete prefix tile: no mask; probabilities against the current
    // max, whose sum exceeds 2^TAU whenever one of them could (then rescale exactly).
    // check_empty: a row with no reference yet (no visible key so far) takes one;
    // the hot steps pass false, as every row has one after its group's first tile.
    auto softmax_full = [&](bool check_empty) __attribute__((always_inline)) {
      float xs[NB][8], p[NB][8], ps[NB];
      bool need[NB], any_need = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[nb][e] = st[nb][e >> 2][e & 3];
          p[nb][e] = fast_exp2(fmaf(xs[nb][e], a.c, negm[nb]));
        }
        ps[nb] = ((p[nb][0] + p[nb][1]) + (p[nb][2] + p[nb][3])) + ((p[nb][4] + p[nb][5]) + (p[nb][6] + p[nb][7]));
        need[nb] = (check_empty && mrun[nb] == -INFINITY) || !(ps[nb] <= P_LIMIT);
        any_need = any_need || need[nb];
      }
      if (__builtin_expect(__any(any_need), 0)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) rescale(nb, xs[nb], p[nb], ps[nb], need[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        lrun[nb] += ps[nb];
        pack(nb, p[nb]);
      }
    };
    // visibility of the lane's 8 keys of a tile (bit e: slot e) for each of its
    // rows: ragged prefix tail (seg 0), soft prompt (seg 1), block rows (seg 2,
    // whose mask words the caller read: mw).  Keys below lim exist; slots e < 4
    // hold tile keys 4 q4 + e, slots e >= 4 keys 16 + 4 q4 + e - 4.
    auto visibility = [&](int seg, int lim, const uint32_t (&mw)[NB], uint32_t (&vis)[NB]) __attribute__((always_inline)) {
      const int nlo = clampi(lim - 4 * q4, 0, 4), nhi = clampi(lim - 16 - 4 * q4, 0, 4);
      const uint32_t in_tile = ((1u << nlo) - 1u) | (((1u << nhi) - 1u) << 4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (seg == 0)
          vis[nb] = row_ok[nb] ? 0xffu : 0u;
        else if (seg == 1)
          vis[nb] = row_sp[nb] ? 0xffu : 0u;
        else
          vis[nb] = ((mw[nb] >> (4 * q4)) & 0xfu) | (((mw[nb] >> (16 + 4 * q4)) & 0xfu) << 4);
        vis[nb] &= in_tile;
      }
    };
    // softmax of a tile that needs masking (the first step's tile).  A hidden
    // key's probability is its computed value with every bit cleared (+0
    // whatever the slot holds, NaN included); the masked scores (-inf where
    // hidden) are formed only when a rescale needs them.  One rescale branch
    // for all row blocks, as in softmax_full.
    auto softmax_masked = [&](int seg, int lim, const uint32_t (&mw)[NB]) __attribute__((always_inline)) {
      uint32_t vis[NB];
      visibility(seg, lim, mw, vis);
      float p[NB][8], ps[NB];
      bool need[NB], any_need = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t keep = (uint32_t)((int32_t)(vis[nb] << (31 - e)) >> 31);   // all ones or zero
          p[nb][e] = __uint_as_float(__float_as_uint(fast_exp2(fmaf(st[nb][e >> 2][e & 3], a.c, negm[nb]))) & keep);
        }
        ps[nb] = ((p[nb][0] + p[nb][1]) + (p[nb][2] + p[nb][3])) + ((p[nb][4] + p[nb][5]) + (p[nb][6] + p[nb][7]));
        need[nb] = !(ps[nb] <= P_LIMIT) || mrun[nb] == -INFINITY;
        any_need = any_need || need[nb];
      }
      if (__builtin_expect(__any(any_need), 0)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float xs[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[e] = ((vis[nb] >> e) & 1u) ? st[nb][e >> 2][e & 3] : -INFINITY;
          rescale(nb, xs, p[nb], ps[nb], need[nb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        lrun[nb] += ps[nb];
        pack(nb, p[nb]);
      }
      // keeps this tail distinct from softmax_full's: where a branch chooses
      // between the two, the compiler would otherwise merge the identical tails
      // behind a choice of array addresses, which puts the arrays in scratch
      __builtin_amdgcn_sched_barrier(0);
    };
    // the additive mask of a tile's scores: +0 for a key the lane's row sees,
    // -inf for one it does not
    auto mask_bias = [&](int seg, int lim, const uint32_t (&mw)[NB], f32x4 (&bias)[NB][2]) __attribute__((always_inline)) {
      uint32_t vis[NB];
      visibility(seg, lim, mw, vis);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 8; ++e) bias[nb][e >> 2][e & 3] = ((vis[nb] >> e) & 1u) ? 0.f : -INFINITY;
    };
    // softmax of a tile whose scores carry mask_bias: the unmasked arithmetic.
    // A hidden key's score is -inf, so its probability is 0, unless its K is
    // not finite: then the score is NaN, the tile's sum is NaN and the wave
    // takes the branch, which redoes the tile as softmax_masked does (hidden
    // keys selected out) -- so a hidden key's K never reaches a row, and every
    // row gets softmax_masked's results bit for bit.
    auto softmax_biased = [&](int seg, int lim, const uint32_t (&mw)[NB]) __attribute__((always_inline)) {
      float p[NB][8], ps[NB];
      bool need[NB], any_need = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[nb][e] = fast_exp2(fmaf(st[nb][e >> 2][e & 3], a.c, negm[nb]));
        ps[nb] = ((p[nb][0] + p[nb][1]) + (p[nb][2] + p[nb][3])) + ((p[nb][4] + p[nb][5]) + (p[nb][6] + p[nb][7]));
        need[nb] = mrun[nb] == -INFINITY || !(ps[nb] <= P_LIMIT);
        any_need = any_need || need[nb];
      }
      if (__builtin_expect(__any(any_need), 0)) {
        uint32_t vis[NB];
        visibility(seg, lim, mw, vis);
        float xs[NB][8];
        any_need = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xs[nb][e] = ((vis[nb] >> e) & 1u) ? st[nb][e >> 2][e & 3] : -INFINITY;
            p[nb][e] = fast_exp2(fmaf(xs[nb][e], a.c, negm[nb]));
          }
          ps[nb] = ((p[nb][0] + p[nb][1]) + (p[nb][2] + p[nb][3])) + ((p[nb][4] + p[nb][5]) + (p[nb][6] + p[nb][7]));
          need[nb] = !(ps[nb] <= P_LIMIT) || mrun[nb] == -INFINITY;
          any_need = any_need || need[nb];
        }
        if (__any(any_need)) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) rescale(nb, xs[nb], p[nb], ps[nb], need[nb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        lrun[nb] += ps[nb];
        pack(nb, p[nb]);
      }
      __builtin_amdgcn_sched_barrier(0);   // a tail of its own, as in softmax_masked
    };
    // segment and in-tile key count of tile t; the block rows' mask words of the lane's rows
    auto tile_kind = [&](int t, int& seg, int& lim) __attribute__((always_inline)) {
      seg = t < ntp ? 0 : (t < ntp + nts ? 1 : 2);
      if (seg == 0) lim = min(C::TK, ke - (ks + t * C::TK));
      else if (seg == 1) lim = min(C::TK, a.S - (t - ntp) * C::TK);
      else lim = min(C::TK, nq - (t - ntp - nts) * C::TK);
    };
    auto read_mask = [&](int t, int seg, uint32_t (&mw)[NB]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        mw[nb] = (seg == 2 && row_ok[nb]) ? mask_lds[row_l[nb] * a.W + (t - ntp - nts)] : 0u;
    };
    auto softmax_any = [&](int t) __attribute__((always_inline)) {
      int seg, lim;
      tile_kind(t, seg, lim);
      if (seg == 0 && lim == C::TK) {
        softmax_full(true);
      } else {
        uint32_t mw[NB];
        read_mask(t, seg, mw);
        softmax_masked(seg, lim, mw);
      }
    };
    // Step s of a group: its matrix half (scores of its tile 2s+g, P*V of its
    // tile 2s+g-2), a barrier, its softmax half (of tile 2s+g).  Every wave runs
    // the same sequence; group 1 passes one extra barrier first, so it runs half
    // a step behind group 0 and the two groups' halves interleave.
    auto matrix_half = [&](int s) __attribute__((always_inline)) {
      const int t = 2 * s + grp;
      if (t < nt) {
        bf16x8 kf[2][DC];
        read_k(t, kf);
        scores(kf, st);
      }
      if (s >= 1 && t - 2 < nt) {
        const int tp = t - 2;
        bf16x8 vf[DB];
        if (VT && tp < ntp) {
          read_vt(tp, vf);
          const int lim = ke - (ks + tp * C::TK);
          if (lim < C::TK) clip_vt(vf, lim);
        } else {
          read_v(tp, vf);
        }
        pv(vf);
      }
    };
    auto generic_step = [&](int s) __attribute__((always_inline)) {
      begin_step(s);
      matrix_half(s);
      block_barrier();
      issue_step(s + C::P / 2);
      if (2 * s + grp < nt) softmax_any(2 * s + grp);
    };
    // own tiles 2s+g (scored and softmaxed) and 2s+g-2 (in P*V) are full prefix
    // tiles and 2s+g is not the group's first: no masks, no branches
    // the matrix instructions of a hot step in issue order: scores (nb, kb, dc),
    // then P*V (db, nb); mat_part issues those with index in [LO, HI)
    auto mat_part = [&](const bf16x8 (&kf)[2][DC], const bf16x8 (&vf)[DB], auto LO, auto HI)
        __attribute__((always_inline)) {
      constexpr int lo = decltype(LO)::value, hi = decltype(HI)::value;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            const int idx = (nb * 2 + kb) * DC + dc;
            if (idx >= lo && idx < hi)
              st[nb][kb] = mfma16x16x32(kf[kb][dc], qf[nb][dc], dc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : st[nb][kb]);
          }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int idx = NB * 2 * DC + db * NB + nb;
          if (idx >= lo && idx < hi) o[nb][db] = mfma16x16x32(vf[db], pf[nb], o[nb][db]);
        }
    };
    auto hot_step = [&](int s) __attribute__((always_inline)) {
      begin_step(s);
      const TileSrc src = tile_src(s + C::P / 2);
      // every fragment read goes out before the first matrix instruction, so
      // the LDS latency is paid once per half; the step's loads follow (issued
      // here they measured a little faster than spread through the softmax half)
      bf16x8 kf[2][DC], vf[DB];
      read_k(2 * s + grp, kf);
      if constexpr (VT)
        read_vt(2 * s + grp - 2, vf);
      else
        read_v(2 * s + grp - 2, vf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < C::LPS; ++j) issue_one(src, j);
      // The barrier that hands the matrix cores to the other group goes after
      // the first 12 of the step's 32 matrix instructions (pinned: the matrix
      // instructions touch no memory, so the compiler would move them across
      // it freely).  The rest then overlap the other group's fragment reads.
      // Measured on the headline workload against other positions (0..32) and
      // against the compiler's own placement, which varies with the code
      // around it: 12 was fastest (78 us against 82-103).
      constexpr int kMat = NB * 2 * DC + DB * NB;
      constexpr int kAt = 12 < kMat ? 12 : kMat;
      mat_part(kf, vf, std::integral_constant<int, 0>{}, std::integral_constant<int, kAt>{});
      __builtin_amdgcn_sched_barrier(0);
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mat_part(kf, vf, std::integral_constant<int, kAt>{}, std::integral_constant<int, kMat>{});
      // the softmax half takes issue priority over the other group's wave on
      // the same SIMD, whose matrix instructions keep the matrix core busy
      // meanwhile (measured 4-12% faster than equal priority or a raised
      // priority for the matrix instructions)
      __builtin_amdgcn_s_setprio(1);
      softmax_full(false);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    };
    // A step after the hot ones (its own tile, if any, is a ragged prefix, soft
    // or block tile; its P*V tile may be too).  K fragments first, then the
    // step's loads, the scores and the hand-off barrier; the V fragments are
    // read only once the K fragments are dead (both at once would overflow the
    // registers here), then P*V and the softmax.
    bool skip_prev = false;   // the group's previous tile was skipped (no P*V for it)
    auto tail_step = [&](int s) __attribute__((always_inline)) {
      begin_step(s);
      const TileSrc src = tile_src(s + C::P / 2);
      const int t = 2 * s + grp, tp = t - 2;   // s >= 1: tp >= 0
      const bool has_t = t < nt, has_p = tp < nt;
      auto read_pv = [&](bf16x8 (&vf)[DB]) __attribute__((always_inline)) {
        if (VT && tp < ntp) {
          read_vt(tp, vf);
          const int plim = ke - (ks + tp * C::TK);
          if (plim < C::TK) clip_vt(vf, plim);
        } else {
          read_v(tp, vf);
        }
      };
      // The mask enters as the scores' initial accumulator, built before the
      // hand-off while the K fragments arrive, so the softmax half -- the
      // longer one in these steps -- runs the unmasked softmax.
      int seg = 0, lim = 0;
      uint32_t mw[NB];
      bool skip = false;
      if (has_t) {   // then has_p as well
        tile_kind(t, seg, lim);
        read_mask(t, seg, mw);
        if (seg == 2) {
          uint32_t seen = 0;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) seen |= mw[nb];
          skip = !__any(seen != 0u);
        }
      }
      if (has_t && !skip) {
        bf16x8 kf[2][DC];
        read_k(t, kf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < C::LPS; ++j) issue_one(src, j);
        f32x4 bias[NB][2];
        mask_bias(seg, lim, mw, bias);
        scores_biased(kf, st, bias);
      } else {
#pragma unroll
        for (int j = 0; j < C::LPS; ++j) issue_one(src, j);
      }
      __builtin_amdgcn_sched_barrier(0);
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (has_p && !skip_prev) {
        bf16x8 vf[DB];
        read_pv(vf);
        pv(vf);
      }
      if (has_t && !skip) {
        __builtin_amdgcn_s_setprio(1);
        softmax_biased(seg, lim, mw);
        __builtin_amdgcn_s_setprio(0);
      }
      skip_prev = skip;
    };
    const int nfull = (ke - ks) / C::TK;
    const int s_hot_end = (nfull - grp + 1) / 2;   // steps whose own tile is a full prefix tile
    // A wave none of whose rows exists (past the kv-head's rows, or past the
    // request's queries) only loads its share of the tiles and keeps the
    // barriers: its SIMD and the LDS are then free for the other waves.  Its
    // rows' accumulators stay zero, which is what the epilogue writes for them.
    bool has_row = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) has_row = has_row || row_ok[nb];
    const bool idle = !__any(has_row);
    if (grp == 1) block_barrier();
    if (idle) {
      for (int s = 0; s <= nsteps; ++s) {
        begin_step(s);
        issue_step(s + C::P / 2);
        block_barrier();
      }
    } else {
      generic_step(0);
      for (int s = 1; s < s_hot_end; ++s) hot_step(s);
      for (int s = max(1, s_hot_end); s <= nsteps; ++s) tail_step(s);
    }
    if (grp == 0) block_barrier();
    __builtin_amdgcn_s_waitcnt(0);
  }
  block_barrier();

  // ---- merge the two wave groups (same rows, alternate tiles) through LDS
  static_assert((4 * NB * DB * 64 * 4 + 4 * NB * 64 * 2) * 4 <= (C::NSK + C::NSV) * C::TILEB,
                "merge scratch must fit in the ring");
  float* xo = reinterpret_cast<float*>(ring);               // [wq][nb][db][lane][4]
  float* xm = xo + 4 * NB * DB * 64 * 4;                    // [wq][nb][lane][2]
  if (grp == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(xo + (((wq * NB + nb) * DB + db) * 64 + lane) * 4) = o[nb][db];
      xm[((wq * NB + nb) * 64 + lane) * 2 + 0] = mrun[nb];
      xm[((wq * NB + nb) * 64 + lane) * 2 + 1] = lrun[nb];
    }
    // the barrier below does not wait for memory operations: publish the stores
    wait_lgkm0();
  }
  block_barrier();
  if (grp == 1) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float m1 = xm[((wq * NB + nb) * 64 + lane) * 2 + 0];
    const float l1 = xm[((wq * NB + nb) * 64 + lane) * 2 + 1];
    const float m0 = mrun[nb];
    const float M = fmaxf(m0, m1);
    const float a0 = (m0 == -INFINITY) ? 0.f : fast_exp2(m0 - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - M);
    lrun[nb] = a0 * lrun[nb] + a1 * l1;
    mrun[nb] = M;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + (((wq * NB + nb) * DB + db) * 64 + lane) * 4);
      o[nb][db] = o[nb][db] * a0 + o1 * a1;
    }
  }

  // ---- epilogue: lane holds O^T[d = 16 db + 4 q4 + i][row l16]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float lsum = lrun[nb];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int m = row0 + row_l[nb];
    if (m >= a.R) continue;
    const int r = row_r[nb];
    if (a.n_split == 1) {
      const int64_t orow = ((int64_t)b * a.Tq + r) * a.Hq + row_j[nb];
      const float inv = row_ok[nb] ? 1.f / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = o[nb][db] * inv;
        const int64_t at = orow * D + 16 * db + 4 * q4;
        if (a.out_bf16) {   // rounded to nearest even, 8 bytes per lane
          typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
          bf16x4v w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)v[i];
          *reinterpret_cast<bf16x4v*>(static_cast<__bf16*>(a.out) + at) = w;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + at) = v;
        }
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

hipError_t launch_attn_mfma(const AttnArgs& args, hipStream_t st) {
  const int64_t nwg = (int64_t)args.n_split * args.row_chunks * args.B * args.Hkv;
  const dim3 grid((unsigned)nwg);
  // longest-first dealing once the grid takes more than one round of
  // workgroups (256 CUs; two 64-row head-dim-64 workgroups fit in one CU)
  AttnArgs a = args;
  const int per_cu = a.D == 64 ? 2 : 1;
  a.balance = a.n_split == 1 && (int64_t)a.B * a.Hkv % 8 == 0 && a.B <= 4096 && nwg > 256 * per_cu;
  const dim3 block(512);
  auto go = [&](auto vt) -> hipError_t {
    constexpr bool VT = decltype(vt)::value;
    // 128-row workgroups run at D = 128 only (the plan gives D = 64 64-row workgroups)
    if (a.rows_per_wg == 128) {
      if (a.D != 128) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_attn_mfma<128, 2, VT>), grid, block, 0, st, a);
    } else {
      if (a.D == 128) hipLaunchKernelGGL((k_attn_mfma<128, 1, VT>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((k_attn_mfma<64, 1, VT>), grid, block, 0, st, a);
    }
    return hipGetLastError();
  };
  return a.v_tiled ? go(std::true_type{}) : go(std::false_type{});
}

}  // namespace sv
