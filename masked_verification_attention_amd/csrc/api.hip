// C ABI of the verification step: argument validation, scheduling, launch.
//
// Every check here runs on the host before anything is enqueued, so a
// rejected call leaves the stream untouched.  The checks make no HIP call
// and do not touch device memory: they are exercised without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "internal.hpp"

// Device scratch of spec_verify_attn_noalloc (split-KV partials), one copy per
// GPU for the life of the process.  In host code `scratch` is only a symbol
// handle: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return SPEC_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SPEC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int esize_of(int dtype) { return dtype == SPEC_F32 ? 4 : 2; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Descriptor checks shared by spec_verify_attn, its workspace query and spec_commit_kv.
int check_desc(const spec_attn_desc* d) {
  REQUIRE(d != nullptr, SPEC_EINVAL, "descriptor is NULL");
  REQUIRE(d->B >= 0, SPEC_EINVAL, "B = %d < 0", d->B);
  REQUIRE(d->Tq >= 1 && d->Tq <= SPEC_MAX_TQ, SPEC_EINVAL, "Tq = %d outside [1, %d]", d->Tq, SPEC_MAX_TQ);
  REQUIRE(d->Hq >= 1 && d->Hkv >= 1, SPEC_EINVAL, "Hq = %d, Hkv = %d must be >= 1", d->Hq, d->Hkv);
  REQUIRE(d->Hq % d->Hkv == 0, SPEC_EINVAL, "Hq = %d is not a multiple of Hkv = %d", d->Hq, d->Hkv);
  REQUIRE(d->dtype == SPEC_F32 || d->dtype == SPEC_BF16, SPEC_EINVAL, "dtype = %d is not a spec_dtype",
          d->dtype);
  REQUIRE(d->D == 64 || d->D == 128, SPEC_EUNSUPPORTED, "D = %d (supported: 64, 128)", d->D);
  REQUIRE(d->S >= 0 && d->S <= SPEC_MAX_SOFT, SPEC_EINVAL, "S = %d outside [0, %d]", d->S, SPEC_MAX_SOFT);
  REQUIRE(d->lmax >= 0 && d->lmax < (int64_t(1) << 31), SPEC_EINVAL, "lmax = %lld outside [0, 2^31)",
          (long long)d->lmax);
  REQUIRE(d->kv_stride_b > 0 && d->kv_stride_l > 0 && d->kv_stride_h > 0, SPEC_EINVAL,
          "cache strides must be positive");
  const int64_t es = esize_of(d->dtype);
  REQUIRE((d->kv_stride_b * es) % 16 == 0 && (d->kv_stride_l * es) % 16 == 0 && (d->kv_stride_h * es) % 16 == 0,
          SPEC_EINVAL, "cache strides must be multiples of 16 bytes");
  REQUIRE(d->kv_stride_h >= d->D || d->Hkv == 1, SPEC_EINVAL, "kv_stride_h < D would overlap heads");
  REQUIRE(d->kv_stride_l * es <= (int64_t(1) << 25), SPEC_EUNSUPPORTED,
          "kv_stride_l of %lld elements exceeds 32 MiB per cache row", (long long)d->kv_stride_l);
  REQUIRE(d->kv_splits >= 0 && d->kv_splits <= 64, SPEC_EINVAL, "kv_splits = %d outside [0, 64]", d->kv_splits);
  REQUIRE(d->v_layout == SPEC_V_ROWS || d->v_layout == SPEC_V_TILE32, SPEC_EINVAL,
          "v_layout = %d is not a spec_v_layout", d->v_layout);
  if (d->v_layout == SPEC_V_TILE32) {
    REQUIRE(d->dtype == SPEC_BF16, SPEC_EUNSUPPORTED, "v_layout SPEC_V_TILE32 needs bf16");
    REQUIRE(d->kv_stride_l == d->D, SPEC_EINVAL,
            "v_layout SPEC_V_TILE32 needs a head-major cache (kv_stride_l == D), got kv_stride_l = %lld",
            (long long)d->kv_stride_l);
    REQUIRE(d->lmax % 32 == 0, SPEC_EINVAL, "v_layout SPEC_V_TILE32 needs lmax %% 32 == 0, got lmax = %lld",
            (long long)d->lmax);
  }
  REQUIRE(isfinite(d->scale) && d->scale >= 0.f, SPEC_EINVAL, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  REQUIRE(d->out_dtype == SPEC_F32 || d->out_dtype == SPEC_BF16, SPEC_EINVAL, "out_dtype = %d is not a spec_dtype",
          d->out_dtype);
  REQUIRE(d->out_dtype == SPEC_F32 || d->dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
          "out_dtype SPEC_BF16 needs bf16 inputs");
  REQUIRE((int64_t)d->B * d->Hkv <= 65535, SPEC_EUNSUPPORTED, "B * Hkv = %lld exceeds 65535",
          (long long)((int64_t)d->B * d->Hkv));
  return SPEC_OK;
}

}  // namespace

namespace sv {

AttnPlan plan_attn(const spec_attn_desc& d) {
  AttnPlan p{};
  const int G = d.Hq / d.Hkv;
  const int R = G * d.Tq;
  const int64_t items_bh = (int64_t)d.B * d.Hkv;
  const int kCUs = 256;
  // bf16 always runs on the matrix cores: even a block of 8 rows per kv-head,
  // padded to 16-row tiles, streams the cache ~3x faster than the VALU kernel
  if (d.dtype == SPEC_BF16) {
    p.path = PATH_MFMA;
    // 128-row workgroups share each K/V tile between more rows, but at head
    // dim 64 the 64-row workgroup (half the LDS ring, under 128 registers a
    // lane) lets two workgroups share a CU, which measured faster
    p.rows_per_wg = (R > 64 && d.D == 128) ? 128 : 64;
    p.row_chunks = (R + p.rows_per_wg - 1) / p.rows_per_wg;
    const int64_t items = items_bh * p.row_chunks;
    int n = 1;
    if (d.kv_splits > 0) {
      n = d.kv_splits;
    } else if (items < kCUs) {
      // fill the chip, but keep at least 512 prefix keys per split
      n = (int)((kCUs + items - 1) / items);
      const int cap = (int)(d.lmax / 512 > 0 ? d.lmax / 512 : 1);
      n = n < cap ? n : cap;
    }
    p.n_split = n < 1 ? 1 : n;
  } else {
    p.path = PATH_VALU;
    p.rows_per_wg = 0;
    p.row_chunks = 1;
    int n = 1;
    if (d.kv_splits > 0) {
      n = d.kv_splits;
    } else {
      // ~512 prefix keys per workgroup: balances ragged prefixes, small partials
      n = (int)((d.lmax + 511) / 512);
      if (n < 1) n = 1;
      if (n > 16) n = 16;
    }
    p.n_split = n;
  }
  if (p.n_split > 1) {
    const size_t rows = (size_t)p.n_split * d.B * d.Hkv * R;
    p.ws_bytes = rows * d.D * sizeof(float) + rows * 2 * sizeof(float) + 256;
  }
  return p;
}

}  // namespace sv

namespace {

int argmax_accept_impl(const char* fn, const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                       const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                       const int32_t* verify_row, int32_t max_depth, int32_t* out_argmax, int32_t* out_len,
                       int32_t* out_path, int32_t* out_bonus, void* stream) {
  REQUIRE(B >= 0, SPEC_EINVAL, "%s: B = %d < 0", fn, B);
  REQUIRE(T >= 1 && T <= SPEC_MAX_NODES, SPEC_EINVAL, "%s: T = %d outside [1, %d]", fn, T, SPEC_MAX_NODES);
  REQUIRE(V >= 1, SPEC_EINVAL, "%s: V = %d < 1", fn, V);
  REQUIRE(max_depth >= 1 && max_depth <= SPEC_MAX_DEPTH, SPEC_EINVAL, "%s: max_depth = %d outside [1, %d]", fn,
          max_depth, SPEC_MAX_DEPTH);
  REQUIRE(logits_dtype == SPEC_F32 || logits_dtype == SPEC_BF16, SPEC_EINVAL,
          "%s: logits_dtype = %d is not a spec_dtype", fn, logits_dtype);
  REQUIRE((int64_t)B * T <= 0x7fffffff, SPEC_EUNSUPPORTED, "%s: B * T too large", fn);
  if (B == 0) return ok();
  REQUIRE(logits && n_nodes && draft_tok && acc_parent && out_argmax && out_len && out_path, SPEC_EINVAL,
          "%s: logits, n_nodes, draft_tok, acc_parent and the outputs argmax, len, path must be non-NULL", fn);
  REQUIRE(aligned(logits, esize_of(logits_dtype)), SPEC_EINVAL, "%s: logits must be aligned to its element size",
          fn);
  REQUIRE(aligned(n_nodes, 4) && aligned(draft_tok, 4) && aligned(acc_parent, 4) && aligned(verify_row, 4) &&
              aligned(out_argmax, 4) && aligned(out_len, 4) && aligned(out_path, 4) && aligned(out_bonus, 4),
          SPEC_EINVAL, "%s: int32 arrays must be 4-byte aligned", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sv::launch_argmax(logits, logits_dtype, B, T, V, n_nodes, out_argmax, s);
  if (e != hipSuccess) return hip_status(e, "argmax launch");
  sv::AcceptRule greedy{};
  sv::CommitArgs no_commit{};
  e = sv::launch_accept(B, T, n_nodes, draft_tok, acc_parent, verify_row, out_argmax, max_depth, out_len,
                        out_path, out_bonus, greedy, no_commit, s);
  return hip_status(e, "acceptance scan launch");
}

}  // namespace

extern "C" {

const char* spec_version(void) { return "0.2.0"; }

const char* spec_last_error(void) { return g_last_error; }

const char* spec_strerror(int status) {
  switch (status) {
    case SPEC_OK: return "success";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EUNSUPPORTED: return "unsupported configuration";
    case SPEC_EWORKSPACE: return "workspace missing or too small";
    case SPEC_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int spec_build_mask(const int32_t* attn_parent, const uint8_t* sp_flag, const int32_t* n_q, int32_t B,
                    int32_t Tq, uint32_t* mask_bits, uint32_t* sp_bits, void* stream) {
  REQUIRE(B >= 0, SPEC_EINVAL, "B = %d < 0", B);
  REQUIRE(Tq >= 1 && Tq <= SPEC_MAX_TQ, SPEC_EINVAL, "Tq = %d outside [1, %d]", Tq, SPEC_MAX_TQ);
  if (B == 0) return ok();
  REQUIRE(attn_parent && n_q && mask_bits && sp_bits, SPEC_EINVAL,
          "attn_parent, n_q, mask_bits and sp_bits must be non-NULL");
  REQUIRE(aligned(attn_parent, 4) && aligned(n_q, 4) && aligned(mask_bits, 4) && aligned(sp_bits, 4),
          SPEC_EINVAL, "int32/uint32 arrays must be 4-byte aligned");
  return hip_status(sv::launch_build_mask(attn_parent, sp_flag, n_q, B, Tq, mask_bits, sp_bits,
                                          static_cast<hipStream_t>(stream)),
                    "spec_build_mask launch");
}

int spec_build_msa_mask(const int32_t* tree_parent, const int32_t* n_nodes, int32_t B, int32_t N,
                        int32_t gamma, int32_t Tq, uint32_t* mask_bits, uint32_t* sp_bits, int32_t* n_q,
                        void* stream) {
  REQUIRE(B >= 0, SPEC_EINVAL, "B = %d < 0", B);
  REQUIRE(gamma >= 0 && gamma < SPEC_MAX_TQ, SPEC_EINVAL, "gamma = %d outside [0, %d)", gamma, SPEC_MAX_TQ);
  REQUIRE(N >= 1 && N <= SPEC_MAX_TQ, SPEC_EINVAL, "N = %d outside [1, %d]", N, SPEC_MAX_TQ);
  REQUIRE(Tq >= 1 && Tq <= SPEC_MAX_TQ, SPEC_EINVAL, "Tq = %d outside [1, %d]", Tq, SPEC_MAX_TQ);
  REQUIRE((int64_t)N * (1 + gamma) <= Tq, SPEC_EINVAL, "N * (1 + gamma) = %lld rows exceed Tq = %d",
          (long long)N * (1 + gamma), Tq);
  if (B == 0) return ok();
  REQUIRE(tree_parent && n_nodes && mask_bits && sp_bits && n_q, SPEC_EINVAL,
          "tree_parent, n_nodes, mask_bits, sp_bits and n_q must be non-NULL");
  REQUIRE(aligned(tree_parent, 4) && aligned(n_nodes, 4) && aligned(mask_bits, 4) && aligned(sp_bits, 4) &&
              aligned(n_q, 4),
          SPEC_EINVAL, "int32/uint32 arrays must be 4-byte aligned");
  return hip_status(sv::launch_build_msa_mask(tree_parent, n_nodes, B, N, gamma, Tq, mask_bits, sp_bits, n_q,
                                              static_cast<hipStream_t>(stream)),
                    "spec_build_msa_mask launch");
}

int spec_draft_tree(const void* logits, int32_t logits_dtype, int32_t B, int32_t R, int32_t V,
                    const int32_t* n_nodes, const int32_t* acc_len, const int32_t* acc_path, int32_t max_depth,
                    const int32_t* root_tok, int32_t gamma, int32_t k, int32_t* out_topk, int32_t* draft_tok,
                    int32_t* tree_parent, int32_t* n_out, void* stream) {
  REQUIRE(B >= 0, SPEC_EINVAL, "B = %d < 0", B);
  REQUIRE(R >= 1 && R <= SPEC_MAX_TQ, SPEC_EINVAL, "R = %d outside [1, %d]", R, SPEC_MAX_TQ);
  REQUIRE(k >= 1 && k <= SPEC_MAX_TOPK, SPEC_EINVAL, "k = %d outside [1, %d]", k, SPEC_MAX_TOPK);
  REQUIRE(gamma >= 0 && gamma < SPEC_MAX_TQ, SPEC_EINVAL, "gamma = %d outside [0, %d)", gamma, SPEC_MAX_TQ);
  REQUIRE(V >= k, SPEC_EINVAL, "V = %d < k = %d", V, k);
  REQUIRE(max_depth >= 1 && max_depth <= SPEC_MAX_DEPTH, SPEC_EINVAL, "max_depth = %d outside [1, %d]", max_depth,
          SPEC_MAX_DEPTH);
  REQUIRE(logits_dtype == SPEC_F32 || logits_dtype == SPEC_BF16, SPEC_EINVAL, "logits_dtype = %d is not a spec_dtype",
          logits_dtype);
  int64_t N = 1, level = 1;
  for (int g = 1; g <= gamma && N <= SPEC_MAX_TQ; ++g) {
    level *= k;
    N += level;
  }
  REQUIRE(N <= SPEC_MAX_TQ, SPEC_EINVAL, "a %d-ary tree of depth %d has more than %d nodes", k, gamma, SPEC_MAX_TQ);
  REQUIRE((int64_t)B * gamma <= 0x7fffffff && (int64_t)B * R <= 0x7fffffff, SPEC_EUNSUPPORTED, "B too large");
  if (B == 0) return ok();
  REQUIRE(logits && n_nodes && acc_len && acc_path && root_tok && draft_tok && tree_parent && n_out &&
              (out_topk || gamma == 0),
          SPEC_EINVAL, "logits, n_nodes, acc_len, acc_path, root_tok, out_topk, draft_tok, tree_parent and n_out "
          "must be non-NULL");
  REQUIRE(aligned(logits, esize_of(logits_dtype)), SPEC_EINVAL, "logits must be aligned to its element size");
  REQUIRE(aligned(n_nodes, 4) && aligned(acc_len, 4) && aligned(acc_path, 4) && aligned(root_tok, 4) &&
              aligned(out_topk, 4) && aligned(draft_tok, 4) && aligned(tree_parent, 4) && aligned(n_out, 4),
          SPEC_EINVAL, "int32 arrays must be 4-byte aligned");
  return hip_status(sv::launch_draft_tree(logits, logits_dtype, B, R, V, n_nodes, acc_len, acc_path, max_depth,
                                          root_tok, gamma, k, (int)N, out_topk, draft_tok, tree_parent, n_out,
                                          static_cast<hipStream_t>(stream)),
                    "spec_draft_tree launch");
}

int spec_prob_accept(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                     const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                     const int32_t* verify_row, int32_t max_depth, int32_t mode, float threshold,
                     const float* draft_prob, const float* uniform, int32_t* out_argmax, float* out_prob,
                     int32_t* out_len, int32_t* out_path, int32_t* out_bonus, void* stream) {
  REQUIRE(B >= 0, SPEC_EINVAL, "B = %d < 0", B);
  REQUIRE(T >= 1 && T <= SPEC_MAX_NODES, SPEC_EINVAL, "T = %d outside [1, %d]", T, SPEC_MAX_NODES);
  REQUIRE(V >= 1, SPEC_EINVAL, "V = %d < 1", V);
  REQUIRE(max_depth >= 1 && max_depth <= SPEC_MAX_DEPTH, SPEC_EINVAL, "max_depth = %d outside [1, %d]", max_depth,
          SPEC_MAX_DEPTH);
  REQUIRE(logits_dtype == SPEC_F32 || logits_dtype == SPEC_BF16, SPEC_EINVAL, "logits_dtype = %d is not a spec_dtype",
          logits_dtype);
  REQUIRE(mode == SPEC_ACCEPT_THRESHOLD || mode == SPEC_ACCEPT_SOFT, SPEC_EINVAL,
          "mode = %d (SPEC_ACCEPT_THRESHOLD or SPEC_ACCEPT_SOFT)", mode);
  REQUIRE(mode != SPEC_ACCEPT_THRESHOLD || (isfinite(threshold) && threshold >= 0.f), SPEC_EINVAL,
          "threshold must be finite and >= 0");
  REQUIRE((int64_t)B * T <= 0x7fffffff && (int64_t)B * T * V < (int64_t(1) << 46), SPEC_EUNSUPPORTED,
          "B * T * V too large");
  if (B == 0) return ok();
  REQUIRE(logits && n_nodes && draft_tok && acc_parent && out_argmax && out_prob && out_len && out_path, SPEC_EINVAL,
          "logits, n_nodes, draft_tok, acc_parent and the outputs argmax, prob, len, path must be non-NULL");
  REQUIRE(mode != SPEC_ACCEPT_SOFT || (draft_prob && uniform), SPEC_EINVAL,
          "soft matching needs draft_prob and uniform");
  REQUIRE(aligned(logits, esize_of(logits_dtype)), SPEC_EINVAL, "logits must be aligned to its element size");
  REQUIRE(aligned(n_nodes, 4) && aligned(draft_tok, 4) && aligned(acc_parent, 4) && aligned(verify_row, 4) &&
              aligned(draft_prob, 4) && aligned(uniform, 4) && aligned(out_argmax, 4) && aligned(out_prob, 4) &&
              aligned(out_len, 4) && aligned(out_path, 4) && aligned(out_bonus, 4),
          SPEC_EINVAL, "int32 / float arrays must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sv::launch_argmax_lse(logits, logits_dtype, B, T, V, n_nodes, out_argmax, out_prob, s);
  if (e != hipSuccess) return hip_status(e, "argmax / log-sum-exp launch");
  sv::AcceptRule rule{};
  rule.mode = mode;
  rule.threshold = threshold;
  rule.draft_prob = draft_prob;
  rule.uniform = uniform;
  rule.logits = logits;
  rule.logits_bf16 = logits_dtype == SPEC_BF16;
  rule.V = V;
  rule.prob = out_prob;
  sv::CommitArgs no_commit{};
  e = sv::launch_accept(B, T, n_nodes, draft_tok, acc_parent, verify_row, out_argmax, max_depth, out_len, out_path,
                        out_bonus, rule, no_commit, s);
  return hip_status(e, "acceptance scan launch");
}

size_t spec_verify_attn_workspace(const spec_attn_desc* d) {
  if (check_desc(d) != SPEC_OK) return 0;
  return sv::plan_attn(*d).ws_bytes;
}

}  // extern "C"

namespace {

// Argument checks of spec_verify_attn and spec_verify_attn_noalloc (the workspace aside).
// tree: the mask comes from a parent array (mask_bits is attn_parent, and
// sp_bits is the optional sp_flag, so it may be NULL and needs no alignment).
int check_attn_args(const char* fn, const spec_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* cache_len, const void* k_blk, const void* v_blk, const void* k_soft,
                    const void* v_soft, const void* mask_bits, const void* sp_bits, const int32_t* n_q,
                    const void* out, const float* lse, bool tree = false) {
  const int st = check_desc(d);
  if (st != SPEC_OK) return st;
  if (d->B == 0) return SPEC_OK;
  const char* mask_name = tree ? "attn_parent" : "mask_bits";
  REQUIRE(q && k_cache && v_cache && cache_len && k_blk && v_blk && mask_bits && n_q && out, SPEC_EINVAL,
          "%s: q, k_cache, v_cache, cache_len, k_blk, v_blk, %s, n_q and out must be non-NULL", fn, mask_name);
  if (tree) {
    if (d->S > 0) {
      REQUIRE(k_soft && v_soft, SPEC_EINVAL, "%s: S = %d needs k_soft and v_soft", fn, d->S);
    } else {
      REQUIRE(!k_soft && !v_soft, SPEC_EINVAL, "%s: k_soft / v_soft given with S = 0", fn);
    }
    sp_bits = nullptr;   // byte flags: no alignment to check
  } else if (d->S > 0) {
    REQUIRE(k_soft && v_soft && sp_bits, SPEC_EINVAL, "%s: S = %d needs k_soft, v_soft and sp_bits", fn, d->S);
  } else {
    REQUIRE(!k_soft && !v_soft, SPEC_EINVAL, "%s: k_soft / v_soft given with S = 0", fn);
  }
  REQUIRE(aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(k_blk, 16) &&
              aligned(v_blk, 16) && aligned(out, 16) && aligned(k_soft, 16) && aligned(v_soft, 16),
          SPEC_EINVAL, "%s: q, caches, block, soft and out must be 16-byte aligned", fn);
  REQUIRE(aligned(cache_len, 4) && aligned(mask_bits, 4) && aligned(sp_bits, 4) && aligned(n_q, 4) &&
              aligned(lse, 4),
          SPEC_EINVAL, "%s: int32/uint32/float arrays must be 4-byte aligned", fn);
  return SPEC_OK;
}

// Enqueue a validated call; `workspace` holds at least plan.ws_bytes bytes.
// Where the kernel's block mask comes from (mask_bits / sp_bits / n_q, or built
// in the kernel: see sv::MaskMode); only the pointers of that source are read.
struct MaskSource {
  sv::MaskMode mode = sv::MASK_WORDS;
  const int32_t* parent = nullptr;   // attn_parent (MASK_PARENT) or tree_parent (MASK_MSA)
  const uint8_t* sp_flag = nullptr;
  const int32_t* n_nodes = nullptr;
  int N = 0, gamma = 0;
};

int launch_verify_attn(const spec_attn_desc* d, const sv::AttnPlan& plan, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* cache_len, const void* k_blk, const void* v_blk,
                       const void* k_soft, const void* v_soft, const uint32_t* mask_bits, const uint32_t* sp_bits,
                       const int32_t* n_q, void* out, float* lse, void* workspace, void* stream,
                       const MaskSource& ms = MaskSource()) {
  sv::AttnArgs a{};
  a.B = d->B;
  a.Tq = d->Tq;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.G = d->Hq / d->Hkv;
  a.D = d->D;
  a.S = d->S;
  a.W = (d->Tq + 31) / 32;
  a.R = a.G * d->Tq;
  const float scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->D);
  a.c = scale * 1.4426950408889634f;
  a.lmax = d->lmax;
  a.sb = d->kv_stride_b;
  a.sl = d->kv_stride_l;
  a.sh = d->kv_stride_h;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_len = cache_len;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_soft = k_soft;
  a.v_soft = v_soft;
  a.mask_bits = mask_bits;
  a.sp_bits = sp_bits;
  a.n_q = n_q;
  a.out = out;
  a.out_bf16 = d->out_dtype == SPEC_BF16;
  a.lse = lse;
  a.n_split = plan.n_split;
  a.row_chunks = plan.row_chunks;
  a.rows_per_wg = plan.rows_per_wg;
  a.v_tiled = d->v_layout == SPEC_V_TILE32;
  a.mask_mode = ms.mode;
  a.attn_parent = ms.parent;
  a.sp_flag = ms.sp_flag;
  a.n_nodes = ms.n_nodes;
  a.msa_N = ms.N;
  a.msa_gamma = ms.gamma;
  if (plan.n_split > 1) {
    const size_t rows = (size_t)plan.n_split * d->B * d->Hkv * a.R;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    const size_t off = (rows * d->D * sizeof(float) + 255) & ~size_t(255);
    a.part_ml = reinterpret_cast<float*>(ws + off);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = plan.path == sv::PATH_MFMA ? sv::launch_attn_mfma(a, s) : sv::launch_attn_valu(a, d->dtype, s);
  if (e != hipSuccess) return hip_status(e, "spec_verify_attn launch");
  if (plan.n_split > 1) {
    e = sv::launch_attn_combine(a, s);
    if (e != hipSuccess) return hip_status(e, "spec_verify_attn combine launch");
  }
  return ok();
}

// Device address of `scratch` on the calling thread's current device, looked up
// once per device (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "spec_verify_attn_noalloc: hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, SPEC_EUNSUPPORTED, "spec_verify_attn_noalloc: device %d >= %d", dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "spec_verify_attn_noalloc: hipGetSymbolAddress(scratch)");
    REQUIRE(ptr != nullptr, SPEC_EHIP, "spec_verify_attn_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify_attn(const spec_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cache_len, const void* k_blk, const void* v_blk, const void* k_soft,
                     const void* v_soft, const uint32_t* mask_bits, const uint32_t* sp_bits,
                     const int32_t* n_q, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const int st = check_attn_args("spec_verify_attn", d, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft,
                                 v_soft, mask_bits, sp_bits, n_q, out, lse);
  if (st != SPEC_OK) return st;
  if (d->B == 0) return ok();
  const sv::AttnPlan plan = sv::plan_attn(*d);
  if (plan.ws_bytes > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= plan.ws_bytes, SPEC_EWORKSPACE,
            "workspace of %zu bytes needed, %zu given", plan.ws_bytes, workspace ? workspace_bytes : 0);
    REQUIRE(aligned(workspace, 16), SPEC_EINVAL, "workspace must be 16-byte aligned");
  }
  return launch_verify_attn(d, plan, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, mask_bits,
                            sp_bits, n_q, out, lse, workspace, stream);
}

int spec_verify_attn_tree(const spec_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cache_len, const void* k_blk, const void* v_blk, const void* k_soft,
                          const void* v_soft, const int32_t* attn_parent, const uint8_t* sp_flag,
                          const int32_t* n_q, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  static const char* fn = "spec_verify_attn_tree";
  const int st0 = check_desc(d);
  if (st0 != SPEC_OK) return st0;
  if (d->B == 0) return ok();
  REQUIRE(d->dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
          "%s: bf16 inputs only (fp32 inputs: spec_build_mask, then spec_verify_attn)", fn);
  const int st = check_attn_args(fn, d, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, attn_parent,
                                 sp_flag, n_q, out, lse, /*tree=*/true);
  if (st != SPEC_OK) return st;
  const sv::AttnPlan plan = sv::plan_attn(*d);
  if (plan.ws_bytes > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= plan.ws_bytes, SPEC_EWORKSPACE,
            "workspace of %zu bytes needed, %zu given", plan.ws_bytes, workspace ? workspace_bytes : 0);
    REQUIRE(aligned(workspace, 16), SPEC_EINVAL, "workspace must be 16-byte aligned");
  }
  MaskSource ms;
  ms.mode = sv::MASK_PARENT;
  ms.parent = attn_parent;
  ms.sp_flag = sp_flag;
  return launch_verify_attn(d, plan, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, nullptr,
                            nullptr, n_q, out, lse, workspace, stream, ms);
}

int spec_verify_attn_msa(const spec_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cache_len, const void* k_blk, const void* v_blk, const void* k_soft,
                         const void* v_soft, const int32_t* tree_parent, const int32_t* n_nodes, int32_t N,
                         int32_t gamma, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  static const char* fn = "spec_verify_attn_msa";
  const int st0 = check_desc(d);
  if (st0 != SPEC_OK) return st0;
  REQUIRE(gamma >= 0 && gamma < SPEC_MAX_TQ, SPEC_EINVAL, "%s: gamma = %d outside [0, %d)", fn, gamma, SPEC_MAX_TQ);
  REQUIRE(N >= 1 && N <= SPEC_MAX_TQ, SPEC_EINVAL, "%s: N = %d outside [1, %d]", fn, N, SPEC_MAX_TQ);
  REQUIRE((int64_t)N * (1 + gamma) <= d->Tq, SPEC_EINVAL, "%s: N * (1 + gamma) = %lld rows exceed Tq = %d", fn,
          (long long)N * (1 + gamma), d->Tq);
  if (d->B == 0) return ok();
  REQUIRE(d->dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
          "%s: bf16 inputs only (fp32 inputs: spec_build_msa_mask, then spec_verify_attn)", fn);
  // spec_verify_attn's checks, the node tree in place of the mask and n_nodes in place of n_q
  REQUIRE(tree_parent != nullptr, SPEC_EINVAL, "%s: tree_parent must be non-NULL", fn);
  REQUIRE(n_nodes != nullptr, SPEC_EINVAL, "%s: n_nodes must be non-NULL", fn);
  const int st = check_attn_args(fn, d, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, tree_parent,
                                 nullptr, n_nodes, out, lse, /*tree=*/true);
  if (st != SPEC_OK) return st;
  const sv::AttnPlan plan = sv::plan_attn(*d);
  if (plan.ws_bytes > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= plan.ws_bytes, SPEC_EWORKSPACE,
            "workspace of %zu bytes needed, %zu given", plan.ws_bytes, workspace ? workspace_bytes : 0);
    REQUIRE(aligned(workspace, 16), SPEC_EINVAL, "workspace must be 16-byte aligned");
  }
  MaskSource ms;
  ms.mode = sv::MASK_MSA;
  ms.parent = tree_parent;
  ms.n_nodes = n_nodes;
  ms.N = N;
  ms.gamma = gamma;
  return launch_verify_attn(d, plan, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, nullptr,
                            nullptr, nullptr, out, lse, workspace, stream, ms);
}

int spec_verify_attn_noalloc(const spec_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cache_len, const void* k_blk, const void* v_blk, const void* k_soft,
                             const void* v_soft, const uint32_t* mask_bits, const uint32_t* sp_bits,
                             const int32_t* n_q, void* out, float* lse, void* stream) {
  const int st = check_attn_args("spec_verify_attn_noalloc", d, q, k_cache, v_cache, cache_len, k_blk, v_blk,
                                 k_soft, v_soft, mask_bits, sp_bits, n_q, out, lse);
  if (st != SPEC_OK) return st;
  if (d->B == 0) return ok();
  const sv::AttnPlan plan = sv::plan_attn(*d);
  REQUIRE(plan.ws_bytes <= (size_t)SPEC_NOALLOC_SCRATCH_BYTES, SPEC_EWORKSPACE,
          "spec_verify_attn_noalloc: this call needs %zu bytes of split-KV scratch, more than the %zu the "
          "library holds per GPU (use fewer splits, or spec_verify_attn with a workspace)",
          plan.ws_bytes, (size_t)SPEC_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    const int sst = scratch_of_current_device(&ws);
    if (sst != SPEC_OK) return sst;
  }
  return launch_verify_attn(d, plan, q, k_cache, v_cache, cache_len, k_blk, v_blk, k_soft, v_soft, mask_bits,
                            sp_bits, n_q, out, lse, ws, stream);
}

int spec_argmax_accept(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                       const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                       int32_t max_depth, int32_t* out_argmax, int32_t* out_len, int32_t* out_path,
                       void* stream) {
  return argmax_accept_impl("spec_argmax_accept", logits, logits_dtype, B, T, V, n_nodes, draft_tok, acc_parent,
                            nullptr, max_depth, out_argmax, out_len, out_path, nullptr, stream);
}

int spec_argmax_accept_rows(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                            const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                            const int32_t* verify_row, int32_t max_depth, int32_t* out_argmax, int32_t* out_len,
                            int32_t* out_path, int32_t* out_bonus, void* stream) {
  return argmax_accept_impl("spec_argmax_accept_rows", logits, logits_dtype, B, T, V, n_nodes, draft_tok,
                            acc_parent, verify_row, max_depth, out_argmax, out_len, out_path, out_bonus, stream);
}

int spec_commit_kv(const spec_attn_desc* d, void* k_cache, void* v_cache, const int32_t* cache_len_in,
                   int32_t* cache_len_out, const void* k_blk, const void* v_blk, const int32_t* out_len,
                   const int32_t* out_path, int32_t max_depth, void* stream) {
  const int st = check_desc(d);
  if (st != SPEC_OK) return st;
  REQUIRE(max_depth >= 1 && max_depth <= SPEC_MAX_DEPTH, SPEC_EINVAL, "max_depth = %d outside [1, %d]",
          max_depth, SPEC_MAX_DEPTH);
  if (d->B == 0) return ok();
  REQUIRE(k_cache && v_cache && cache_len_in && cache_len_out && k_blk && v_blk && out_len && out_path,
          SPEC_EINVAL, "all array arguments must be non-NULL");
  REQUIRE(aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(k_blk, 16) && aligned(v_blk, 16),
          SPEC_EINVAL, "caches and block must be 16-byte aligned");
  REQUIRE(aligned(cache_len_in, 4) && aligned(cache_len_out, 4) && aligned(out_len, 4) && aligned(out_path, 4),
          SPEC_EINVAL, "int32 arrays must be 4-byte aligned");
  const hipError_t e =
      sv::launch_commit(d->B, d->Tq, d->Hkv, d->D, esize_of(d->dtype), d->lmax, d->kv_stride_b,
                        d->kv_stride_l, d->kv_stride_h, d->v_layout == SPEC_V_TILE32, k_cache, v_cache,
                        cache_len_in, cache_len_out, k_blk, v_blk, out_len, out_path, max_depth,
                        static_cast<hipStream_t>(stream));
  return hip_status(e, "spec_commit_kv launch");
}

int spec_argmax_accept_commit(const void* logits, int32_t logits_dtype, int32_t T, int32_t V, const int32_t* n_nodes,
                              const int32_t* draft_tok, const int32_t* acc_parent, const int32_t* verify_row,
                              int32_t max_depth, int32_t* out_argmax, int32_t* out_len, int32_t* out_path,
                              int32_t* out_bonus, const spec_attn_desc* d, void* k_cache, void* v_cache,
                              const int32_t* cache_len_in, int32_t* cache_len_out, const void* k_blk,
                              const void* v_blk, void* stream) {
  const int st = check_desc(d);
  if (st != SPEC_OK) return st;
  const int B = d->B;
  REQUIRE(T >= 1 && T <= SPEC_MAX_NODES, SPEC_EINVAL, "T = %d outside [1, %d]", T, SPEC_MAX_NODES);
  REQUIRE(T <= d->Tq, SPEC_EINVAL, "T = %d acceptance nodes exceed the block's Tq = %d rows", T, d->Tq);
  REQUIRE(V >= 1, SPEC_EINVAL, "V = %d < 1", V);
  REQUIRE(max_depth >= 1 && max_depth <= SPEC_MAX_DEPTH, SPEC_EINVAL, "max_depth = %d outside [1, %d]", max_depth,
          SPEC_MAX_DEPTH);
  REQUIRE(logits_dtype == SPEC_F32 || logits_dtype == SPEC_BF16, SPEC_EINVAL, "logits_dtype = %d is not a spec_dtype",
          logits_dtype);
  REQUIRE((int64_t)B * T <= 0x7fffffff, SPEC_EUNSUPPORTED, "B * T too large");
  if (B == 0) return ok();
  REQUIRE(logits && n_nodes && draft_tok && acc_parent && out_argmax && out_len && out_path && k_cache && v_cache &&
              cache_len_in && cache_len_out && k_blk && v_blk,
          SPEC_EINVAL, "all array arguments except verify_row and out_bonus must be non-NULL");
  REQUIRE(aligned(logits, esize_of(logits_dtype)), SPEC_EINVAL, "logits must be aligned to its element size");
  REQUIRE(aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(k_blk, 16) && aligned(v_blk, 16), SPEC_EINVAL,
          "caches and block must be 16-byte aligned");
  REQUIRE(aligned(n_nodes, 4) && aligned(draft_tok, 4) && aligned(acc_parent, 4) && aligned(verify_row, 4) &&
              aligned(out_argmax, 4) && aligned(out_len, 4) && aligned(out_path, 4) && aligned(out_bonus, 4) &&
              aligned(cache_len_in, 4) && aligned(cache_len_out, 4),
          SPEC_EINVAL, "int32 arrays must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sv::launch_argmax(logits, logits_dtype, B, T, V, n_nodes, out_argmax, s);
  if (e != hipSuccess) return hip_status(e, "argmax launch");
  sv::AcceptRule greedy{};
  sv::CommitArgs c{1, d->Tq, d->Hkv, d->D, esize_of(d->dtype), d->lmax, d->kv_stride_b, d->kv_stride_l,
                   d->kv_stride_h, d->v_layout == SPEC_V_TILE32, static_cast<char*>(k_cache),
                   static_cast<char*>(v_cache), cache_len_in, cache_len_out, static_cast<const char*>(k_blk),
                   static_cast<const char*>(v_blk)};
  e = sv::launch_accept(B, T, n_nodes, draft_tok, acc_parent, verify_row, out_argmax, max_depth, out_len, out_path,
                        out_bonus, greedy, c, s);
  return hip_status(e, "acceptance + commit launch");
}

}  // extern "C"
