// Internal interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// Fully resolved arguments of one verify-attention call.
struct AttnArgs {
  int B, Tq, Hq, Hkv, G, D, S, W;   // W = mask words per row
  int R;                            // attention rows per (request, kv-head) = G * Tq
  float c;                          // softmax scale * log2(e): scores live in the log2 domain
  int64_t lmax, sb, sl, sh;         // cache capacity and element strides
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cache_len;
  const void* k_blk;
  const void* v_blk;
  const void* k_soft;
  const void* v_soft;
  const uint32_t* mask_bits;
  const uint32_t* sp_bits;
  const int32_t* n_q;
  void* out;                        // float32, or bf16 when out_bf16
  int out_bf16;
  float* lse;
  // split-KV partials (only when n_split > 1):
  //   part_o  [n_split][B][Hkv][R][D]  unnormalised accumulators
  //   part_ml [n_split][B][Hkv][R][2]  running max (log2 domain) and sum
  float* part_o;
  float* part_ml;
  int n_split;
  int row_chunks;                   // MFMA path: row chunks per (request, kv-head)
  int rows_per_wg;                  // MFMA path: 64 or 128 rows per workgroup
  int v_tiled;                      // V cache in SPEC_V_TILE32 layout (MFMA path only)
  // where the block mask comes from: MASK_WORDS = mask_bits / sp_bits / n_q
  // (spec_verify_attn); MASK_PARENT = built in the kernel from attn_parent,
  // sp_flag and n_q (spec_verify_attn_tree); MASK_MSA = built in the kernel from
  // the node tree (attn_parent = tree_parent [B][msa_N], n_nodes, msa_gamma), the
  // row count being n_nodes * (1 + gamma) (spec_verify_attn_msa)
  int mask_mode;
  const int32_t* attn_parent;
  const uint8_t* sp_flag;           // [B][Tq] or NULL (MASK_PARENT)
  const int32_t* n_nodes;           // [B] (MASK_MSA)
  int msa_N, msa_gamma;
  // MFMA path: deal the (request, kv-head) pairs over the XCDs longest prefix
  // first (set by the launcher when the grid takes more than one round of
  // workgroups; needs n_split == 1 and B * Hkv a multiple of 8)
  int balance;
};

enum MaskMode { MASK_WORDS = 0, MASK_PARENT = 1, MASK_MSA = 2 };

enum AttnPath { PATH_VALU = 0, PATH_MFMA = 1 };

struct AttnPlan {
  AttnPath path;
  int n_split;
  int row_chunks;
  int rows_per_wg;
  size_t ws_bytes;
};

// Schedule for a validated descriptor (deterministic in the descriptor).
AttnPlan plan_attn(const spec_attn_desc& d);

hipError_t launch_build_mask(const int32_t* attn_parent, const uint8_t* sp_flag, const int32_t* n_q,
                             int B, int Tq, uint32_t* mask_bits, uint32_t* sp_bits, hipStream_t st);
hipError_t launch_build_msa_mask(const int32_t* tree_parent, const int32_t* n_nodes, int B, int N,
                                 int gamma, int Tq, uint32_t* mask_bits, uint32_t* sp_bits,
                                 int32_t* n_q, hipStream_t st);
hipError_t launch_draft_tree(const void* logits, int dtype, int B, int R, int V, const int32_t* n_nodes,
                             const int32_t* acc_len, const int32_t* acc_path, int max_depth,
                             const int32_t* root_tok, int gamma, int k, int N, int32_t* out_topk,
                             int32_t* draft_tok, int32_t* tree_parent, int32_t* n_out, hipStream_t st);
hipError_t launch_attn_valu(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st);
hipError_t launch_argmax(const void* logits, int dtype, int B, int T, int V, const int32_t* n_nodes,
                         int32_t* out_argmax, hipStream_t st);
// Cache commit of an accepted path (k_commit, or fused after the acceptance scan).
struct CommitArgs {
  int enabled;              // fused form: 0 = acceptance only
  int Tq, Hkv, D, esize;
  int64_t lmax, sb, sl, sh; // cache capacity and element strides
  int v_tiled;              // V cache in SPEC_V_TILE32 layout
  char* k_cache;
  char* v_cache;
  const int32_t* cache_len_in;
  int32_t* cache_len_out;
  const char* k_blk;
  const char* v_blk;
};

// Per-node acceptance decision of k_accept.
struct AcceptRule {
  int mode;                 // 0: the draft equals the row's greedy token; 1: p > threshold; 2: u * p_draft < p
  float threshold;          // mode 1
  const float* draft_prob;  // mode 2: [B, T]
  const float* uniform;     // mode 2: [B, T]
  const void* logits;       // modes 1, 2: [B, T, V], for the draft's logit
  int logits_bf16;
  int V;
  float* prob;              // modes 1, 2: [B, T]; in: each row's log-sum-exp, out: each node's p
};

hipError_t launch_argmax_lse(const void* logits, int dtype, int B, int T, int V, const int32_t* n_nodes,
                             int32_t* out_argmax, float* out_lse, hipStream_t st);
// verify_row == nullptr: row v verifies node v; out_bonus may be nullptr
hipError_t launch_accept(int B, int T, const int32_t* n_nodes, const int32_t* draft_tok,
                         const int32_t* acc_parent, const int32_t* verify_row, const int32_t* argmax,
                         int max_depth, int32_t* out_len, int32_t* out_path, int32_t* out_bonus,
                         const AcceptRule& rule, const CommitArgs& commit, hipStream_t st);
hipError_t launch_commit(int B, int Tq, int Hkv, int D, int esize, int64_t lmax, int64_t sb,
                         int64_t sl, int64_t sh, int v_tiled, void* k_cache, void* v_cache,
                         const int32_t* cache_len_in, int32_t* cache_len_out, const void* k_blk,
                         const void* v_blk, const int32_t* out_len, const int32_t* out_path,
                         int max_depth, hipStream_t st);

}  // namespace sv
