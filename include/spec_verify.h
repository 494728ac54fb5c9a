/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) verification step for
 * self-speculative decoding.
 *
 * One decode iteration of self-speculative decoding runs the target model
 * once over [cached prefix + a block of speculative tokens], accepts or
 * rejects the drafts from the block's logits, and keeps only the accepted
 * tokens' K/V.  This library implements the data-parallel parts of that step
 * as hand-written HIP kernels:
 *
 *   spec_build_mask     parent array -> bit-packed block visibility mask
 *   spec_build_msa_mask the same for multi-stream rows (main + speculative
 *                       streams per tree node)
 *   spec_verify_attn    attention of the block's queries over
 *                       [soft prompt | cached prefix | block] under that mask
 *   spec_verify_attn_noalloc  the same without a workspace argument (for
 *                       callers that cannot allocate)
 *   spec_verify_attn_tree  mask build and attention in one launch
 *   spec_verify_attn_msa   multi-stream mask build and attention in one launch
 *   spec_argmax_accept  per-node greedy token, longest accepted path
 *   spec_argmax_accept_rows  the same with explicit verification rows, an
 *                       explicit root and the correction token
 *   spec_prob_accept    the same scan with a threshold or soft-matching rule
 *                       on the target's probability of each draft
 *   spec_commit_kv      append the accepted nodes' K/V to the cache
 *   spec_argmax_accept_commit  argmax, acceptance and commit, fused
 *   spec_draft_tree     the next tree draft from the new root's streams
 *
 * Sources (page titles; sections, equations):
 *   [LA] "Lookahead Attention: Self-Speculative Verification via Parallel
 *        Token Proposals" -- 2.1 dual-stream mask, 2.3/2.4 verification and
 *        longest consistent prefix, 3.1 M_LA, 3.2 KV discarded, 3.3 padding.
 *   [CF] "ConFu: Contemplate the Future for Better Speculative Sampling" --
 *        key design 1: soft prompt in the KV cache visible only to
 *        contemplate tokens; one contemplate token per tree node (2T rows).
 *   [SS] "Speculative Streaming: Fast LLM Inference without Auxiliary
 *        Models" -- Equation 1 (attention, 1/sqrt(d) scale), Equation 2
 *        (multi-stream attention), tree draft construction and Equation 4
 *        (each node sees its root-to-node path), batching with speculative
 *        streams, the verification step (depth-first, hard or soft matching,
 *        longest accepted path, correction token), parallel new draft
 *        generation, lazy KV garbage collection after the step.
 *
 * Conventions (all entry points):
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     stated otherwise.  The library allocates no memory and keeps no state
 *     between calls; calls are reentrant (spec_verify_attn_noalloc aside,
 *     which uses a scratch array the library holds per GPU).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; the functions never synchronise.  Values that
 *     depend on data (accepted lengths and paths, cache lengths) stay on the
 *     device, so the calls chain on one stream without a host round trip.
 *   - Return value: SPEC_OK, or a negative spec_status.  Shapes, dtypes,
 *     pointers and alignment are validated on the host BEFORE anything is
 *     enqueued; on failure nothing is enqueued.  spec_last_error() returns a
 *     thread-local description of the most recent failure in this thread.
 *   - Contents of device arrays (parents, lengths, token ids) cannot be
 *     checked on the host; they are preconditions stated per function.  The
 *     kernels clamp every index they derive from such data, so a violated
 *     precondition gives unspecified results but never an out-of-bounds
 *     access.
 *   - bf16 is IEEE-style bfloat16 (the upper 16 bits of a float32).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_F32 = 0,   /* float32  */
  SPEC_BF16 = 1   /* bfloat16 */
} spec_dtype;

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,        /* bad argument: null pointer, bad shape, misaligned */
  SPEC_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  SPEC_EWORKSPACE = -3,    /* workspace missing or smaller than required       */
  SPEC_EHIP = -4           /* the HIP runtime reported an error                */
} spec_status;

/* Limits of this implementation. */
#define SPEC_MAX_TQ 256        /* query rows per request in the block      */
#define SPEC_MAX_NODES 256     /* acceptance nodes per request             */
#define SPEC_MAX_DEPTH 16      /* longest accepted path                    */
#define SPEC_MAX_SOFT 256      /* soft-prompt rows                          */
#define SPEC_MAX_TOPK 8        /* tokens per speculative stream in a draft  */
/* device scratch spec_verify_attn_noalloc holds per GPU (32 MiB) */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)

/* acceptance rules of spec_prob_accept */
#define SPEC_ACCEPT_THRESHOLD 1 /* [LA]: target probability of the draft > threshold          */
#define SPEC_ACCEPT_SOFT 2      /* [SS] soft matching: accept with probability min(1, p/p_d) */

/* Shape and layout of one verify-attention call (one transformer layer). */
typedef struct {
  int32_t B;       /* requests                                                */
  int32_t Tq;      /* query rows of the speculative block per request (<=256) */
  int32_t Hq;      /* query heads                                             */
  int32_t Hkv;     /* key/value heads; Hq % Hkv == 0; q-head j reads kv-head
                      j / (Hq / Hkv) (contiguous groups)                      */
  int32_t D;       /* head dimension: 64 or 128                               */
  int32_t S;       /* soft-prompt rows (0 = none)                             */
  int32_t dtype;   /* spec_dtype of q, caches, block and soft K/V             */
  float scale;     /* softmax scale; 0 selects 1/sqrt(D) ([SS] Equation 1)    */
  int64_t lmax;    /* cache capacity in rows per request                      */
  int64_t kv_stride_b, kv_stride_l, kv_stride_h; /* element strides of the
                      caches for request, row and head; D is contiguous.
                      [B, lmax, Hkv, D] contiguous: (lmax*Hkv*D, Hkv*D, D);
                      [B, Hkv, lmax, D] contiguous: (Hkv*lmax*D, D, lmax*D). */
  int32_t kv_splits; /* 0 = automatic; else split each request's prefix into
                        this many key ranges (tuning and testing)             */
  int32_t v_layout;  /* spec_v_layout of v_cache (K always uses the strides)  */
  int32_t out_dtype; /* spec_dtype of out: SPEC_F32 (0, the default) or
                        SPEC_BF16 (bf16 inputs only): each output value is the
                        float32 result rounded to nearest even             */
} spec_attn_desc;

/* Layout of the V cache (spec_attn_desc.v_layout).
 *   SPEC_V_ROWS    V has K's layout: element (b, l, h, d) at
 *                  b*kv_stride_b + l*kv_stride_l + h*kv_stride_h + d.
 *   SPEC_V_TILE32  V is stored in tiles of 32 keys, each tile a contiguous
 *                  [D/16][4][16][8] block -- head-dim block, key group, head dim
 *                  within the block, key within the group -- so that every
 *                  16 bytes is one operand of the attention's P*V matrix
 *                  instruction.  Key l = 32t + k, head dim x of head h is at
 *                  b*kv_stride_b + h*kv_stride_h + 32t*D
 *                    + (x/16)*512 + g*128 + (x%16)*8 + e,
 *                  g = (k%16)/4, e = k%4 + 4*(k/16) (a group holds keys
 *                  4g..4g+3 and 16+4g..16+4g+3, the keys one lane's score
 *                  accumulators hold).  Needs bf16, a head-major cache
 *                  (kv_stride_l == D, so K is [B, Hkv, lmax, D] and V fills
 *                  the same space) and lmax % 32 == 0.  spec_commit_kv and
 *                  spec_argmax_accept_commit write accepted rows in this layout. */
#define SPEC_V_ROWS 0
#define SPEC_V_TILE32 1

/*
 * spec_build_mask -- bit-packed visibility of block keys for each query row.
 *
 * Row r of request b sees block key c iff r < n_q[b] and (c == r or c is an
 * ancestor of r through attn_parent).  This one rule gives every mask of the
 * sources: [SS] tree (a node sees its root-to-node path and no other branch;
 * the printed Equation 4 is read through its prose, self included), [LA]
 * M_LA (originals as a chain, lookahead rows hanging off the last original:
 * causal originals, lookahead rows see the originals and themselves only;
 * with the originals cached, all parents are -1: prefix + self), [CF]
 * contemplate rows (parent = their node: the node's path, the node, itself).
 * Every valid row also sees the whole cached prefix (implicit, not stored).
 *
 *   attn_parent [B, Tq] int32   parent row, -1 = hangs off the prefix.
 *                               Precondition: -1 <= attn_parent[b][r] < r.
 *                               A link that breaks it ends the walk.
 *   sp_flag     [B, Tq] uint8   nonzero = the row sees the soft prompt
 *                               ([CF] contemplate rows); NULL = no row does.
 *   n_q         [B] int32       valid rows per request; rows r >= n_q[b] are
 *                               batch padding ([LA] 3.3) and see nothing.
 *                               Clamped to [0, Tq].
 *   mask_bits   [B, Tq, W] uint32 out, W = ceil(Tq/32): bit (c % 32) of
 *                               word c / 32 is key c; unused high bits are 0.
 *   sp_bits     [B, W] uint32   out: bit r = row r sees the soft prompt.
 *
 * Limits: 1 <= Tq <= 256.  B == 0 is a no-op.
 */
int spec_build_mask(const int32_t* attn_parent, const uint8_t* sp_flag, const int32_t* n_q,
                    int32_t B, int32_t Tq, uint32_t* mask_bits, uint32_t* sp_bits,
                    void* stream);

/*
 * spec_build_msa_mask -- block masks for multi-stream (MSA) verification rows.
 *
 * [SS] Multi-Stream Attention: every node of the flattened tree draft carries
 * one main-stream query and gamma speculative-stream queries (the batching
 * paragraph: (1 + gamma) rows per tree node).  Row layout of request b with
 * n = n_nodes[b] nodes: rows 0..n-1 are the main streams of nodes 0..n-1,
 * row n + v*gamma + (j-1) is speculative stream j (1..gamma) of node v, and
 * rows from n*(1+gamma) on are padding.  What each row sees (Equations 1 and
 * 2 over the tree of Equation 4, read through its prose):
 *   main stream of v      the main rows of the nodes on the root-to-v path
 *                         (v included), never another branch;
 *   stream j of v         the same main rows plus streams 1..j of v itself,
 *                         never another node's streams.
 * Every valid row also sees the whole cached prefix; no row sees the soft
 * prompt (sp_bits is all zero).  The main rows of nodes are the first n rows,
 * so a node's parent index is also the row of its parent's main stream: pass
 * tree_parent as verify_row to spec_argmax_accept_rows (root: -1, accepted
 * unchecked), and the accepted path's node indices are the main rows to
 * commit (stream K/V is never committed).
 *
 *   tree_parent [B, N] int32    parent node, -1 = the root.  Precondition:
 *                               -1 <= tree_parent[b][v] < v; a link that
 *                               breaks it ends the walk.
 *   n_nodes     [B] int32       tree nodes per request, clamped to [0, N].
 *   gamma                       speculative streams per node, >= 0.
 *   Tq                          rows of the block, >= N * (1 + gamma).
 *   mask_bits   [B, Tq, W] uint32 out, W = ceil(Tq/32), as spec_build_mask.
 *   sp_bits     [B, W] uint32   out: all zero.
 *   n_q         [B] int32       out: valid rows n_nodes[b] * (1 + gamma), the
 *                               n_q argument of spec_verify_attn.
 *
 * Limits: 1 <= N, N * (1 + gamma) <= Tq <= 256.  B == 0 is a no-op.
 */
int spec_build_msa_mask(const int32_t* tree_parent, const int32_t* n_nodes, int32_t B, int32_t N,
                        int32_t gamma, int32_t Tq, uint32_t* mask_bits, uint32_t* sp_bits, int32_t* n_q,
                        void* stream);

/*
 * spec_prob_accept -- acceptance by the target's probability of each draft.
 *
 * The scan of spec_argmax_accept_rows (a node counts only if its whole root
 * path is accepted; longest path, depth-first-first among equals; an explicit
 * root, verification row -1, is accepted unchecked; a row outside [0, n)
 * never accepts; the correction token is the greedy token of the last
 * accepted node's row), with the per-node decision taken on
 * p = softmax(logits[b, u])[draft_tok[b, v]], u the node's verification row:
 *   SPEC_ACCEPT_THRESHOLD  p > threshold ([LA] verification: each proposal's
 *                          probability exceeds a threshold; longest prefix);
 *   SPEC_ACCEPT_SOFT       uniform[b,v] * draft_prob[b,v] < p, i.e. acceptance
 *                          with probability min(1, p / p_draft) for a uniform
 *                          draw in [0, 1) ([SS] verification, soft matching
 *                          after Leviathan et al.; the draw is an input).
 * p is computed in float32 from the row's log-sum-exp (one streaming pass per
 * row that also yields the greedy token).
 *
 *   logits, logits_dtype, B, T, V, n_nodes, draft_tok, acc_parent,
 *   verify_row (NULL = row v verifies node v), max_depth, out_argmax,
 *   out_len, out_path, out_bonus (may be NULL): as spec_argmax_accept_rows.
 *   threshold   SPEC_ACCEPT_THRESHOLD: finite, >= 0.
 *   draft_prob  [B, T] float: SPEC_ACCEPT_SOFT only, the draft's probability
 *               of its token (0 = accept iff p > 0).
 *   uniform     [B, T] float: SPEC_ACCEPT_SOFT only, draws in [0, 1).
 *   out_prob    [B, T] float out: p of each node (1 for the unchecked root, 0
 *               for a row or token out of range; NaN past n_nodes[b]).
 *
 * Limits as spec_argmax_accept_rows.  A row holding a NaN logit, or none
 * above -inf, has an undefined softmax: its p is NaN and its drafts are not
 * accepted.
 */
int spec_prob_accept(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                     const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                     const int32_t* verify_row, int32_t max_depth, int32_t mode, float threshold,
                     const float* draft_prob, const float* uniform, int32_t* out_argmax, float* out_prob,
                     int32_t* out_len, int32_t* out_path, int32_t* out_bonus, void* stream);

/*
 * spec_draft_tree -- the next tree draft from the new root's speculative
 * streams ([SS] tree draft construction and parallel new draft generation).
 *
 * The pass that verifies a draft also drafts the next one.  The new root is
 * the last node of the accepted path (acc_path[b][acc_len[b]-1]); its gamma
 * speculative streams sit at block rows n + last*gamma + (j-1), j = 1..gamma,
 * of the multi-stream layout (spec_build_msa_mask), n = n_nodes[b].  From each
 * stream's logit row the k best tokens are taken (largest logit first, equal
 * logits in increasing token order; k = 1 is greedy).  Stream j's tokens are
 * the children of every node of level j-1 and the root carries root_tok[b]
 * (the correction token, spec_argmax_accept_rows' out_bonus): a complete
 * k-ary tree of depth gamma with N = 1 + k + ... + k^gamma nodes, flattened
 * level by level -- the children of node p are k*p+1 .. k*p+k in the rank
 * order of their tokens, so tree_parent[v] = (v-1)/k.  It feeds the next
 * spec_build_msa_mask directly.
 *
 *   logits      [B, R, V] float32 or bf16 (logits_dtype), the block's rows;
 *               NaN ranks after every number (-inf included), NaN entries
 *               in increasing token order.
 *   n_nodes     [B] int32   nodes of the verified tree.
 *   acc_len     [B] int32, acc_path [B, max_depth] int32: the accepted paths
 *               (spec_argmax_accept_rows' out_len and out_path).
 *   root_tok    [B] int32   token of the new root.
 *   out_topk    [B, gamma, k] int32 out: each stream's k tokens (may be NULL
 *               only when gamma == 0).
 *   draft_tok   [B, N] int32 out, tree_parent [B, N] int32 out.
 *   n_out       [B] int32 out: N, or 0 when request b has no new root (no
 *               accepted node, a path entry outside [0, n_nodes[b]), or
 *               n_nodes[b] * (1 + gamma) > R); its out_topk, draft_tok and
 *               tree_parent entries are then all -1.
 *
 * Limits: 0 <= gamma, 1 <= k <= 8, N <= 256, k <= V, 1 <= max_depth <= 16,
 * 1 <= R <= 256.  B == 0 is a no-op.
 */
int spec_draft_tree(const void* logits, int32_t logits_dtype, int32_t B, int32_t R, int32_t V,
                    const int32_t* n_nodes, const int32_t* acc_len, const int32_t* acc_path, int32_t max_depth,
                    const int32_t* root_tok, int32_t gamma, int32_t k, int32_t* out_topk, int32_t* draft_tok,
                    int32_t* tree_parent, int32_t* n_out, void* stream);

/*
 * spec_verify_attn_workspace -- bytes of device workspace spec_verify_attn
 * needs for this descriptor (0 if none).  Returns 0 for an invalid
 * descriptor as well; spec_verify_attn reports the error.
 */
size_t spec_verify_attn_workspace(const spec_attn_desc* d);

/*
 * spec_verify_attn -- masked attention of the speculative block.
 *
 * For request b, valid row r (< n_q[b]) and query head j (kv-head
 * h = j / (Hq/Hkv)), over the keys the row sees:
 *   soft keys s < S        iff bit r of sp_bits[b]              ([CF])
 *   prefix keys l < L_b    always, L_b = cache_len[b]          ([LA], [SS])
 *   block keys c < Tq      iff bit c of mask_bits[b][r]        (spec_build_mask)
 * out[b,r,j,:] = sum_k softmax_k(scale * <q, k>) v_k              ([SS] Eq. 1)
 * lse[b,r,j]   = natural log of sum_k exp(scale * <q, k>).
 * Padded rows (r >= n_q[b]) get out = 0 and lse = -inf.
 *
 *   q        [B, Tq, Hq, D] dtype, contiguous
 *   k_cache, v_cache  cache rows per the descriptor's strides; only rows
 *            [0, L_b) are read.  Precondition: 0 <= cache_len[b] <= lmax
 *            (clamped).
 *   k_blk, v_blk  [B, Tq, Hkv, D] dtype, contiguous: the block's own K/V
 *   k_soft, v_soft [S, Hkv, D] dtype, shared by all requests; NULL iff S == 0
 *   mask_bits [B, Tq, W], sp_bits [B, W] as produced by spec_build_mask
 *            (sp_bits may be NULL iff S == 0)
 *   n_q      [B] int32, clamped to [0, Tq]
 *   out      [B, Tq, Hq, D] float32, or bf16 when d->out_dtype is SPEC_BF16
 *   lse      [B, Tq, Hq] float32, or NULL
 *   workspace  device buffer of at least spec_verify_attn_workspace(d)
 *            bytes (may be NULL when that is 0).  Contents need no
 *            initialisation and are scratch after the call.
 *
 * Computation: fp32 accumulation; bf16 inputs use bf16 MFMA for QK^T and PV
 * (probabilities rounded to bf16 for PV); fp32 inputs use fp32 VALU
 * arithmetic throughout.  A key a row does not see never reaches that row
 * through its K, whatever the K holds; its V enters the P*V product times a
 * zero probability, so the V rows of keys within [0, L_b), [0, S) and
 * [0, n_q[b]) must be finite (cache rows past L_b are never read).
 * Alignment: all tensors 16-byte aligned, and
 * the strides a multiple of 16 bytes.
 * Limits: D in {64, 128}; 1 <= Tq <= 256; 0 <= S <= 256; B == 0 is a no-op.
 */
int spec_verify_attn(const spec_attn_desc* d, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* cache_len,
                     const void* k_blk, const void* v_blk,
                     const void* k_soft, const void* v_soft,
                     const uint32_t* mask_bits, const uint32_t* sp_bits, const int32_t* n_q,
                     void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * spec_verify_attn_tree -- spec_build_mask and spec_verify_attn in one launch:
 * the attention builds each row's block mask itself from the parent array
 * (the rule of spec_build_mask: row r < n_q[b] sees block key c iff c == r or
 * c is an ancestor of r through parent links that point strictly upwards; the
 * first link that does not ends the chain), so the mask never goes through
 * memory and the step saves a kernel.  Sources: as spec_build_mask ([SS] tree
 * draft and Equation 4, [LA] 3.1 M_LA, [CF] key design 1) and spec_verify_attn.
 *
 *   attn_parent [B, Tq] int32   as spec_build_mask (4-byte aligned)
 *   sp_flag     [B, Tq] uint8   as spec_build_mask; NULL = no row sees the
 *                               soft prompt (then S > 0 still needs k_soft
 *                               and v_soft)
 * Every other argument, the workspace (spec_verify_attn_workspace) and the
 * results are those of spec_verify_attn; out and lse are bitwise equal to
 * spec_build_mask followed by spec_verify_attn on the same inputs.
 *
 * bf16 inputs only (the matrix-core kernel); fp32 inputs return
 * SPEC_EUNSUPPORTED (use the two calls).  Errors otherwise as
 * spec_verify_attn, with attn_parent in place of mask_bits.
 */
int spec_verify_attn_tree(const spec_attn_desc* d, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* cache_len,
                          const void* k_blk, const void* v_blk,
                          const void* k_soft, const void* v_soft,
                          const int32_t* attn_parent, const uint8_t* sp_flag, const int32_t* n_q,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * spec_verify_attn_msa -- spec_build_msa_mask and spec_verify_attn in one
 * launch: the attention builds the multi-stream rows' masks itself from the
 * node tree ([SS] Multi-Stream Attention, Equations 1 and 2 over the tree
 * draft of Equation 4, and the batching paragraph: (1 + gamma) rows per node),
 * with the rule and row layout of spec_build_msa_mask: rows 0..n-1 are the
 * main streams of nodes 0..n-1, row n + v*gamma + (j-1) is stream j of node v;
 * a main row sees the main rows of its node's root path (tree-parent links
 * that point strictly upwards), stream j of v sees those and streams 1..j of
 * v; n = clamp(n_nodes[b], 0, N), and rows from n * (1 + gamma) on are padding.
 * No row sees the soft prompt.
 *
 *   tree_parent [B, N] int32   node parents, -1 = the root's parent (4-byte aligned)
 *   n_nodes     [B] int32      nodes per request (takes the place of n_q)
 *   N, gamma                   as spec_build_msa_mask: 1 <= N, 0 <= gamma,
 *                              N * (1 + gamma) <= Tq
 * Every other argument, the workspace (spec_verify_attn_workspace) and the
 * results are those of spec_verify_attn; out and lse are bitwise equal to
 * spec_build_msa_mask followed by spec_verify_attn on the same inputs.  The
 * row counts n_q are not written (spec_build_msa_mask writes them).
 *
 * bf16 inputs only; fp32 inputs return SPEC_EUNSUPPORTED.  Errors otherwise
 * as spec_verify_attn and spec_build_msa_mask.
 */
int spec_verify_attn_msa(const spec_attn_desc* d, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* cache_len,
                         const void* k_blk, const void* v_blk,
                         const void* k_soft, const void* v_soft,
                         const int32_t* tree_parent, const int32_t* n_nodes, int32_t N, int32_t gamma,
                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * spec_verify_attn_noalloc -- spec_verify_attn without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and kernels as spec_verify_attn minus
 * (workspace, workspace_bytes).  The split-KV partials, when the schedule
 * splits (automatic, or kv_splits > 0), go to a file-scope device array of
 * SPEC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress) on the first call that needs it, on the calling
 * thread's current device, which must be the device of `stream`.  The call
 * allocates nothing (no hipMalloc / hipFree).  The scratch needs no
 * initialisation: every partial is written before it is read.
 *
 * All calls on one GPU share that array: two calls whose work overlaps on
 * the device (different streams, no ordering between them) race and give
 * unspecified results.  Calls ordered on one stream are safe.
 *
 * Errors: as spec_verify_attn; SPEC_EWORKSPACE when the call would need more
 * than SPEC_NOALLOC_SCRATCH_BYTES of partials (spec_verify_attn_workspace
 * gives the amount), checked before anything is enqueued; SPEC_EHIP when the
 * scratch's address cannot be obtained.
 */
int spec_verify_attn_noalloc(const spec_attn_desc* d, const void* q,
                             const void* k_cache, const void* v_cache, const int32_t* cache_len,
                             const void* k_blk, const void* v_blk,
                             const void* k_soft, const void* v_soft,
                             const uint32_t* mask_bits, const uint32_t* sp_bits, const int32_t* n_q,
                             void* out, float* lse, void* stream);

/*
 * spec_argmax_accept -- greedy verification of a draft tree.
 *
 * For node v < n_nodes[b] ([SS] verification step, hard matching; [LA] 2.3):
 *   out_argmax[b][v] = index of the largest logits[b][v][:] (lowest index
 *                      on ties; -0 == +0; NaN ranks after every number,
 *                      so a row of NaN only gives 0)
 *   match(v)  = draft_tok[b][v] == out_argmax[b][v]
 *   accepted(v) = match(v) and (acc_parent[b][v] == -1 or accepted(parent)),
 *                 and depth(v) <= max_depth (depth 1 for parent -1)
 *   out_len[b]  = largest depth of an accepted node, 0 if none
 *                 (the longest accepted path; [LA] 2.4 longest prefix)
 *   out_path[b][d] = node at depth d+1 on the accepted path that a
 *                 depth-first walk from the root (children in increasing
 *                 index) reaches first; -1 for d >= out_len[b].
 * Row v of logits verifies node v.  Entries out_argmax[b][v] for
 * v >= n_nodes[b] are -1.
 *
 *   logits     [B, T, V] logits_dtype, contiguous
 *   n_nodes    [B] int32, clamped to [0, T]
 *   draft_tok, acc_parent [B, T] int32.  Precondition: -1 <= acc_parent[b][v] < v.
 *   out_argmax [B, T] int32 out; out_len [B] int32 out;
 *   out_path   [B, max_depth] int32 out.
 * Limits: 1 <= T <= 256; 1 <= V < 2^31; 1 <= max_depth <= 16; B == 0 is a no-op.
 */
int spec_argmax_accept(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                       const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                       int32_t max_depth, int32_t* out_argmax, int32_t* out_len,
                       int32_t* out_path, void* stream);

/*
 * spec_argmax_accept_rows -- greedy verification with explicit verification
 * rows: the alignment of a real model's verification pass.
 *
 * In [SS]'s verification step the walk starts at the root, the previous
 * step's correction token, which is part of the flattened tree ([SS] tree
 * draft construction, step 2); the target's output at a node's position is
 * its prediction for the NEXT token, so a drafted node is checked against
 * its parent's row; and at the point where the walk stops the target's logits
 * give one correction token, so the step advances by the accepted drafts plus
 * one.  [CF] likewise hands the last accepted node's own output (its future
 * prediction) to the next round.  This call takes that alignment as data:
 * For node v < n_nodes[b]:
 *   out_argmax[b][v] as in spec_argmax_accept (row v's greedy token)
 *   u = verify_row[b][v]
 *   match(v) = (u == -1)            node v is accepted unchecked (an explicit,
 *                                   already accepted root)
 *           or (0 <= u < n_nodes[b] and draft_tok[b][v] == out_argmax[b][u]);
 *              any other u never matches
 *   accepted, depth, out_len, out_path exactly as in spec_argmax_accept
 *   out_bonus[b] = out_argmax[b][out_path[b][out_len[b] - 1]], the greedy
 *                  token of the last accepted node's row (the correction
 *                  token); -1 when out_len[b] == 0.
 * With the root in the block (verify_row -1, parent -1) and every other node
 * verified by its parent's row, out_len[b] = beta + 1 counts the root: the
 * path is exactly the set of rows whose K/V spec_commit_kv appends, and the
 * step advances by out_len[b] tokens (beta drafts + the correction token).
 * verify_row == NULL means verify_row[b][v] = v, i.e. spec_argmax_accept;
 * out_bonus may be NULL.
 *
 *   verify_row [B, T] int32 or NULL; out_bonus [B] int32 out or NULL;
 *   every other argument as in spec_argmax_accept.
 * Limits and errors as in spec_argmax_accept.
 */
int spec_argmax_accept_rows(const void* logits, int32_t logits_dtype, int32_t B, int32_t T, int32_t V,
                            const int32_t* n_nodes, const int32_t* draft_tok, const int32_t* acc_parent,
                            const int32_t* verify_row, int32_t max_depth, int32_t* out_argmax,
                            int32_t* out_len, int32_t* out_path, int32_t* out_bonus, void* stream);

/*
 * spec_commit_kv -- keep the accepted tokens' K/V ([SS] lazy garbage
 * collection after the step; [LA] 3.2: callers of the lookahead form commit
 * nothing, since lookahead K/V is dropped after the pass).
 *
 * For request b with L = cache_len_in[b] and A = out_len[b]:
 *   for d < A with L + d < lmax:
 *     cache[b, L + d, :, :] = blk[b, out_path[b][d], :, :]   (K and V)
 *   cache_len_out[b] = L + (number of rows written).
 * Every other cache row is left untouched.  Node v is block row v.
 *
 *   d          the descriptor used for spec_verify_attn (B, Tq, Hkv, D,
 *              dtype, lmax and strides are used)
 *   k_cache, v_cache  in/out caches
 *   cache_len_in [B] int32; cache_len_out [B] int32 out (may alias
 *              cache_len_in for an in-place update)
 *   k_blk, v_blk [B, Tq, Hkv, D]
 *   out_len [B], out_path [B, max_depth] as produced by spec_argmax_accept.
 *              Path entries outside [0, Tq) are skipped.
 * Limits: 1 <= max_depth <= 16.  B == 0 is a no-op.
 */
int spec_commit_kv(const spec_attn_desc* d, void* k_cache, void* v_cache,
                   const int32_t* cache_len_in, int32_t* cache_len_out,
                   const void* k_blk, const void* v_blk,
                   const int32_t* out_len, const int32_t* out_path, int32_t max_depth,
                   void* stream);

/*
 * spec_argmax_accept_commit -- spec_argmax_accept_rows followed by
 * spec_commit_kv of the accepted path, in two launches instead of three (the
 * acceptance scan's workgroup copies its request's rows as soon as its path
 * is known).  Same arguments, meanings and results as those two calls, with
 * B taken from the descriptor; block row v holds node v (T <= d->Tq).
 */
int spec_argmax_accept_commit(const void* logits, int32_t logits_dtype, int32_t T, int32_t V, const int32_t* n_nodes,
                              const int32_t* draft_tok, const int32_t* acc_parent, const int32_t* verify_row,
                              int32_t max_depth, int32_t* out_argmax, int32_t* out_len, int32_t* out_path,
                              int32_t* out_bonus, const spec_attn_desc* d, void* k_cache, void* v_cache,
                              const int32_t* cache_len_in, int32_t* cache_len_out, const void* k_blk,
                              const void* v_blk, void* stream);

/* Static description of a status code. */
const char* spec_strerror(int status);

/* Thread-local detail of the last failure in this thread ("" if none). */
const char* spec_last_error(void);

/* Library version as "major.minor.patch". */
const char* spec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
