/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash drafter hot path.
 *
 * Three operations make up one speculative-decoding cycle of a block-diffusion drafter with KV injection:
 *
 *   dflash_inject_ctx   fuse the target model's hidden states of newly committed tokens and write them as
 *                       extra K/V into every drafter layer's paged cache
 *                       ("DFlash: Block Diffusion for Flash Speculative Decoding", paper-graph summary,
 *                        section 3.4.3, "Feature fusion" and "What KV injection means operationally";
 *                        section 3.2, step 5: features are refreshed after every verification);
 *   dflash_draft_block  one parallel drafter pass over the block [anchor, mask x (L-1)] of each request,
 *                       returning per-position greedy tokens and top-k log-probabilities
 *                       (same page, section 3.4.4 "Input structure", "Attention pattern", "Single forward
 *                        pass prediction"; "Accelerating Speculative Decoding with Block Diffusion Draft
 *                        Trees", paper-graph summary, section 3.4.2: per-position marginals softmax(l_i));
 *   dflash_accept_len   greedy acceptance: accepted drafts up to the first mismatch, plus the bonus token
 *                       (DFlash page, section 3.4.1, the bonus-token paragraph under Eq. 1).
 *   dflash_draft_block_sample, dflash_verify_sample
 *                       the same pass and its verification at temperature 1 (section 3.4.4 "Single forward
 *                       pass prediction" and "Integration with verification").
 *   dflash_topk_logprobs, dflash_ddtree_build, dflash_ddtree_walk, dflash_tree_attention
 *                       DDTree on the drafter's marginals and the tree attention that verifies its trees
 *                       ("Accelerating Speculative Decoding with Block Diffusion Draft Trees", §3.4.4-§3.4.5).
 *
 * Conventions
 *   - Every pointer marked "device" is GPU memory owned by the caller; the library never allocates, frees
 *     or keeps device memory between calls, except the static scratch of dflash_draft_block_noalloc.  Host structs are read during the call only (the handle keeps
 *     a copy of the config and of the weight pointers).
 *   - Matrices are row-major [out, in] ("W[n][k]"), bfloat16 (DFLASH_BF16) or float32 (DFLASH_F32).
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream) and never
 *     synchronise.  They are safe to capture into a HIP graph (no memset or allocation is enqueued).
 *   - Arguments are validated before anything is enqueued; on error nothing runs and a negative status is
 *     returned, with a message available from dflash_last_error() on the calling thread.
 *   - Device-side checks (page ids, positions, token ids) cannot fail the call; a kernel that meets a bad
 *     value skips the access and ORs a flag into the 32-bit error word at the start of the workspace
 *     (DFLASH_DEVERR_*).  Each call clears that word first.  Read it after synchronising.
 *   - One handle per stream: calls on one handle must not overlap.
 *
 * Numerics (bfloat16 drafters): weights, input features and the cached K/V are bfloat16; the cached K/V
 * are rounded to bfloat16 (nearest, ties to even) once, when injected.  GEMMs accumulate in float32 and
 * the residual stream is float32.  Every other tensor the pass keeps between kernels (fused feature f,
 * normalised activations, q/k/v after RoPE, attention output, SwiGLU output, final normalised state) is
 * transient and keeps about float32 precision: it is stored as two bfloat16 planes, hi = bf16(v) and
 * lo = bf16(v - hi) (relative error <= 2^-17), and each plane meets the bfloat16 weights in its own MFMA.
 * Attention probabilities enter the PV product as such a pair too.  Logits are float32 and never written
 * to memory except through the optional debug tap.  Float32 drafters compute and store float32 throughout.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------------------- */
#define DFLASH_OK 0
#define DFLASH_E_ARG (-1)         /* null pointer, negative or zero size, inconsistent sizes            */
#define DFLASH_E_SHAPE (-2)       /* config fields inconsistent with each other                          */
#define DFLASH_E_CAPACITY (-3)    /* workspace smaller than dflash_*_workspace_bytes() for the call     */
#define DFLASH_E_UNSUPPORTED (-4) /* a shape outside what the kernels implement (see dflash_create)       */
#define DFLASH_E_HIP (-5)         /* a HIP runtime call failed (launch error, bad stream)                */

/* ---- device error word flags (first 4 bytes of the workspace) -------------------------------------- */
#define DFLASH_DEVERR_PAGE 1u     /* a page-table entry was outside [0, n_pages): access skipped           */
#define DFLASH_DEVERR_POS 2u      /* a position fell beyond max_pages * page_size, or ctx_len > max_ctx    */
#define DFLASH_DEVERR_TOKEN 4u    /* a block token id outside [0, vocab): embedding row 0 used instead    */
#define DFLASH_DEVERR_ROWS 8u     /* inject row offsets not non-decreasing within [0, n_rows]              */
#define DFLASH_DEVERR_TREE 16u    /* a tree parent link not pointing to an earlier token, or depth > 62   */

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  Block row i of a request with ctx_len C sits at position C + i; context token j sits at
 * position j.  rope_theta == 0 switches rotary embedding off (identity).                                  */
typedef struct {
    int n_layers;       /* drafter transformer layers (>= 1)                                               */
    int hidden;         /* drafter hidden size H = width of the fused feature                              */
    int n_q_heads;      /* query heads                                                                      */
    int n_kv_heads;     /* key/value heads; n_q_heads % n_kv_heads == 0 (grouped-query attention)           */
    int head_dim;       /* d: bf16 needs 64 or 128; f32 allows even d <= 128                                */
    int ffn;            /* SwiGLU width                                                                     */
    int vocab;          /* V of the shared embedding and LM head                                            */
    int feat_dim;       /* width of the concatenated target hidden states (n_feature_layers * H_target)     */
    int block_len;      /* L: anchor + L-1 masks, 2 <= L <= 16                                              */
    int page_size;      /* tokens per KV page; must be 16                                                   */
    float rms_eps;      /* RMSNorm epsilon                                                                  */
    float rope_theta;   /* rotary base; 0 = off                                                             */
    int dtype;          /* dflash_dtype of weights, features, cache and activations                         */
} dflash_config;

/* Per-layer weights (device pointers, row-major [out, in]).                                               */
typedef struct {
    const void *attn_norm;  /* [H] RMSNorm gain before attention                                           */
    const void *wq;         /* [n_q*d, H]                                                                   */
    const void *wk;         /* [n_kv*d, H]                                                                  */
    const void *wv;         /* [n_kv*d, H]                                                                  */
    const void *wo;         /* [H, n_q*d]                                                                   */
    const void *uk;         /* [n_kv*d, H] context-key projection of the fused feature (may alias wk)       */
    const void *uv;         /* [n_kv*d, H] context-value projection (may alias wv)                          */
    const void *ffn_norm;   /* [H]                                                                          */
    const void *w_gate;     /* [ffn, H]                                                                     */
    const void *w_up;       /* [ffn, H]                                                                     */
    const void *w_down;     /* [H, ffn]                                                                     */
} dflash_layer_weights;

typedef struct {
    const void *fc_w;       /* [H, feat_dim] feature-fusion projection                                     */
    const void *fc_b;       /* [H] or NULL (zero bias)                                                      */
    const void *embed;      /* [V, H] shared, frozen token embedding                                        */
    const void *final_norm; /* [H]                                                                          */
    const void *lm_head;    /* [V, H] shared, frozen LM head                                                */
    const dflash_layer_weights *layers; /* host array [n_layers]                                            */
} dflash_weights;

/* Paged KV pool (device).  Layout, in elements of the config dtype:
 *   k: [n_layers][n_pages][n_kv][page_size][head_dim]   (a page holds 16 consecutive keys)
 *   v: [n_layers][n_pages][n_kv][head_dim][page_size]   (values stored transposed within the page)
 * Position p of request r lives in page page_table[r * max_pages + p / 16], slot p % 16.                   */
typedef struct {
    void *k;
    void *v;
    int n_pages;
} dflash_kv;

/* Optional test taps (device pointers, float32; NULL = off).                                              */
typedef struct {
    float *logits;  /* [batch][L][V] full logits (tests; the input of the DDTree wide top-K below)         */
    float *hidden;  /* [n_layers + 1][batch * L][H] residual stream after the embedding and each layer       */
} dflash_debug;

typedef struct dflash_handle dflash_handle;

/* Create a handle for a drafter.  Validates the config (no HIP call is made).  Supported: dtype BF16 with
 * head_dim 64 or 128, hidden/ffn/feat_dim/n_q*d multiples of 256; dtype F32 with even head_dim <= 128 and
 * hidden/ffn/feat_dim/n_q*d multiples of 4; 2 <= L <= 16; page_size 16; n_q/n_kv <= 8.
 * Returns DFLASH_OK and *out, or an error status (and *out = NULL).                                       */
int dflash_create(const dflash_config *cfg, const dflash_weights *w, dflash_handle **out);
void dflash_destroy(dflash_handle *h);

/* Packed weight store.  A BF16 handle streams every projection matrix (wq, wk, wv, wo, w_gate, w_up,
 * w_down, uk, uv of each layer, fc_w, lm_head) from a copy in MFMA fragment order: 16 rows x 32 k-values
 * per 1 KB fragment, in the order one 64-lane wave reads them, so that each weight load of the
 * weight-streaming GEMMs is one coalesced 1 KB access.  This is a re-layout only (the values are the
 * row-major matrices' bits), made once per handle.
 * dflash_packed_weight_bytes: bytes the store needs (0 for F32 handles, which read the row-major matrices).
 * dflash_pack_weights: enqueues the repacking on `stream` into dst (device memory the caller owns, 256-byte
 * aligned, at least dflash_packed_weight_bytes(h) bytes, kept allocated while the handle is used); the
 * handle reads dst from then on, and the row-major projection matrices are not read again (embed, the
 * norm gains and fc_b still are).  Must be called before dflash_draft_block / dflash_inject_ctx on a BF16
 * handle (they return DFLASH_E_ARG otherwise).  Every matrix must be 16-byte aligned.  F32 handles: no-op. */
size_t dflash_packed_weight_bytes(const dflash_handle *h);
int dflash_pack_weights(dflash_handle *h, void *dst, size_t dst_bytes, void *stream);

/* Workspace bytes for dflash_draft_block with batch <= max_batch, context lengths <= max_ctx and
 * top_k <= 8.  Returns 0 on invalid arguments.                                                           */
size_t dflash_draft_workspace_bytes(const dflash_handle *h, int max_batch, int max_ctx);

/* Workspace bytes for dflash_inject_ctx with n_rows <= max_rows.  Returns 0 on invalid arguments.         */
size_t dflash_inject_workspace_bytes(const dflash_handle *h, int max_rows);

/* Append context tokens.  For request r, feature rows row_offsets[r] .. row_offsets[r+1]-1 of `feats` are
 * fused (f = W_fc x + b) and projected per layer into K = RoPE(U_K f) at positions start_pos[r] + j and
 * V = U_V f, which are stored in the pages named by page_table.  Rows >= row_offsets[batch] are computed
 * but not stored.  Rows of different requests are independent, so any row split gives the same cache.
 *   feats          device [n_rows][feat_dim], row stride feat_row_stride elements (>= feat_dim)
 *   row_offsets    device int32 [batch + 1]
 *   start_pos      device int32 [batch]
 *   page_table     device int32 [batch][max_pages]
 *   ws, ws_bytes   device workspace of at least dflash_inject_workspace_bytes(h, n_rows) bytes           */
int dflash_inject_ctx(dflash_handle *h, int batch, int n_rows, const void *feats, int64_t feat_row_stride,
                      const int32_t *row_offsets, const int32_t *start_pos, const int32_t *page_table,
                      int max_pages, const dflash_kv *kv, void *ws, size_t ws_bytes, void *stream);

/* One drafter pass per request over block_tokens (anchor, then mask ids) against that request's first
 * ctx_len[r] cached context tokens.  Attention is non-causal over [context ; block].
 *   block_tokens   device int32 [batch][L]
 *   ctx_len        device int32 [batch], each in [0, max_ctx]
 *   page_table     device int32 [batch][max_pages]
 *   max_ctx        host upper bound of ctx_len (sizes the split of the context across workgroups)
 *   top_k          0..8
 *   tokens         device int32 [batch][L]: greedy argmax per row (ties -> smaller id); the drafts are
 *                  rows 1..L-1
 *   topk_ids       device int32 [batch][L][top_k] ordered by (logit desc, id asc); NULL if top_k == 0
 *   topk_logprobs  device float [batch][L][top_k]: logit - logsumexp over the full vocabulary
 *   dbg            host struct of optional taps, or NULL
 *   ws, ws_bytes   at least dflash_draft_workspace_bytes(h, batch, max_ctx) bytes                       */
int dflash_draft_block(dflash_handle *h, int batch, const int32_t *block_tokens, const int32_t *ctx_len,
                       const int32_t *page_table, int max_pages, const dflash_kv *kv, int max_ctx, int top_k,
                       int32_t *tokens, int32_t *topk_ids, float *topk_logprobs, const dflash_debug *dbg,
                       void *ws, size_t ws_bytes, void *stream);

/* Allocation-free variant of dflash_draft_block, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same pass, arguments (less the
 * workspace) and results.  The workspace is a static device array of DFLASH_NOALLOC_SCRATCH_BYTES inside the
 * library, which each GPU the library runs on holds from the code object's load until the process ends; the
 * first call on a device looks up its address there (no allocation).  A call whose
 * dflash_draft_workspace_bytes(h, batch, max_ctx) exceeds the array returns DFLASH_E_CAPACITY before anything
 * runs (every batch-1 pass of the 4B- and 8B-sized drafters fits, at any context length).  Every call on one
 * GPU uses that GPU's one array, which keeps the last call's contents (the pass writes every byte it reads):
 * calls that overlap on one GPU -- on several streams, threads or handles -- race and give undefined results.
 * The device error word of this variant lives in the array and is not reported; dflash_draft_block reports
 * it.                                                                                                      */
#define DFLASH_NOALLOC_SCRATCH_BYTES (32u << 20)
int dflash_draft_block_noalloc(dflash_handle *h, int batch, const int32_t *block_tokens, const int32_t *ctx_len,
                               const int32_t *page_table, int max_pages, const dflash_kv *kv, int max_ctx,
                               int top_k, int32_t *tokens, int32_t *topk_ids, float *topk_logprobs,
                               const dflash_debug *dbg, void *stream);

/* tau[r] = 1 + the number of leading j < n_draft with draft[r*draft_stride + j] == target[r*target_stride
 * + j]; tau lies in [1, n_draft + 1].  Typical call: draft = tokens + 1 with stride L, n_draft = L - 1.
 * All arrays are device int32.  No workspace is used.                                                     */
int dflash_accept_len(int batch, int n_draft, const int32_t *draft, int64_t draft_stride, const int32_t *target,
                      int64_t target_stride, int32_t *tau, void *stream);

/* ---- Temperature 1 (DFlash page, section 3.4.4: "Single forward pass prediction" samples each row from the
 * softmax of its logits, "Integration with verification" verifies by standard speculative decoding) --------
 * Random draws come from Philox4x32-10 (Salmon et al., SC 2011), counter-based: the word for (tag, row, j)
 * under a 64-bit seed is word j % 4 of the block at counter (j / 4, row, tag, 0), key (seed & 0xffffffff,
 * seed >> 32); a word c is the uniform u = (c + 1/2) / 2^32 and the Gumbel variable -ln(-ln(1 - u)).  Use a
 * fresh seed per cycle.                                                                                   */

/* As dflash_draft_block, but each row's token is sampled from softmax(logits) by the Gumbel-max rule:
 * tokens[r][i] = argmax_j logit_j + G_j (ties -> smaller id), G from stream tag 1, row r * L + i, j = token
 * id.  top-k outputs are unchanged (by logit).  logits: device float [batch][L][V] full logits, or NULL;
 * dflash_verify_sample needs them (the drafter rows of the drafts are rows 1 .. L-1).  Same workspace as
 * dflash_draft_block.                                                                                     */
int dflash_draft_block_sample(dflash_handle *h, int batch, const int32_t *block_tokens, const int32_t *ctx_len,
                              const int32_t *page_table, int max_pages, const dflash_kv *kv, int max_ctx, int top_k,
                              uint64_t seed, int32_t *tokens, int32_t *topk_ids, float *topk_logprobs, float *logits,
                              void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for dflash_verify_sample (0 on invalid arguments).                                      */
size_t dflash_verify_sample_workspace_bytes(int batch, int n_draft, int vocab);

/* Verification at temperature 1 by modified rejection sampling (Leviathan, Kalman and Matias, ICML 2023,
 * Algorithm 1).  For request r, with p_j = softmax of target row j and q_j = softmax of drafter row j:
 * draft j (in order, j < n_draft) is kept iff ln u_j < ln p_j(y_j) - ln q_j(y_j), u_j from stream tag 2,
 * row r, index j; a draft id outside [0, vocab) is rejected.  At the first rejection k the next token is a
 * Gumbel-max sample (tag 3, row r, j = token id) from max(0, p_k - q_k), or from p_k where that vanishes;
 * if all drafts are kept, from p_{n_draft} (the bonus row).  tau[r] = kept + 1, next_token[r] = the token.
 *   draft        device int32, draft[r * draft_stride + j]; typical: sampled tokens + 1, stride L
 *   q_logits     device float, drafter row j of request r at q_logits + r * q_req_stride + j * vocab
 *                (typical: dflash_draft_block_sample's logits + vocab, stride L * vocab); NULL if n_draft == 0
 *   p_logits     device float, target row j (0 .. n_draft) of request r at p_logits + r * p_req_stride +
 *                j * vocab: row j is the target's distribution after the block prefix ending in draft j - 1
 *   Every row needs a finite entry.  0 <= n_draft <= 63, 1 <= batch <= 65535.  ws: 256-byte aligned, at least
 *   dflash_verify_sample_workspace_bytes(batch, n_draft, vocab) bytes.                                    */
int dflash_verify_sample(int batch, int n_draft, int vocab, const int32_t *draft, int64_t draft_stride,
                         const float *q_logits, int64_t q_req_stride, const float *p_logits, int64_t p_req_stride,
                         uint64_t seed, int32_t *tau, int32_t *next_token, void *ws, size_t ws_bytes, void *stream);

/* ---- DDTree on the drafter's marginals ("Accelerating Speculative Decoding with Block Diffusion Draft
 * Trees", §3.4.4 Lemma 1 and Algorithm 1, §3.4.5 the verifier walk) --------------------------------------
 * The drafter's full logits come from dflash_draft_block's dbg->logits output ([batch][L][V]); block row d
 * (1 .. L-1) is the distribution of draft depth d.                                                        */

/* The k best tokens of each of `rows` logit rows (device float, row stride row_stride >= vocab), ordered by
 * (logit descending, id ascending), and their log-probabilities logit - logsumexp(row) ([DDT] §3.4.4
 * Lemma 1: only each depth's top K can enter the tree).  Outputs are device [rows][k] int32 ids and float
 * log-probs.  1 <= k <= min(vocab, 1024).  With few rows each row is split over several workgroups whose
 * partial results go through `workspace` (device, 16-byte aligned, at least
 * dflash_topk_logprobs_workspace_bytes(rows, vocab, k) bytes; NULL allowed when that is 0).                */
size_t dflash_topk_logprobs_workspace_bytes(int rows, int vocab, int k);
int dflash_topk_logprobs(int rows, int vocab, int k, const float *logits, int64_t row_stride, int32_t *ids,
                         float *logprobs, void *workspace, size_t workspace_bytes, void *stream);

/* Algorithm 1 per request: the `budget` most probable prefixes under the factorised distribution, in the
 * order a best-first heap of rank tuples pops them (next sibling and first child pushed per pop; equal
 * scores pop in creation order).  Input: depth d (0-based, d < depth) of request r has its k sorted
 * log-probs and ids at logprobs / ids + r * req_stride + d * k (device).  Output, device [batch][budget],
 * node i = the i-th pop: node_token (token id), node_parent (node index of its prefix, -1 = the root / bonus
 * token), node_depth (1-based), node_logq (log-probability score, float32 sums: parent's score + own
 * log-prob); n_nodes[b] = nodes written (min(budget, prefixes available)).  depth <= 16, k <= 1024,
 * budget <= 2047.  The tree is found by a parallel selection of the top-`budget` prefixes (Proposition 2 of
 * §3.4.3) followed by a sort into pop order; a request the selection cannot decide (rows that are not
 * non-increasing log-probabilities <= 0, long runs of exactly equal scores) is built by the heap itself.
 * Both give the heap's result.  No workspace.                                                              */
int dflash_ddtree_build(int batch, int depth, int k, const float *logprobs, const int32_t *ids, int64_t req_stride,
                        int budget, int32_t *node_token, int32_t *node_parent, int32_t *node_depth,
                        float *node_logq, int32_t *n_nodes, void *stream);

/* The parallel selection of dflash_ddtree_build alone, for callers that want to see which requests it
 * decides: same arguments and outputs, except that n_nodes[b] = -1 marks a request it left undecided (its
 * other outputs are then unspecified).                                                                    */
int dflash_ddtree_select(int batch, int depth, int k, const float *logprobs, const int32_t *ids, int64_t req_stride,
                         int budget, int32_t *node_token, int32_t *node_parent, int32_t *node_depth,
                         float *node_logq, int32_t *n_nodes, void *stream);

/* Greedy verifier walk per request over a tree from dflash_ddtree_build: target_next[b][0] is the target's
 * choice after the root and target_next[b][i + 1] its choice after node i (device [batch][budget + 1]).
 * From the root, move to the child holding the target's choice while there is one.  Outputs (device):
 * accept_len[b] = nodes accepted (<= max_accept), accept_nodes[b][0 .. accept_len) their indices,
 * bonus[b] = the target's choice where the walk stopped.  budget <= 2047.                                 */
int dflash_ddtree_walk(int batch, int budget, int max_accept, const int32_t *node_token, const int32_t *node_parent,
                       const int32_t *n_nodes, const int32_t *target_next, int32_t *accept_len,
                       int32_t *accept_nodes, int32_t *bonus, void *stream);

/* ---- Tree attention (the verification side of DDTree: "Accelerating Speculative Decoding with Block
 * Diffusion Draft Trees", §3.4.5 "Verification: Tree Attention and the Verifier Walk") ---------------------
 * One attention layer of a target model over a flattened draft tree.  Tree token 0 is the root (the bonus
 * token); token i > 0 is a tree node whose parent token parent[i] precedes it (0 <= parent[i] < i), as in
 * the pop order of dflash_ddtree_build (token i = node i - 1, parent token = node_parent + 1).  A token's
 * position id is its depth (root 0), i.e. absolute position ctx_len + depth.  Each token attends to every
 * cached context key and, in the tree, only to its ancestors and itself.
 *   n_tokens     device int32 [batch]: tree tokens of each request (root included), <= max_tokens; later
 *                rows are neither read nor written
 *   parent       device int32 [batch][max_tokens]; parent[0] is ignored; depth <= 62
 *   q            device bfloat16 [batch][max_tokens][n_q_heads][128], before RoPE
 *   k, v         device bfloat16 [batch][max_tokens][n_kv_heads][128], k before RoPE
 *   k_pages      device bfloat16 [n_pages][n_kv_heads][16][128]: one layer's cached context keys (rotated
 *                at their own positions); v_pages [n_pages][n_kv_heads][128][16] (values transposed per page)
 *   page_table   device int32 [batch][max_pages]; position p of request r in page page_table[r][p / 16],
 *                slot p % 16
 *   ctx_len      device int32 [batch], each <= max_ctx (host bound; 0 = no context)
 *   rope_theta   rotary base (0: no rotation); q and k are rotated in float32 and rounded to bfloat16
 *   out          device bfloat16 [batch][max_tokens][n_q_heads][128]
 * Query head h reads KV head h / (n_q_heads / n_kv_heads); that ratio is 1, 2, 4 or 8; head_dim 128;
 * max_tokens <= 2048; batch * ceil(max_tokens / 16) * (ceil(max_ctx / 64) + 64) < 2^31 (else
 * DFLASH_E_UNSUPPORTED).  q, k, v, out and the pages 16-byte aligned; ws 256-byte aligned, at least
 * dflash_tree_attention_workspace_bytes(...) bytes; its first 4 bytes are the device error word
 * (DFLASH_DEVERR_PAGE / _POS / _TREE), cleared by every call.                                             */
size_t dflash_tree_attention_workspace_bytes(int batch, int max_tokens, int n_q_heads, int n_kv_heads,
                                             int head_dim, int max_ctx);
int dflash_tree_attention(int batch, int max_tokens, const int32_t *n_tokens, const int32_t *parent,
                          int n_q_heads, int n_kv_heads, int head_dim, const void *q, const void *k, const void *v,
                          const void *k_pages, const void *v_pages, int n_pages, const int32_t *page_table,
                          int max_pages, const int32_t *ctx_len, int max_ctx, float rope_theta, void *out, void *ws,
                          size_t ws_bytes, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none).                                */
const char *dflash_last_error(void);

/* ---- building blocks (tests, measurement) ----------------------------------------------------------- */

/* y[m][n] = sum_k x[m][k] * w[n][k] for m < M, n < N, with float32 output (row stride N).  x is [M][K]
 * (row stride ldx elements) and w [N][K] row-major, both of `dtype`, 16-byte aligned.  Uses the same GEMM
 * kernels as the drafter pass (BF16: w is first packed into the workspace).  ws (16-byte aligned) must hold
 * dflash_linear_workspace_bytes(dtype, M, N, K) bytes.                                                     */
size_t dflash_linear_workspace_bytes(int dtype, int M, int N, int K);
int dflash_linear(int dtype, int M, int N, int K, const void *x, int64_t ldx, const void *w, float *y, void *ws,
                  size_t ws_bytes, void *stream);

/* Stream copy of n_bytes (multiple of 16, 16-byte aligned pointers) for measuring HBM bandwidth.           */
int dflash_copy(void *dst, const void *src, size_t n_bytes, void *stream);

/* Per-kernel timing.  When enabled, every kernel a handle launches is bracketed by HIP events.
 * dflash_profile_collect synchronises those events, fills up to max_entries records (kernel name, number
 * of launches, total milliseconds) accumulated since the last collect, and returns the number written.   */
typedef struct {
    char name[48];
    int launches;
    double total_ms;
} dflash_kernel_stat;
int dflash_profile_enable(dflash_handle *h, int on);
int dflash_profile_collect(dflash_handle *h, dflash_kernel_stat *out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
