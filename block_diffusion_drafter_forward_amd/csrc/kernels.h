// Host-side launchers of the gfx950 kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace df {

// Per-kernel timing (the library's profiling mode): the host layer points df_launch_timing at a pair of
// events around one launch; a launcher that supports it hands them to hipExtLaunchKernelGGL, which records
// the kernel's own start and end (without the dispatch latency an event pair around the launch also
// measures), and marks them used.  Launchers without it leave the events to the host layer's records.
struct LaunchTiming {
    hipEvent_t start, stop;
    bool used;
};
extern thread_local LaunchTiming* df_launch_timing;
#define DF_LAUNCH(kernel, grid, block, shmem, st, ...)                                                     \
    do {                                                                                                   \
        LaunchTiming* lt_ = df_launch_timing;                                                              \
        if (lt_ && !lt_->used) {                                                                           \
            lt_->used = true;                                                                              \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, lt_->start, lt_->stop, 0, __VA_ARGS__);  \
        } else {                                                                                           \
            hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);                               \
        }                                                                                                  \
    } while (0)

// ---- allocation-free scratch -------------------------------------------------------------------------------
// The calling device's copy of the library's static scratch (DFLASH_NOALLOC_SCRATCH_BYTES): its device address
// and size.  The first call on a device looks the address up (no allocation); later calls reuse it.
hipError_t scratch_region(void** ptr, size_t* bytes);

// ---- GEMM ------------------------------------------------------------------------------------------------
enum GemmKind { GEMM_SKINNY1 = 0, GEMM_SKINNY2 = 1, GEMM_TILED = 2, GEMM_F32 = 3 };
struct GemmPlan {
    int kind;
    int splits;  // number of float32 partial products written (grid split of K)
    int kpw;     // skinny: k-range per wave (multiple of 256)
    int waves;   // skinny: waves per workgroup (4 or 8)
    int kps;     // tiled: k-range per split (multiple of 64)
    int nt;      // tiled: n-tiles of 16 per wave (8: 256-wide workgroup tiles, 6: 192-wide)
};
// few_splits: prefer fewer, longer k-ranges per wave (set for the drafter layer's GEMMs, where it was measured
// to pay off through cheaper split-K consumers).
GemmPlan plan_gemm(int dtype_bf16, int M, int N, int K, bool few_splits = false);
// Packs the N x K bfloat16 matrix stacked from the row segments of src (row-major rows, K a multiple of 256)
// into the chunk-major fragment layout of gemm_core.h at dst.
hipError_t launch_pack(const Segs& src, int N, int K, void* dst, hipStream_t st);
// bfloat16: wpacked is the packed N x K matrix.  xplane != 0: x is an activation pair of bfloat16 planes
// (lo plane xplane elements after hi).
hipError_t launch_gemm_bf16(const GemmPlan& p, const void* x, int ldx, size_t xplane, int M, const void* wpacked,
                            int N, int K, float* part, hipStream_t st);
// float32: row-major weight segments.
hipError_t launch_gemm_f32(const float* x, int ldx, int M, const Segs& w, int N, int K, float* part, hipStream_t st);
const char* gemm_kernel_name(const GemmPlan& p, bool pair);

// ---- row-wise kernels ------------------------------------------------------------------------------------
// h = embed[tok]; u = RMSNorm(h) * g.  Also clears the device error word (block 0).
hipError_t launch_embed_norm(int bf16, const int32_t* tok, int M, int V, const void* embed, const void* gain, int H,
                             float eps, float* h, void* u, float* tap, uint32_t* err, hipStream_t st);
// h += sum_s part[s]; u = RMSNorm(h) * g.
hipError_t launch_resid_norm(int bf16, const float* part, int S, int M, int H, float* h, const void* gain, float eps,
                             void* u, float* tap, hipStream_t st);
// q/k/v from the QKV partials: RoPE at ctx_len[b] + i, rounding, block K [B][n_kv][16][d] and V^T
// [B][n_kv][d][16] layouts.
hipError_t launch_qkv_epilogue(int bf16, const float* part, int S, int B, int L, int nq, int nkv, int d,
                               const int32_t* ctx_len, const RopeFreq& rf, void* q, void* kb, void* vbt,
                               hipStream_t st);
// a = silu(sum_s gate) * (sum_s up); partial columns [0, F) are gate, [F, 2F) up.
hipError_t launch_swiglu(int bf16, const float* part, int S, int M, int F, void* a, hipStream_t st);
// out[m][n] = round(sum_s part[s][m][n] + bias[n]).
hipError_t launch_reduce_cast(int bf16, const float* part, int S, int M, int N, const void* bias, void* out,
                              uint32_t* clear_err, hipStream_t st);
// Context K/V from the stacked [U_K^0; U_V^0; U_K^1; ...] partials, RoPE at each row's position, scatter into
// the paged pool.  row0 = index of the first row of this chunk among all n_rows rows.
// Columns of part cover layers layer0 .. layer0 + nl - 1.
hipError_t launch_kv_scatter(int bf16, const float* part, int S, int rows, int row0, int layer0, int nl, int nkv,
                             int d, int batch, const int32_t* row_offsets, const int32_t* start_pos,
                             const int32_t* page_table, int max_pages, int n_pages, void* kpool, void* vpool,
                             const RopeFreq& rf, uint32_t* err, hipStream_t st);
hipError_t launch_clear_err(uint32_t* err, hipStream_t st);
hipError_t launch_accept(int batch, int n_draft, const int32_t* draft, int64_t ds, const int32_t* target, int64_t ts,
                         int32_t* tau, hipStream_t st);
hipError_t launch_copy(void* dst, const void* src, size_t n16, hipStream_t st);

// ---- attention -------------------------------------------------------------------------------------------
struct AttnPlan {
    int n_chunks;      // context chunks (chunk 0 also takes the block's own keys)
    int chunk_tokens;  // multiple of the kernel's staging round (64 or 128 keys)
    int stream_kv;     // cached K/V read with non-temporal loads (the pass's K/V exceed half the Infinity Cache)
};
// workgroups (and partial slots) per (request, KV head): one per chunk, one without context
inline int attn_slots(const AttnPlan& p) { return p.n_chunks > 0 ? p.n_chunks : 1; }
AttnPlan plan_attention(int batch, int n_q, int n_kv, int max_ctx, int n_layers);
hipError_t launch_attention(int bf16, const AttnPlan& p, int B, int L, int nq, int nkv, int d, const void* q,
                            const void* kb, const void* vbt, const void* kpool, const void* vpool, int layer,
                            int n_pages, const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                            int max_ctx, float* opart, float* mlpart, uint32_t* err, hipStream_t st);
hipError_t launch_attn_merge(int bf16, const AttnPlan& p, int B, int L, int nq, int d, const float* opart,
                             const float* mlpart, void* o, hipStream_t st);

// ---- LM head ---------------------------------------------------------------------------------------------
int head_group_width(int bf16, int M);  // vocabulary columns per record group (64 or 128)
int head_groups(int V, int width);
size_t head_partial_floats(int bf16, int V, int M);
// bfloat16: wlm is the packed V x K matrix; float32: row-major.
// sample != 0: temperature 1, each row's token is a Gumbel-max sample with draws keyed by `seed`.
hipError_t launch_lm_head(int bf16, const void* z, int M, const void* wlm, int V, int K, float* hpart,
                          float* logits_dbg, int sample, uint64_t seed, hipStream_t st);
// Also flags block tokens outside [0, V) in the device error word.
hipError_t launch_head_merge(int bf16, int M, int V, int top_k, int sample, const float* hpart,
                             const int32_t* block_tokens, int32_t* tokens, int32_t* topk_ids, float* topk_lp,
                             uint32_t* err, hipStream_t st);

// ---- DDTree ----------------------------------------------------------------------------------------------
// Per row of logits[rows][stride]: the K best (value desc, id asc) and their log-probabilities.
hipError_t launch_topk_rows(int rows, const float* logits, int64_t stride, int V, int K, int32_t* ids, float* lp,
                            void* ws, hipStream_t st);
// Workspace of launch_topk_rows (0 when each row gets one workgroup).
size_t topk_workspace_bytes(int rows, int V, int K);
// Algorithm 1 per request: depth d (0-based) of request r reads lp / ids at r * req_stride + d * K.
hipError_t launch_ddtree_build(int batch, int D, int K, const float* lp, const int32_t* ids, int64_t req_stride,
                               int budget, int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                               float* node_logq, int32_t* n_nodes, bool select_only, hipStream_t st);
hipError_t launch_ddtree_walk(int batch, int budget, int max_accept, const int32_t* node_token,
                              const int32_t* node_parent, const int32_t* n_nodes, const int32_t* target_next,
                              int32_t* accept_len, int32_t* accept_nodes, int32_t* bonus, hipStream_t st);

// ---- verification at temperature 1 -------------------------------------------------------------------
size_t sv_workspace_bytes(int B, int n_draft, int V);
// Drafter rows of request b at q + b * q_req + j * V (j < n_draft), target rows at p + b * p_req + j * V
// (j <= n_draft); n_draft < 64.
hipError_t launch_verify_sample(int batch, int n_draft, int V, const int32_t* draft, int64_t dstride, const float* q,
                                int64_t q_req, const float* p, int64_t p_req, uint64_t seed, int32_t* tau,
                                int32_t* next_token, void* ws, hipStream_t st);

// ---- tree attention -----------------------------------------------------------------------------------
#define TREE_MAX_TOKENS 2048  // tree tokens per request, root included
#define TREE_MAX_ANC 64       // per token: its depth, then the root-to-token path (depth <= 62)
// The context part is split stream-K: per KV head, the (request, super tile) units' 64-key rounds form one
// sequence, and workgroup j of that head takes rounds [j rpw, (j + 1) rpw).  Each unit segment a workgroup
// covers leaves one (m, l, O) partial in slot (workgroup - first workgroup of the unit), slots < `slots`.
// A unit's rounds past its context (padding to whole workgroups) are empty.
struct TreePlan {
    int tiles, stiles;  // 16-token tiles, workgroup super tiles
    int rpu, rpw;       // 64-key rounds per unit in the sequence (the context, maybe padded), per workgroup
    int wgs, slots;     // workgroups per KV head, partial slots per unit (0: no context)
    size_t q_off, k_off, anc_off, o_off, ml_off, total;
};
TreePlan plan_tree(int batch, int max_tokens, int nq, int nkv, int max_ctx);
// q, k, v: bfloat16 [batch][T][heads][128]; kpool / vpool: one layer's pages; out: bfloat16 [batch][T][nq][128].
hipError_t launch_tree_attention(const TreePlan& p, int batch, int T, const int32_t* n_tokens, const int32_t* parent,
                                 int nq, int nkv, const void* q, const void* k, const void* v, const void* kpool,
                                 const void* vpool, int n_pages, const int32_t* pt, int max_pages,
                                 const int32_t* ctx_len, int max_ctx, const RopeFreq& rf, void* out, void* ws,
                                 hipStream_t st);

}  // namespace df
