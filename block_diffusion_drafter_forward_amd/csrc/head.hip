// Shared LM head fused with the per-row reductions the drafter needs: running max, sum of exponentials
// (for the log-sum-exp over the full vocabulary) and the top-8 (logit, id) list, ordered by logit then id.
// Logits live only in registers and LDS.  Stage 1 (lm_head): one workgroup per 64 vocabulary rows, four
// waves splitting K, writes one (max, sumexp, top-8) record per block row.  Stage 2 (head_merge): one
// workgroup per block row merges the records in a fixed order and emits the greedy token, the top-k ids
// and their log-probabilities.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace df {

#define HEAD_REC 18  // max, sumexp, 8 values, 8 ids (as int bits)

// Vocabulary columns per record group: 64 for the skinny head (block rows <= 32), 128 for the tiled head.
int head_group_width(int bf16, int M) { return (bf16 && M > 32) ? 128 : 64; }
int head_groups(int V, int width) { return (V + width - 1) / width; }
size_t head_partial_floats(int bf16, int V, int M) {
    return (size_t)head_groups(V, head_group_width(bf16, M)) * M * HEAD_REC;
}

__device__ __forceinline__ void topk_insert(TopK& s, float x, int xid) {
    if (!df_better(x, xid, s.v[DF_TOPK - 1], s.id[DF_TOPK - 1])) return;
    float cv = x;
    int ci = xid;
#pragma unroll
    for (int j = 0; j < DF_TOPK; ++j) {
        const bool b = df_better(cv, ci, s.v[j], s.id[j]);
        const float tv = s.v[j];
        const int ti = s.id[j];
        s.v[j] = b ? cv : tv;
        s.id[j] = b ? ci : ti;
        cv = b ? tv : cv;
        ci = b ? ti : ci;
    }
}

// merge state o into s: lists by insertion (o's list is sorted, so the first candidate that does not make
// s's list ends the merge), (max, sumexp) by rescaling to the larger max
__device__ __forceinline__ void topk_merge(TopK& s, const float* ov, const int* oid, float omx, float ose) {
    bool go = true;  // fully unrolled with a predicate so that ov / oid stay in registers
#pragma unroll
    for (int j = 0; j < DF_TOPK; ++j) {
        go = go && df_better(ov[j], oid[j], s.v[DF_TOPK - 1], s.id[DF_TOPK - 1]);
        if (go) topk_insert(s, ov[j], oid[j]);
    }
    if (omx == -INFINITY) return;
    if (s.mx == -INFINITY) { s.mx = omx; s.se = ose; return; }
    const float M = fmaxf(s.mx, omx);
    s.se = s.se * expf(s.mx - M) + ose * expf(omx - M);
    s.mx = M;
}

// Row reductions over a logits tile lg[R][C] held in LDS (vocabulary columns n0 .. n0+C-1, block rows
// row0 .. row0+R-1, of which `rows` are valid).  Threads split each row into TPR pieces, then the first
// thread of the row merges the pieces and writes the record of (group, row).
template <int R, int C>
__device__ void head_epilogue(const float (*lg)[C + 1], float (*st)[HEAD_REC], int rows, int row0, int Mtot, int n0,
                              int V, int group, float* __restrict__ hpart, float* __restrict__ logits_dbg) {
    constexpr int TPR = 256 / R, CPT = C / TPR;
    const int t = threadIdx.x;
    const int m = t / TPR, c0 = (t % TPR) * CPT;
    TopK s;
    s.init();
    if (m < rows) {
        for (int c = c0; c < c0 + CPT; ++c) {
            const int v = n0 + c;
            if (v >= V) break;
            const float x = lg[m][c];
            s.push(x, v);
            if (logits_dbg) logits_dbg[(size_t)(row0 + m) * V + v] = x;
        }
    }
    st[t][0] = s.mx;
    st[t][1] = s.se;
#pragma unroll
    for (int j = 0; j < DF_TOPK; ++j) {
        st[t][2 + j] = s.v[j];
        st[t][2 + DF_TOPK + j] = __int_as_float(s.id[j]);
    }
    __syncthreads();
    if (m < rows && (t % TPR) == 0) {
        for (int q = 1; q < TPR; ++q) {
            const float* o = st[t + q];
            int oid[DF_TOPK];
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(o[2 + DF_TOPK + j]);
            topk_merge(s, o + 2, oid, o[0], o[1]);
        }
        float* dst = hpart + ((size_t)group * Mtot + row0 + m) * HEAD_REC;
        dst[0] = s.mx;
        dst[1] = s.se;
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {
            dst[2 + j] = s.v[j];
            dst[2 + DF_TOPK + j] = __int_as_float(s.id[j]);
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// bfloat16 MFMA LM head: the GEMM core of the skinny kernel with the reductions as epilogue
// ------------------------------------------------------------------------------------------------------
// W is the packed (fragment-major) V x K matrix; z is an activation pair of bfloat16 planes (lo plane at
// z + zplane): two MFMAs per weight fragment.
template <int MT>
__global__ __launch_bounds__(256) void lm_head_bf16(const bf16_t* __restrict__ z, size_t zplane, int M,
                                                    const bf16_t* __restrict__ W, int V, int K,
                                                    float* __restrict__ hpart, float* __restrict__ logits_dbg) {
    constexpr int NT = 4;
    __shared__ f32x4 red[4][NT * MT][64];
    __shared__ float lg[16 * MT][65];
    __shared__ float st[256][HEAD_REC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64;
    const int chunks = K / 256;
    const int kb = (wave * chunks / 4) * 256, ke = ((wave + 1) * chunks / 4) * 256;

    const int KS = K / 32, tiles = (V + 15) / 16;
    const bf16_t* wt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wt[nt] = W + (size_t)min(blockIdx.x * NT + nt, tiles - 1) * KS * DF_FRAG + lane * 8;
    const bf16_t* zrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) zrow[mt] = z + (size_t)min(mt * 16 + r, M - 1) * K + g * 8;

    constexpr bool SEP = MT == 1;  // separate hi / lo accumulators at one m-tile
    f32x4 acc[NT][MT], acl[SEP ? NT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (SEP) acl[SEP ? nt : 0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int kc = kb; kc < ke; kc += 256) {
        u32x4 wf[NT][8];
        u32x4 zf[MT][8], zl[MT][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wf[nt][j] = ld16_nt(wt[nt] + (size_t)(kc / 32 + j) * DF_FRAG);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                zf[mt][j] = ld16(zrow[mt] + kc + j * 32);
                zl[mt][j] = ld16(zrow[mt] + zplane + kc + j * 32);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads of the chunk in flight before the MFMAs
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[nt][mt] = mfma16(wf[nt][j], zf[mt][j], acc[nt][mt]);
                    if (SEP) acl[SEP ? nt : 0] = mfma16(wf[nt][j], zl[0][j], acl[SEP ? nt : 0]);
                    else acc[nt][mt] = mfma16(wf[nt][j], zl[mt][j], acc[nt][mt]);
                }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 v = acc[nt][mt];
            if (SEP) {
                const f32x4 u = acl[SEP ? nt : 0];
                v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
            }
            red[wave][nt * MT + mt][lane] = v;
        }
    __syncthreads();
    for (int e = threadIdx.x; e < NT * MT * 64; e += 256) {
        const int t = e >> 6, l = e & 63;
        const int nt = t / MT, mt = t % MT;
        f32x4 v = red[0][t][l];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            const f32x4 u = red[q][t][l];
            v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
        }
        const int m = mt * 16 + (l & 15);
        const int c = nt * 16 + 4 * (l >> 4);
        lg[m][c + 0] = v[0];
        lg[m][c + 1] = v[1];
        lg[m][c + 2] = v[2];
        lg[m][c + 3] = v[3];
    }
    __syncthreads();
    head_epilogue<16 * MT, 64>(lg, st, M, 0, M, n0, V, blockIdx.x, hpart, logits_dbg);
}

// ------------------------------------------------------------------------------------------------------
// float32 LM head (float32 drafters, M <= 32)
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lm_head_f32(const float* __restrict__ z, int M, const float* __restrict__ W,
                                                   int V, int K, float* __restrict__ hpart,
                                                   float* __restrict__ logits_dbg) {
    __shared__ float lg[32][65];
    __shared__ float st[256][HEAD_REC];
    const int n0 = blockIdx.x * 64;
    const int c = threadIdx.x & 63;
    const float* wr = W + (size_t)min(n0 + c, V - 1) * K;
    for (int m = threadIdx.x >> 6; m < 32; m += 4) {
        float a = 0.f;
        if (m < M) {
            const float* zr = z + (size_t)m * K;
            for (int k = 0; k < K; ++k) a += zr[k] * wr[k];
        }
        lg[m][c] = a;
    }
    __syncthreads();
    head_epilogue<32, 64>(lg, st, M, 0, M, n0, V, blockIdx.x, hpart, logits_dbg);
}

// ------------------------------------------------------------------------------------------------------
// LDS-tiled MFMA LM head for many block rows (serving batches): tile 128 vocabulary x 128 rows
// ------------------------------------------------------------------------------------------------------
// The tiled GEMM main loop leaves each wave a 64 x 64 block of logits in registers; the tile is parked in
// LDS (over the staging buffers, which are free after the loop) and the row reductions run on it.
#define TH_LG_BYTES (128 * 129 * 4)
#define TH_ST_BYTES (256 * HEAD_REC * 4)
__global__ __launch_bounds__(256) void lm_head_tiled_bf16(const bf16_t* __restrict__ z, size_t zplane, int M,
                                                          const bf16_t* __restrict__ W, int V, int K,
                                                          float* __restrict__ hpart, float* __restrict__ logits_dbg) {
    static_assert(TH_LG_BYTES >= (TL_SW + 2 * TL_BM * TL_LD) * 2, "logits tile must cover the staging buffers");
    __shared__ __attribute__((aligned(16))) char smem[TH_LG_BYTES + TH_ST_BYTES];
    bf16_t* sw = (bf16_t*)smem;
    bf16_t* sx = sw + TL_SW;
    float(*lg)[129] = (float(*)[129])smem;
    float(*st)[HEAD_REC] = (float(*)[HEAD_REC])(smem + TH_LG_BYTES);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const int n0 = blockIdx.x * TL_BN, m0 = blockIdx.y * TL_BM;
    f32x4 acc[4][4];
    tiled_mainloop<true>(z, K, zplane, M, W, V, K, n0, m0, 0, K, sw, sx, acc);
    __syncthreads();  // staging buffers are dead from here on: reuse them for the logits tile
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = wn * 64 + a * 16 + 4 * g;
            const int m = wm * 64 + b * 16 + r;
            lg[m][n + 0] = acc[a][b][0];
            lg[m][n + 1] = acc[a][b][1];
            lg[m][n + 2] = acc[a][b][2];
            lg[m][n + 3] = acc[a][b][3];
        }
    __syncthreads();
    head_epilogue<128, 128>(lg, st, min(128, M - m0), m0, M, n0, V, blockIdx.x, hpart, logits_dbg);
}

hipError_t launch_lm_head(int bf16, const void* z, int M, const void* wlm, int V, int K, float* hpart,
                          float* logits_dbg, hipStream_t st) {
    const dim3 grid(head_groups(V, head_group_width(bf16, M)));
    const size_t zplane = (size_t)M * K;
    if (bf16 && M > 32)
        hipLaunchKernelGGL(lm_head_tiled_bf16, dim3(grid.x, (M + TL_BM - 1) / TL_BM), dim3(256), 0, st,
                           (const bf16_t*)z, zplane, M, (const bf16_t*)wlm, V, K, hpart, logits_dbg);
    else if (!bf16)
        hipLaunchKernelGGL(lm_head_f32, grid, dim3(256), 0, st, (const float*)z, M, (const float*)wlm, V, K, hpart,
                           logits_dbg);
    else if (M <= 16)
        hipLaunchKernelGGL(lm_head_bf16<1>, grid, dim3(256), 0, st, (const bf16_t*)z, zplane, M, (const bf16_t*)wlm,
                           V, K, hpart, logits_dbg);
    else
        hipLaunchKernelGGL(lm_head_bf16<2>, grid, dim3(256), 0, st, (const bf16_t*)z, zplane, M, (const bf16_t*)wlm,
                           V, K, hpart, logits_dbg);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// stage 2: merge the per-group records of one block row
// ------------------------------------------------------------------------------------------------------
#define MERGE_THREADS 1024
__global__ __launch_bounds__(MERGE_THREADS) void head_merge(int M, int V, int n_groups, int top_k,
                                                            const float* __restrict__ hpart,
                                                            const int32_t* __restrict__ btok,
                                                            int32_t* __restrict__ tokens, int32_t* __restrict__ topk_ids,
                                                            float* __restrict__ topk_lp, uint32_t* err) {
    __shared__ float st[MERGE_THREADS / 2][HEAD_REC];
    const int m = blockIdx.x, t = threadIdx.x;
    if (t == 0 && (btok[m] < 0 || btok[m] >= V)) set_err(err, DFLASH_DEVERR_TOKEN);
    TopK s;
    s.init();
    for (int gi = t; gi < n_groups; gi += MERGE_THREADS) {
        const float* rec = hpart + ((size_t)gi * M + m) * HEAD_REC;
        float r[HEAD_REC];
#pragma unroll
        for (int j = 0; j < HEAD_REC; ++j) r[j] = rec[j];
        int oid[DF_TOPK];
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(r[2 + DF_TOPK + j]);
        topk_merge(s, r + 2, oid, r[0], r[1]);
    }
    // fixed-order tree over the thread states
    for (int half = MERGE_THREADS / 2; half > 0; half >>= 1) {
        __syncthreads();
        if (t >= half && t < 2 * half) {
            float* d = st[t - half];
            d[0] = s.mx;
            d[1] = s.se;
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) {
                d[2 + j] = s.v[j];
                d[2 + DF_TOPK + j] = __int_as_float(s.id[j]);
            }
        }
        __syncthreads();
        if (t < half) {
            const float* o = st[t];
            int oid[DF_TOPK];
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(o[2 + DF_TOPK + j]);
            topk_merge(s, o + 2, oid, o[0], o[1]);
        }
    }
    if (t == 0) {
        const float lse = s.mx + logf(s.se);
        tokens[m] = s.id[0];
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {  // static indices keep the state in registers
            if (j < top_k) {
                topk_ids[(size_t)m * top_k + j] = s.id[j];
                topk_lp[(size_t)m * top_k + j] = s.v[j] - lse;
            }
        }
    }
}

hipError_t launch_head_merge(int bf16, int M, int V, int top_k, const float* hpart, const int32_t* block_tokens,
                             int32_t* tokens, int32_t* topk_ids, float* topk_lp, uint32_t* err, hipStream_t st) {
    const int groups = head_groups(V, head_group_width(bf16, M));
    hipLaunchKernelGGL(head_merge, dim3(M), dim3(MERGE_THREADS), 0, st, M, V, groups, top_k, hpart, block_tokens,
                       tokens,
                       topk_ids, topk_lp, err);
    return hipGetLastError();
}

}  // namespace df
