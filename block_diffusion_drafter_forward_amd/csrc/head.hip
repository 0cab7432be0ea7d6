// Shared LM head fused with the per-row reductions the drafter needs: running max, sum of exponentials
// (for the log-sum-exp over the full vocabulary) and the top-8 (logit, id) list, ordered by logit then id.
// Logits live only in registers and LDS.  Stage 1 (lm_head): one workgroup per 64 vocabulary rows, four
// waves splitting K, writes one (max, sumexp, top-8) record per block row.  Stage 2 (head_merge): one
// workgroup per block row merges the records in a fixed order and emits the greedy token, the top-k ids
// and their log-probabilities.
#include "common.h"
#include "kernels.h"

namespace df {

#define HEAD_REC 18  // max, sumexp, 8 values, 8 ids (as int bits)

int head_groups(int V) { return (V + 63) / 64; }
size_t head_partial_floats(int V, int M) { return (size_t)head_groups(V) * M * HEAD_REC; }

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

// merge state o into s: lists by insertion, (max, sumexp) by rescaling to the larger max
__device__ __forceinline__ void topk_merge(TopK& s, const float* ov, const int* oid, float omx, float ose) {
#pragma unroll
    for (int j = 0; j < DF_TOPK; ++j) topk_insert(s, ov[j], oid[j]);
    if (omx == -INFINITY) return;
    if (s.mx == -INFINITY) { s.mx = omx; s.se = ose; return; }
    const float M = fmaxf(s.mx, omx);
    s.se = s.se * expf(s.mx - M) + ose * expf(omx - M);
    s.mx = M;
}

// Row reductions over a logits tile lg[R][64] held in LDS (columns n0 .. n0+63 of the vocabulary).  Threads
// split each row into TPR pieces, then the first thread of the row merges the pieces.
template <int R>
__device__ void head_epilogue(const float (*lg)[65], float (*st)[HEAD_REC], int M, int n0, int V,
                              float* __restrict__ hpart, float* __restrict__ logits_dbg) {
    constexpr int TPR = 256 / R, CPT = 64 / TPR;
    const int t = threadIdx.x;
    const int m = t / TPR, c0 = (t % TPR) * CPT;
    TopK s;
    s.init();
    if (m < M) {
        for (int c = c0; c < c0 + CPT; ++c) {
            const int v = n0 + c;
            if (v >= V) break;
            const float x = lg[m][c];
            s.push(x, v);
            if (logits_dbg) logits_dbg[(size_t)m * V + v] = x;
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
    if (m < M && (t % TPR) == 0) {
        for (int q = 1; q < TPR; ++q) {
            const float* o = st[t + q];
            int oid[DF_TOPK];
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(o[2 + DF_TOPK + j]);
            topk_merge(s, o + 2, oid, o[0], o[1]);
        }
        float* dst = hpart + ((size_t)blockIdx.x * M + m) * HEAD_REC;
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
template <int MT>
__global__ __launch_bounds__(256) void lm_head_bf16(const bf16_t* __restrict__ z, int M, const bf16_t* __restrict__ W,
                                                    int V, int K, float* __restrict__ hpart,
                                                    float* __restrict__ logits_dbg) {
    constexpr int NT = 4;
    __shared__ f32x4 red[4][NT * MT][64];
    __shared__ float lg[16 * MT][65];
    __shared__ float st[256][HEAD_REC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64;
    const int chunks = K / 256;
    const int kb = (wave * chunks / 4) * 256, ke = ((wave + 1) * chunks / 4) * 256;

    const bf16_t* wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wrow[nt] = W + (size_t)min(n0 + nt * 16 + r, V - 1) * K + g * 8;
    const bf16_t* zrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) zrow[mt] = z + (size_t)min(mt * 16 + r, M - 1) * K + g * 8;

    f32x4 acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = kb; kc < ke; kc += 256) {
        u32x4 wf[NT][8];
        u32x4 zf[MT][8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                wf[nt][j] = ld16_nt(wrow[nt] + kc + j * 32);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 8; ++j) zf[mt][j] = ld16(zrow[mt] + kc + j * 32);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = mfma16(wf[nt][j], zf[mt][j], acc[nt][mt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wave][nt * MT + mt][lane] = acc[nt][mt];
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
    head_epilogue<16 * MT>(lg, st, M, n0, V, hpart, logits_dbg);
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
    head_epilogue<32>(lg, st, M, n0, V, hpart, logits_dbg);
}

hipError_t launch_lm_head(int bf16, const void* z, int M, const void* wlm, int V, int K, float* hpart,
                          float* logits_dbg, hipStream_t st) {
    const dim3 grid(head_groups(V));
    if (!bf16)
        hipLaunchKernelGGL(lm_head_f32, grid, dim3(256), 0, st, (const float*)z, M, (const float*)wlm, V, K, hpart,
                           logits_dbg);
    else if (M <= 16)
        hipLaunchKernelGGL(lm_head_bf16<1>, grid, dim3(256), 0, st, (const bf16_t*)z, M, (const bf16_t*)wlm, V, K,
                           hpart, logits_dbg);
    else
        hipLaunchKernelGGL(lm_head_bf16<2>, grid, dim3(256), 0, st, (const bf16_t*)z, M, (const bf16_t*)wlm, V, K,
                           hpart, logits_dbg);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// stage 2: merge the per-group records of one block row
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void head_merge(int M, int V, int n_groups, int top_k,
                                                  const float* __restrict__ hpart, const int32_t* __restrict__ btok,
                                                  int32_t* __restrict__ tokens, int32_t* __restrict__ topk_ids,
                                                  float* __restrict__ topk_lp, uint32_t* err) {
    __shared__ float st[256][HEAD_REC];
    const int m = blockIdx.x, t = threadIdx.x;
    if (t == 0 && (btok[m] < 0 || btok[m] >= V)) set_err(err, DFLASH_DEVERR_TOKEN);
    TopK s;
    s.init();
    for (int gi = t; gi < n_groups; gi += 256) {
        const float* rec = hpart + ((size_t)gi * M + m) * HEAD_REC;
        int oid[DF_TOPK];
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(rec[2 + DF_TOPK + j]);
        topk_merge(s, rec + 2, oid, rec[0], rec[1]);
    }
    // fixed-order tree over the 256 thread states
    for (int half = 128; half > 0; half >>= 1) {
        __syncthreads();
        if (t >= half && t < 2 * half) {
            st[t][0] = s.mx;
            st[t][1] = s.se;
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) {
                st[t][2 + j] = s.v[j];
                st[t][2 + DF_TOPK + j] = __int_as_float(s.id[j]);
            }
        }
        __syncthreads();
        if (t < half) {
            const float* o = st[t + half];
            int oid[DF_TOPK];
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) oid[j] = __float_as_int(o[2 + DF_TOPK + j]);
            topk_merge(s, o + 2, oid, o[0], o[1]);
        }
    }
    if (t == 0) {
        const float lse = s.mx + logf(s.se);
        tokens[m] = s.id[0];
        for (int j = 0; j < top_k; ++j) {
            topk_ids[(size_t)m * top_k + j] = s.id[j];
            topk_lp[(size_t)m * top_k + j] = s.v[j] - lse;
        }
    }
}

hipError_t launch_head_merge(int M, int V, int top_k, const float* hpart, const int32_t* block_tokens,
                             int32_t* tokens, int32_t* topk_ids, float* topk_lp, uint32_t* err, hipStream_t st) {
    hipLaunchKernelGGL(head_merge, dim3(M), dim3(256), 0, st, M, V, head_groups(V), top_k, hpart, block_tokens, tokens,
                       topk_ids, topk_lp, err);
    return hipGetLastError();
}

}  // namespace df
