// Block attention over [injected context ; block] (non-causal), grouped-query, paged context.
//
// Work split: one workgroup per (request, KV head, chunk).  Chunk 0 is the block's own 16-slot K/V page;
// chunks 1..n are consecutive ranges of the request's cached context.  Wave w of the workgroup serves query
// head kv_head * G + w (G = query heads per KV head), whose L block rows form one 16-row MFMA tile.  Per pair
// of 16-key pages the wave computes S^T = K Q^T (keys in rows, so a lane's four scores belong to one query
// row), updates an online softmax in the log2 domain, and accumulates O^T = V^T P^T.  Values are cached
// transposed inside each page ([d][slot]) so that the V^T operand is two 8-byte loads per lane, and the
// probabilities enter the MFMA as P = P_hi + P_lo (two bfloat16 terms), which keeps them float32-exact.
// Each chunk writes (m, l, O) partials; attn_merge combines the chunks in a fixed order.
#include "common.h"
#include "kernels.h"

namespace df {

AttnPlan plan_attention(int batch, int n_kv, int max_ctx) {
    AttnPlan p{0, 32};
    if (max_ctx <= 0) return p;
    const int units = batch * n_kv;
    int want = (256 + units - 1) / units;
    const int max_chunks = (max_ctx + 31) / 32;
    if (want > max_chunks) want = max_chunks;
    if (want < 1) want = 1;
    int ct = (max_ctx + want - 1) / want;
    ct = (ct + 31) / 32 * 32;
    p.chunk_tokens = ct;
    p.n_chunks = (max_ctx + ct - 1) / ct;
    return p;
}

size_t attn_partial_floats(int batch, int nq, int n_chunks, int d) {
    return (size_t)batch * nq * (n_chunks + 1) * 16 * (size_t)(d + 2);
}

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// ------------------------------------------------------------------------------------------------------
// bfloat16 MFMA kernel (head_dim 128)
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(512) void attn_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kb,
                                                 const bf16_t* __restrict__ vbt, const bf16_t* __restrict__ kpool,
                                                 const bf16_t* __restrict__ vpool, int layer, int n_pages,
                                                 const int32_t* __restrict__ pt, int max_pages,
                                                 const int32_t* __restrict__ ctx_len, int max_ctx, int chunk_tokens,
                                                 int n_chunks, int L, int nq, int nkv, float* __restrict__ opart,
                                                 float* __restrict__ mlpart, uint32_t* err) {
    constexpr int D = 128;
    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int G = nq / nkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int h = kvh * G + w;
    const int C1 = n_chunks + 1;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);

    // key range of this chunk
    int t0 = 0, t1 = 0;
    bool block_chunk = (c == 0);
    if (!block_chunk) {
        int ctx = ctx_len[b];
        if (ctx > max_ctx || ctx < 0) {
            if (c == 1 && threadIdx.x == 0) set_err(err, DFLASH_DEVERR_POS);
            ctx = ctx < 0 ? 0 : max_ctx;
        }
        t0 = (c - 1) * chunk_tokens;
        t1 = min(ctx, t0 + chunk_tokens);
    } else {
        t1 = L;
    }

    // Q^T operand: lane supplies query row r (zero beyond L), eight d-values per 32-wide k-step
    u32x4 qf[4];
    {
        const bool ok = r < L;
        const bf16_t* qp = q + ((size_t)(b * L + (ok ? r : 0)) * nq + h) * D + g * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = ok ? ld16(qp + s * 32) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const size_t page_elems = (size_t)16 * D;
    for (int tp = t0; tp < t1; tp += 32) {
        // the two pages of this step (the block chunk has one)
        const bf16_t* kp[2];
        const bf16_t* vp[2];
        bool pvalid[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int ts = tp + 16 * e;
            pvalid[e] = false;
            kp[e] = kb;
            vp[e] = vbt;
            if (block_chunk) {
                if (e == 0) {
                    kp[e] = kb + ((size_t)b * nkv + kvh) * page_elems;
                    vp[e] = vbt + ((size_t)b * nkv + kvh) * page_elems;
                    pvalid[e] = true;
                }
            } else if (ts < t1) {
                const int pi = ts >> 4;
                int page = pi < max_pages ? pt[(size_t)b * max_pages + pi] : -1;
                if (pi >= max_pages) {
                    if (lane == 0 && w == 0) set_err(err, DFLASH_DEVERR_POS);
                } else if (page < 0 || page >= n_pages) {
                    if (lane == 0 && w == 0) set_err(err, DFLASH_DEVERR_PAGE);
                } else {
                    const size_t pg = ((size_t)layer * n_pages + page) * nkv + kvh;
                    kp[e] = kpool + pg * page_elems;
                    vp[e] = vpool + pg * page_elems;
                    pvalid[e] = true;
                }
            }
        }
        // scores S^T[key][query]: lane holds keys 4g+i of each page for query r
        float x[2][4];
        bool kvalid[2][4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
            if (pvalid[e]) {
                const bf16_t* kr = kp[e] + (size_t)r * D + g * 8;
#pragma unroll
                for (int s = 0; s < 4; ++s) sa = mfma16(ld16(kr + s * 32), qf[s], sa);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = tp + 16 * e + 4 * g + i;
                kvalid[e][i] = pvalid[e] && key < t1;
                x[e][i] = kvalid[e][i] ? sa[i] * scale_log2 : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[e][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        // no branch around the MFMAs: while every key so far is masked, use 0 as the reference so that
        // alpha and p evaluate to 0 instead of exp2(-inf + inf)
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_ref);
        m_run = m_new;
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[e][i] = exp2f(x[e][i] - m_ref);
                psum += p[e][i];
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
        }
        // P^T operand, split into two bfloat16 terms
        bf16_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = p[e][i];
                const bf16_t hb = f2bf(v);
                hi[4 * e + i] = hb;
                lo[4 * e + i] = f2bf(v - bf2f(hb));
            }
        const u32x4 phi = u32x4{pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(hi[4], hi[5]), pack2(hi[6], hi[7])};
        const u32x4 plo = u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]), pack2(lo[6], lo[7])};
        // V^T operand: lane row d = 16 dt + r, keys 4g..4g+3 of each page (masked keys read as zero)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            u32x2 va = u32x2{0u, 0u}, vb2 = u32x2{0u, 0u};
            const int d = dt * 16 + r;
            if (pvalid[0]) va = *(const u32x2*)(vp[0] + (size_t)d * 16 + 4 * g);
            if (pvalid[1]) vb2 = *(const u32x2*)(vp[1] + (size_t)d * 16 + 4 * g);
            uint32_t a0 = va.x, a1 = va.y, b0 = vb2.x, b1 = vb2.y;
            if (!kvalid[0][0]) a0 &= 0xFFFF0000u;
            if (!kvalid[0][1]) a0 &= 0x0000FFFFu;
            if (!kvalid[0][2]) a1 &= 0xFFFF0000u;
            if (!kvalid[0][3]) a1 &= 0x0000FFFFu;
            if (!kvalid[1][0]) b0 &= 0xFFFF0000u;
            if (!kvalid[1][1]) b0 &= 0x0000FFFFu;
            if (!kvalid[1][2]) b1 &= 0xFFFF0000u;
            if (!kvalid[1][3]) b1 &= 0x0000FFFFu;
            const u32x4 vf = u32x4{a0, a1, b0, b1};
            o[dt] = mfma16(vf, phi, o[dt]);
            o[dt] = mfma16(vf, plo, o[dt]);
        }
    }

    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const size_t base = (((size_t)b * nq + h) * C1 + c) * 16 + r;
    float* op = opart + base * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        *(float4*)(op + dt * 16 + 4 * g) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
        mlpart[base * 2 + 0] = m_run;
        mlpart[base * 2 + 1] = l_tot;
    }
}

// ------------------------------------------------------------------------------------------------------
// merge of the chunk partials -> o (rounded), and the float32 attention kernel
// ------------------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_merge(const float* __restrict__ opart, const float* __restrict__ mlpart,
                                                  int B, int L, int nq, int d, int C1, T* __restrict__ o) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)B * L * nq * d) return;
    const int dd = idx % d;
    const int h = (idx / d) % nq;
    const int row = (idx / ((long)d * nq)) % L;
    const int b = idx / ((long)d * nq * L);
    const size_t base = ((size_t)b * nq + h) * C1;
    float M = -INFINITY;
    for (int c = 0; c < C1; ++c) M = fmaxf(M, mlpart[((base + c) * 16 + row) * 2]);
    float lsum = 0.f, acc = 0.f;
    for (int c = 0; c < C1; ++c) {
        const float mc = mlpart[((base + c) * 16 + row) * 2];
        if (mc == -INFINITY) continue;
        const float wgt = exp2f(mc - M);
        lsum += wgt * mlpart[((base + c) * 16 + row) * 2 + 1];
        acc += wgt * opart[((base + c) * 16 + row) * d + dd];
    }
    o[((size_t)(b * L + row) * nq + h) * d + dd] = Act<T>::from(acc / lsum);
}

// Float32 drafters: one wave per (block row, query head, request); lanes take keys round-robin with their
// own online softmax, then the wave merges the 64 partial states through LDS.  Writes o directly.
__global__ __launch_bounds__(64) void attn_f32(const float* __restrict__ q, const float* __restrict__ kb,
                                               const float* __restrict__ vbt, const float* __restrict__ kpool,
                                               const float* __restrict__ vpool, int layer, int n_pages,
                                               const int32_t* __restrict__ pt, int max_pages,
                                               const int32_t* __restrict__ ctx_len, int max_ctx, int L, int nq,
                                               int nkv, int d, float* __restrict__ o, uint32_t* err) {
    __shared__ float sq[128];
    __shared__ float sm[64], sl[64];
    __shared__ float so[64][129];
    const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int kvh = h / (nq / nkv);
    for (int j = lane; j < d; j += 64) sq[j] = q[((size_t)(b * L + row) * nq + h) * d + j];
    __syncthreads();
    int ctx = ctx_len[b];
    if (ctx > max_ctx || ctx < 0) {
        if (row == 0 && h == 0 && lane == 0) set_err(err, DFLASH_DEVERR_POS);
        ctx = ctx < 0 ? 0 : max_ctx;
    }
    const float scale = 1.0f / sqrtf((float)d);
    float m = -INFINITY, l = 0.f;
    float acc[128];
    for (int j = 0; j < d; ++j) acc[j] = 0.f;
    const size_t pe = (size_t)16 * d;
    for (int t = lane; t < ctx + L; t += 64) {
        const float* kr;
        const float* vc;
        if (t < ctx) {
            const int pi = t >> 4, slot = t & 15;
            const int page = pi < max_pages ? pt[(size_t)b * max_pages + pi] : -1;
            if (page < 0 || page >= n_pages) {
                set_err(err, pi >= max_pages ? DFLASH_DEVERR_POS : DFLASH_DEVERR_PAGE);
                continue;
            }
            const size_t pg = ((size_t)layer * n_pages + page) * nkv + kvh;
            kr = kpool + pg * pe + (size_t)slot * d;
            vc = vpool + pg * pe + slot;
        } else {
            const int slot = t - ctx;
            kr = kb + ((size_t)b * nkv + kvh) * pe + (size_t)slot * d;
            vc = vbt + ((size_t)b * nkv + kvh) * pe + slot;
        }
        float s = 0.f;
        for (int j = 0; j < d; ++j) s += sq[j] * kr[j];
        s *= scale;
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn), p = expf(s - mn);
        l = l * a + p;
        for (int j = 0; j < d; ++j) acc[j] = acc[j] * a + p * vc[(size_t)j * 16];
        m = mn;
    }
    sm[lane] = m;
    sl[lane] = l;
    for (int j = 0; j < d; ++j) so[lane][j] = acc[j];
    __syncthreads();
    float M = -INFINITY;
    for (int i = 0; i < 64; ++i) M = fmaxf(M, sm[i]);
    for (int j = lane; j < d; j += 64) {
        float num = 0.f, den = 0.f;
        for (int i = 0; i < 64; ++i) {
            if (sm[i] == -INFINITY) continue;
            const float wgt = expf(sm[i] - M);
            num += wgt * so[i][j];
            den += wgt * sl[i];
        }
        o[((size_t)(b * L + row) * nq + h) * d + j] = num / den;
    }
}

hipError_t launch_attention(int bf16, const AttnPlan& p, int B, int L, int nq, int nkv, int d, const void* q,
                            const void* kb, const void* vbt, const void* kpool, const void* vpool, int layer,
                            int n_pages, const int32_t* page_table, int max_pages, const int32_t* ctx_len,
                            int max_ctx, float* opart, float* mlpart, uint32_t* err, hipStream_t st) {
    if (bf16) {
        const int G = nq / nkv;
        hipLaunchKernelGGL(attn_bf16, dim3(p.n_chunks + 1, nkv, B), dim3(64 * G), 0, st, (const bf16_t*)q,
                           (const bf16_t*)kb, (const bf16_t*)vbt, (const bf16_t*)kpool, (const bf16_t*)vpool, layer,
                           n_pages, page_table, max_pages, ctx_len, max_ctx, p.chunk_tokens, p.n_chunks, L, nq, nkv,
                           opart, mlpart, err);
    } else {
        // writes o (float32) straight into opart's storage; no merge step
        hipLaunchKernelGGL(attn_f32, dim3(L, nq, B), dim3(64), 0, st, (const float*)q, (const float*)kb,
                           (const float*)vbt, (const float*)kpool, (const float*)vpool, layer, n_pages, page_table,
                           max_pages, ctx_len, max_ctx, L, nq, nkv, d, opart, err);
    }
    return hipGetLastError();
}

hipError_t launch_attn_merge(int bf16, const AttnPlan& p, int B, int L, int nq, int d, const float* opart,
                             const float* mlpart, void* o, hipStream_t st) {
    const long n = (long)B * L * nq * d;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(attn_merge<bf16_t>, grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d, p.n_chunks + 1,
                           (bf16_t*)o);
    else
        hipLaunchKernelGGL(attn_merge<float>, grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d, p.n_chunks + 1,
                           (float*)o);
    return hipGetLastError();
}

}  // namespace df
