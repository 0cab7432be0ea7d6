// Verification at temperature 1 by modified rejection sampling (Leviathan, Kalman and Matias, "Fast Inference
// from Transformers via Speculative Decoding", ICML 2023, section 2.3 and Algorithm 1; the DFlash page names
// this procedure in section 3.4.4 "Integration with verification").  Per request, draft j is kept when
// u_j < p_j(y_j) / q_j(y_j); at the first rejection k the next token is drawn from max(0, p_k - q_k)
// (renormalised; from p_k if that vanishes in floating point), and when every draft is kept the bonus token
// is drawn from the target's last row.  Both draws are Gumbel-max samples, so no row is normalised or
// prefix-summed: three passes over HBM-resident float32 logits, each coalesced and spread over the chip.
//
//   sv_row_stats   one workgroup per 4096-logit chunk of every target and drafter row: (max, sum of exp)
//   sv_resample    one workgroup per 1024-logit chunk of the row where the request stops: every workgroup
//                  first merges the row statistics (waves split the rows, lanes the chunks, all loads issued
//                  at once) and takes the acceptance tests itself (one lane per draft, a ballot finds the
//                  first rejection), then scores its chunk of that row
//   sv_finish      one wave per request: the best chunk candidate is the next token; tau = kept + 1
#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace df {

#define SV_CHUNK 4096   // logits per workgroup of the statistics pass
#define SV_RCHUNK 1024  // logits per workgroup of the resampling pass (four per thread: one generator block)
#define SV_THREADS 256
#define SV_PER_THREAD (SV_CHUNK / SV_THREADS)
#define SV_MAX_ROWS 127  // 2 * 63 + 1

int sv_chunks(int V) { return (V + SV_CHUNK - 1) / SV_CHUNK; }
static int sv_rchunks(int V) { return (V + SV_RCHUNK - 1) / SV_RCHUNK; }

static size_t sv_align(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: row statistics [B][2 n_draft + 1][chunks] float2, chunk candidates [B][rchunks] float4, k [B]
size_t sv_workspace_bytes(int B, int n_draft, int V) {
    return sv_align((size_t)B * (2 * n_draft + 1) * sv_chunks(V) * 8) + sv_align((size_t)B * sv_rchunks(V) * 16) +
           sv_align((size_t)B * 4);
}

__device__ __forceinline__ float sv_block_max(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < SV_THREADS / 64; ++i) t = fmaxf(t, red[i]);
    return t;
}

// Row r of request b (r <= n_draft: target row r; otherwise drafter row r - n_draft - 1).
__global__ __launch_bounds__(SV_THREADS) void sv_row_stats(int n_draft, int V, int nc, const float* __restrict__ p,
                                                           int64_t p_req, const float* __restrict__ q, int64_t q_req,
                                                           float2* __restrict__ stats) {
    __shared__ float red[SV_THREADS / 64];
    const int R = 2 * n_draft + 1;
    const int c = blockIdx.x % nc, rr = blockIdx.x / nc;
    const int b = rr / R, r = rr % R;
    const float* row = r <= n_draft ? p + b * p_req + (int64_t)r * V : q + b * q_req + (int64_t)(r - n_draft - 1) * V;
    const int x0 = c * SV_CHUNK;
    float v[SV_PER_THREAD];
    float m = -INFINITY;
    if ((V & 3) == 0 && (((uintptr_t)row) & 15) == 0) {  // 16-byte loads (x < V implies x + 3 < V)
#pragma unroll
        for (int i = 0; i < SV_PER_THREAD / 4; ++i) {
            const int x = x0 + 4 * (i * SV_THREADS + threadIdx.x);
            const float4 f = x < V ? *(const float4*)(row + x) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < SV_PER_THREAD; ++i) {
            const int x = x0 + i * SV_THREADS + threadIdx.x;
            v[i] = x < V ? row[x] : -INFINITY;
        }
    }
#pragma unroll
    for (int i = 0; i < SV_PER_THREAD; ++i) m = fmaxf(m, v[i]);
    m = sv_block_max(m, red);
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < SV_PER_THREAD; ++i) s += expf(v[i] - m);  // exp(-inf) = 0 for padding
    }
    s = block_sum(s, red);
    if (threadIdx.x == 0) stats[(size_t)rr * nc + c] = make_float2(m, s);
}

__device__ __forceinline__ void sv_take(float v, int id, float& bv, int& bid) {
    if (df_better(v, id, bv, bid)) {
        bv = v;
        bid = id;
    }
}

// (m, s) += chunk record (cm, cs): running max and sum of exponentials; -inf records carry no mass.
__device__ __forceinline__ void sv_merge(float& m, float& s, float2 r) {
    if (r.x == -INFINITY) return;
    if (r.x > m) {
        s = s * expf(m - r.x) + r.y;  // exp(-inf) = 0 on the first record
        m = r.x;
    } else {
        s += r.y * expf(r.x - m);
    }
}

__global__ __launch_bounds__(SV_THREADS) void sv_resample(int n_draft, int V, int nc, const int32_t* __restrict__ draft,
                                                          int64_t dstride, const float* __restrict__ p, int64_t p_req,
                                                          const float* __restrict__ q, int64_t q_req,
                                                          const float2* __restrict__ stats, RngKey key,
                                                          float4* __restrict__ cand, int32_t* __restrict__ kbuf) {
    __shared__ float lse[SV_MAX_ROWS];
    __shared__ float s_lsep, s_lseq;
    __shared__ int s_k;
    __shared__ float rv[SV_THREADS / 64][2];
    __shared__ int ri[SV_THREADS / 64][2];
    const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int R = 2 * n_draft + 1;
    const float2* st = stats + (size_t)b * R * nc;
    // the drafts and their two logits do not depend on the statistics: in flight while those are merged
    int y = -1;
    float py = 0.f, qy = 0.f;
    if (t < n_draft) {
        y = draft[b * dstride + t];
        if (y >= 0 && y < V) {
            py = p[b * p_req + (int64_t)t * V + y];
            qy = q[b * q_req + (int64_t)t * V + y];
        }
    }
    // log-sum-exp of every row of the request: wave w takes rows w, w + 4, ... (eight per pass), lane l the
    // chunks l, l + 64, ...; every load of a pass is issued before any is consumed
    for (int r0 = 0; r0 < R; r0 += 32) {
        float m[8], sm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            m[i] = -INFINITY;
            sm[i] = 0.f;
        }
        for (int c0 = 0; c0 < nc; c0 += 64) {
            float2 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = r0 + wave + 4 * i;
                v[i] = (r < R && c0 + lane < nc) ? st[(size_t)r * nc + c0 + lane] : make_float2(-INFINITY, 0.f);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sv_merge(m[i], sm[i], v[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = r0 + wave + 4 * i;
            const float M = wave_max(m[i]);
            const float S = wave_sum(m[i] == -INFINITY ? 0.f : sm[i] * expf(m[i] - M));
            if (lane == 0 && r < R) lse[r] = M == -INFINITY ? -INFINITY : M + logf(S);
        }
    }
    __syncthreads();
    if (t < 64) {  // one lane per draft position (n_draft < 64)
        const int j = t;
        float lsep = -INFINITY, lseq = -INFINITY;
        bool keep = true;
        if (j <= n_draft) lsep = lse[j];
        if (j < n_draft) {
            lseq = lse[n_draft + 1 + j];
            keep = false;  // an id outside the vocabulary counts as rejected
            if (y >= 0 && y < V) {
                const float lp = py - lsep;
                const float lq = qy - lseq;
                const float u = rng_uniform(rng_word(key, (uint32_t)j, (uint32_t)b, RNG_TAG_ACCEPT));
                keep = logf(u) < lp - lq;  // u < p / q
            }
        }
        const unsigned long long rej = __ballot(j < n_draft && !keep);
        const int k = rej ? __ffsll(rej) - 1 : n_draft;
        if (j == k) {
            s_lsep = lsep;
            s_lseq = lseq;
            s_k = k;
        }
    }
    __syncthreads();
    const int k = s_k;
    const float lsep = s_lsep, lseq = s_lseq;
    const bool resid = k < n_draft;
    const float* prow = p + b * p_req + (int64_t)k * V;
    const float* qrow = resid ? q + b * q_req + (int64_t)k * V : nullptr;
    float bs = -INFINITY, fs = -INFINITY;  // residual score, plain-p score (fallback / bonus)
    int bi = 0x7FFFFFFF, fi = 0x7FFFFFFF;
    {
        const int xb = c * SV_RCHUNK + 4 * t;  // four consecutive ids: one generator block
        uint32_t w[4];
        if (xb < V) philox_block(key, (uint32_t)xb >> 2, (uint32_t)b, RNG_TAG_RESAMPLE, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = xb + e;
            if (x < V) {
                const float g = rng_gumbel(w[e]);
                const float lp = prow[x] - lsep;
                if (lp + g > fs) {  // ids ascend within a thread: ties keep the smaller id
                    fs = lp + g;
                    fi = x;
                }
                if (resid) {
                    const float r = expf(lp) - expf(qrow[x] - lseq);
                    if (r > 0.f && logf(r) + g > bs) {
                        bs = logf(r) + g;
                        bi = x;
                    }
                }
            }
        }
    }
    if (!resid) {
        bs = fs;
        bi = fi;
    }
    for (int o = 32; o > 0; o >>= 1) {
        sv_take(__shfl_xor(bs, o, DF_WAVE), __shfl_xor(bi, o, DF_WAVE), bs, bi);
        sv_take(__shfl_xor(fs, o, DF_WAVE), __shfl_xor(fi, o, DF_WAVE), fs, fi);
    }
    if (lane == 0) {
        rv[wave][0] = bs;
        ri[wave][0] = bi;
        rv[wave][1] = fs;
        ri[wave][1] = fi;
    }
    __syncthreads();
    if (t == 0) {
        for (int i = 1; i < SV_THREADS / 64; ++i) {
            sv_take(rv[i][0], ri[i][0], bs, bi);
            sv_take(rv[i][1], ri[i][1], fs, fi);
        }
        cand[(size_t)b * gridDim.x + c] = make_float4(bs, __int_as_float(bi), fs, __int_as_float(fi));
        if (c == 0) kbuf[b] = k;
    }
}

__global__ __launch_bounds__(64) void sv_finish(int nc, const float4* __restrict__ cand, const int32_t* __restrict__ kbuf,
                                                int32_t* __restrict__ tau, int32_t* __restrict__ next_token) {
    const int b = blockIdx.x, lane = threadIdx.x;
    float bs = -INFINITY, fs = -INFINITY;
    int bi = 0x7FFFFFFF, fi = 0x7FFFFFFF;
    for (int c = lane; c < nc; c += 64) {
        const float4 v = cand[(size_t)b * nc + c];
        sv_take(v.x, __float_as_int(v.y), bs, bi);
        sv_take(v.z, __float_as_int(v.w), fs, fi);
    }
    for (int o = 32; o > 0; o >>= 1) {
        sv_take(__shfl_xor(bs, o, DF_WAVE), __shfl_xor(bi, o, DF_WAVE), bs, bi);
        sv_take(__shfl_xor(fs, o, DF_WAVE), __shfl_xor(fi, o, DF_WAVE), fs, fi);
    }
    if (lane == 0) {
        next_token[b] = bs != -INFINITY ? bi : fi;  // a residual that vanished everywhere: sample p instead
        tau[b] = kbuf[b] + 1;
    }
}

hipError_t launch_verify_sample(int batch, int n_draft, int V, const int32_t* draft, int64_t dstride, const float* q,
                                int64_t q_req, const float* p, int64_t p_req, uint64_t seed, int32_t* tau,
                                int32_t* next_token, void* ws, hipStream_t st) {
    const int nc = sv_chunks(V), nr = sv_rchunks(V);
    char* W = (char*)ws;
    float2* stats = (float2*)W;
    float4* cand = (float4*)(W + sv_align((size_t)batch * (2 * n_draft + 1) * nc * 8));
    int32_t* kbuf = (int32_t*)((char*)cand + sv_align((size_t)batch * nr * 16));
    const RngKey key{(uint32_t)seed, (uint32_t)(seed >> 32)};
    hipLaunchKernelGGL(sv_row_stats, dim3(nc * batch * (2 * n_draft + 1)), dim3(SV_THREADS), 0, st, n_draft, V, nc, p,
                       p_req, q, q_req, stats);
    hipLaunchKernelGGL(sv_resample, dim3(nr, batch), dim3(SV_THREADS), 0, st, n_draft, V, nc, draft, dstride, p, p_req,
                       q, q_req, stats, key, cand, kbuf);
    hipLaunchKernelGGL(sv_finish, dim3(batch), dim3(64), 0, st, nr, cand, kbuf, tau, next_token);
    return hipGetLastError();
}

}  // namespace df
