// Row-wise kernels around the GEMMs: embedding + RMSNorm, split-K reduction + residual + RMSNorm, the QKV
// epilogue (RoPE and block K/V layouts), SwiGLU, fused-feature rounding, the paged K/V scatter of the
// injected context, and greedy acceptance.  All of them are bandwidth-trivial next to the weight streams;
// they exist to keep every reduction in a fixed order and every stored tensor in its final layout.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace df {

// ------------------------------------------------------------------------------------------------------
// row kernels: 1024 threads per block row, four consecutive columns per thread and pass (H <= 16384)
// ------------------------------------------------------------------------------------------------------
#define ROW_THREADS 1024
#define ROW_PASSES 4

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }

// Split-K sums in a fixed order (s = 0, 1, ..., S - 1, the same additions as a plain loop), with the loads of
// up to SPLIT_BATCH splits issued before the first add so that they are in flight together.
#define SPLIT_BATCH 8
__device__ __forceinline__ float split_sum(const float* p, size_t stride, int S) {
    float acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += SPLIT_BATCH) {
        float v[SPLIT_BATCH];
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u) v[u] = s0 + u < S ? p[(size_t)(s0 + u) * stride] : 0.f;
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u)
            if (s0 + u < S) acc += v[u];
    }
    return acc;
}
// The same sums for NP columns (offsets col[c] from p) at once: every column's loads of a batch are issued
// before the first add.
template <int NP>
__device__ __forceinline__ void split_sums(const float* p, const int (&col)[NP], size_t stride, int S,
                                           float (&acc)[NP]) {
#pragma unroll
    for (int c = 0; c < NP; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < S; s0 += SPLIT_BATCH) {
        float v[NP][SPLIT_BATCH];
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u)
#pragma unroll
            for (int c = 0; c < NP; ++c) v[c][u] = s0 + u < S ? p[(size_t)(s0 + u) * stride + col[c]] : 0.f;
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u)
            if (s0 + u < S)
#pragma unroll
                for (int c = 0; c < NP; ++c) acc[c] += v[c][u];
    }
}
__device__ __forceinline__ void st4(float* p, float4 v) { *(float4*)p = v; }
// float4 split sums starting from split 0 (no +0 first), batched like split_sum
__device__ __forceinline__ float4 split_sum4(const float* p, size_t stride, int S) {
    float4 acc = ld4(p);
    for (int s0 = 1; s0 < S; s0 += SPLIT_BATCH) {
        float4 v[SPLIT_BATCH];
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u)
            v[u] = s0 + u < S ? ld4(p + (size_t)(s0 + u) * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < SPLIT_BATCH; ++u)
            if (s0 + u < S) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
    }
    return acc;
}
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
    const uint2 b = *(const uint2*)p;
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u), __uint_as_float(b.y << 16),
                       __uint_as_float(b.y & 0xFFFF0000u));
}
// four consecutive activations: a pair of bfloat16 planes, or float32
__device__ __forceinline__ void st4_act(bf16_t* p, size_t plane, float4 v) {
    uint2 hb, lb;
    const bf16_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
    hb.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
    hb.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
    lb.x = (uint32_t)f2bf(v.x - bf2f(h0)) | ((uint32_t)f2bf(v.y - bf2f(h1)) << 16);
    lb.y = (uint32_t)f2bf(v.z - bf2f(h2)) | ((uint32_t)f2bf(v.w - bf2f(h3)) << 16);
    *(uint2*)p = hb;
    *(uint2*)(p + plane) = lb;
}
__device__ __forceinline__ void st4_act(float* p, size_t, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float dot4(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

// u = RMSNorm(v) * g for the row values held in registers (u stored as an activation pair)
// (gv: the gains of this thread's columns, loaded with the row values)
template <typename T>
__device__ __forceinline__ void norm_store(const float4 (&v)[ROW_PASSES], const float4 (&gv)[ROW_PASSES], float ss,
                                           int H, float eps, T* __restrict__ urow, size_t plane, float* red) {
    ss = block_sum(ss, red);
    const float rs = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int q = 0; q < ROW_PASSES; ++q) {
        const int j = (threadIdx.x + q * ROW_THREADS) * 4;
        if (j >= H) break;
        const float4 g = gv[q];
        st4_act(urow + j, plane,
                make_float4(v[q].x * rs * g.x, v[q].y * rs * g.y, v[q].z * rs * g.z, v[q].w * rs * g.w));
    }
}

// Block row m gathers its token's embedding row (the drafter shares the target's frozen embedding), keeps it
// as the float32 residual, and writes u = RMSNorm(h) * g.  Block 0 clears the call's device error word
// before any later kernel can set a flag; an out-of-range token reads row 0 (flagged later by head_merge).
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void embed_norm(const int32_t* __restrict__ tok, int V,
                                                          const T* __restrict__ embed, const T* __restrict__ gain, int H,
                                                          float eps, float* __restrict__ h, T* __restrict__ u,
                                                          float* __restrict__ tap, uint32_t* err) {
    __shared__ float red[ROW_THREADS / 64];
    const int m = blockIdx.x;
    if (m == 0 && threadIdx.x == 0 && err) *err = 0u;
    int t = tok[m];
    if (t < 0 || t >= V) t = 0;
    const T* e = embed + (size_t)t * H;
    float4 v[ROW_PASSES], gv[ROW_PASSES];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < ROW_PASSES; ++q) {
        const int j = (threadIdx.x + q * ROW_THREADS) * 4;
        if (j >= H) break;
        gv[q] = ld4(gain + j);
        v[q] = ld4(e + j);
        st4(h + (size_t)m * H + j, v[q]);
        if (tap) st4(tap + (size_t)m * H + j, v[q]);
        ss += dot4(v[q]);
    }
    norm_store(v, gv, ss, H, eps, u + (size_t)m * H, (size_t)gridDim.x * H, red);
}

hipError_t launch_embed_norm(int bf16, const int32_t* tok, int M, int V, const void* embed, const void* gain, int H,
                             float eps, float* h, void* u, float* tap, uint32_t* err, hipStream_t st) {
    if (bf16)
        hipLaunchKernelGGL(embed_norm<bf16_t>, dim3(M), dim3(ROW_THREADS), 0, st, tok, V, (const bf16_t*)embed,
                           (const bf16_t*)gain, H, eps, h, (bf16_t*)u, tap, err);
    else
        hipLaunchKernelGGL(embed_norm<float>, dim3(M), dim3(ROW_THREADS), 0, st, tok, V, (const float*)embed,
                           (const float*)gain, H, eps, h, (float*)u, tap, err);
    return hipGetLastError();
}

// h += sum over splits of a GEMM product (fixed order), then u = RMSNorm(h) * g.
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void resid_norm(const float* __restrict__ part, int S, int M, int H,
                                                          float* __restrict__ h, const T* __restrict__ gain, float eps,
                                                          T* __restrict__ u, float* __restrict__ tap) {
    __shared__ float red[ROW_THREADS / 64];
    const int m = blockIdx.x;
    float4 v[ROW_PASSES], gv[ROW_PASSES];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < ROW_PASSES; ++q) {
        const int j = (threadIdx.x + q * ROW_THREADS) * 4;
        if (j >= H) break;
        // the residual and the gains are requested with the splits: one round trip
        gv[q] = ld4(gain + j);
        const float4 hv = ld4(h + (size_t)m * H + j);
        const float4 a = split_sum4(part + (size_t)m * H + j, (size_t)M * H, S);
        v[q] = add4(hv, a);
        st4(h + (size_t)m * H + j, v[q]);
        if (tap) st4(tap + (size_t)m * H + j, v[q]);
        ss += dot4(v[q]);
    }
    norm_store(v, gv, ss, H, eps, u + (size_t)m * H, (size_t)M * H, red);
}

hipError_t launch_resid_norm(int bf16, const float* part, int S, int M, int H, float* h, const void* gain, float eps,
                             void* u, float* tap, hipStream_t st) {
    if (bf16)
        hipLaunchKernelGGL(resid_norm<bf16_t>, dim3(M), dim3(ROW_THREADS), 0, st, part, S, M, H, h, (const bf16_t*)gain,
                           eps, (bf16_t*)u, tap);
    else
        hipLaunchKernelGGL(resid_norm<float>, dim3(M), dim3(ROW_THREADS), 0, st, part, S, M, H, h, (const float*)gain,
                           eps, (float*)u, tap);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// QKV epilogue
// ------------------------------------------------------------------------------------------------------
// One thread per (block row m = grid y, head, rotary pair i): sums the splits of columns i and i + d/2,
// applies the rotation at position ctx_len[b] + row to q and k heads, rounds, and stores q row-major, the
// block's keys as a 16-slot page [b][kv head][slot][d] and its values transposed [b][kv head][d][slot].
template <typename T>
__global__ __launch_bounds__(256) void qkv_epilogue(const float* __restrict__ part, int S, int B, int L, int nq,
                                                    int nkv, int d, const int32_t* __restrict__ ctx_len, RopeFreq rf,
                                                    T* __restrict__ q, T* __restrict__ kb, T* __restrict__ vbt) {
    const int half = d >> 1;
    const int heads = nq + 2 * nkv;
    const int M = B * L;
    const int N = heads * d;
    const int x = blockIdx.x * 256 + threadIdx.x;  // (32-bit index arithmetic: no 64-bit division)
    if (x >= heads * half) return;
    const int i = x % half;
    const int hd = x / half;
    const int m = blockIdx.y;
    const int c1 = hd * d + i, c2 = c1 + half;
    // the context length and the frequency are requested before the splits and first used after them
    const int ctx = ctx_len[m / L];
    const float inv = rf.inv[i];
    const int col[2] = {c1, c2};
    float sum[2];
    split_sums<2>(part + (size_t)m * N, col, (size_t)M * N, S, sum);
    qkv_store(sum[0], sum[1], m, hd, i, B, L, nq, nkv, d, ctx + m % L, rf.on != 0, inv, q, kb, vbt);
}

hipError_t launch_qkv_epilogue(int bf16, const float* part, int S, int B, int L, int nq, int nkv, int d,
                               const int32_t* ctx_len, const RopeFreq& rf, void* q, void* kb, void* vbt,
                               hipStream_t st) {
    const int n = (nq + 2 * nkv) * (d / 2);
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)(B * L));
    if (bf16)
        hipLaunchKernelGGL(qkv_epilogue<bf16_t>, grid, dim3(256), 0, st, part, S, B, L, nq, nkv, d, ctx_len, rf,
                           (bf16_t*)q, (bf16_t*)kb, (bf16_t*)vbt);
    else
        hipLaunchKernelGGL(qkv_epilogue<float>, grid, dim3(256), 0, st, part, S, B, L, nq, nkv, d, ctx_len, rf,
                           (float*)q, (float*)kb, (float*)vbt);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// SwiGLU and plain reduce + cast
// ------------------------------------------------------------------------------------------------------
// Four consecutive columns per thread (F % 4 == 0 for every drafter the API accepts): 16-byte split loads
// of gate and up, 8-byte stores per activation plane.
template <typename T>
__global__ __launch_bounds__(256) void swiglu(const float* __restrict__ part, int S, int M, int F,
                                              T* __restrict__ a) {
    const int j = (blockIdx.x * 256 + threadIdx.x) * 4, m = blockIdx.y;  // first column, row (grid y)
    if (j >= F) return;
    const size_t N = 2 * (size_t)F;
    const float* pr = part + (size_t)m * N;
    const float4 g = split_sum4(pr + j, (size_t)M * N, S);
    const float4 u = split_sum4(pr + F + j, (size_t)M * N, S);
    st4_act(a + (size_t)m * F + j, (size_t)M * F,
            make_float4(swiglu_value(g.x, u.x), swiglu_value(g.y, u.y), swiglu_value(g.z, u.z),
                        swiglu_value(g.w, u.w)));
}

hipError_t launch_swiglu(int bf16, const float* part, int S, int M, int F, void* a, hipStream_t st) {
    if (F % 4) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((F / 4 + 255) / 256), (unsigned)M);
    if (bf16) hipLaunchKernelGGL(swiglu<bf16_t>, grid, dim3(256), 0, st, part, S, M, F, (bf16_t*)a);
    else hipLaunchKernelGGL(swiglu<float>, grid, dim3(256), 0, st, part, S, M, F, (float*)a);
    return hipGetLastError();
}

// clear_err (nullable): the call's device error word, zeroed by block 0 (this kernel sets no flag itself).
template <typename T>
__global__ __launch_bounds__(256) void reduce_cast(const float* __restrict__ part, int S, int M, int N,
                                                   const T* __restrict__ bias, T* __restrict__ out,
                                                   uint32_t* clear_err) {
    if (clear_err && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *clear_err = 0u;
    const int n = blockIdx.x * 256 + threadIdx.x;  // column; the row is grid y
    if (n >= N) return;
    const size_t idx = (size_t)blockIdx.y * N + n;
    T braw{};
    if (bias) braw = bias[n];  // requested before the splits, converted after them
    float v = split_sum(part + idx, (size_t)M * N, S);
    if (bias) v += Act<T>::load(&braw);
    put_act(out, (size_t)M * N, idx, v);
}

hipError_t launch_reduce_cast(int bf16, const float* part, int S, int M, int N, const void* bias, void* out,
                              uint32_t* clear_err, hipStream_t st) {
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)M);
    if (bf16)
        hipLaunchKernelGGL(reduce_cast<bf16_t>, grid, dim3(256), 0, st, part, S, M, N, (const bf16_t*)bias,
                           (bf16_t*)out, clear_err);
    else
        hipLaunchKernelGGL(reduce_cast<float>, grid, dim3(256), 0, st, part, S, M, N, (const float*)bias, (float*)out,
                           clear_err);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// injected context: RoPE + paged scatter
// ------------------------------------------------------------------------------------------------------
// One thread per (row, layer, kv head, rotary pair).  The row's request comes from a binary search of
// row_offsets; its position is start_pos[r] + (row - row_offsets[r]).  A position beyond the page table or a
// page id outside the pool is skipped and flagged.
template <typename T>
__global__ __launch_bounds__(256) void kv_scatter(const float* __restrict__ part, int S, int rows, int row0,
                                                  int layer0, int n_layers, int nkv, int d, int batch,
                                                  const int32_t* __restrict__ off, const int32_t* __restrict__ start,
                                                  const int32_t* __restrict__ pt, int max_pages, int n_pages,
                                                  T* __restrict__ kpool, T* __restrict__ vpool, RopeFreq rf,
                                                  uint32_t* err) {
    const int half = d >> 1;
    const int x = blockIdx.x * 256 + threadIdx.x;  // (layer, kv head, rotary pair); the row is grid y
    if (x >= n_layers * nkv * half) return;
    const int i = x % half;
    const int kh = (x / half) % nkv;
    const int l = x / (half * nkv);
    const int j = blockIdx.y;
    const int R = row0 + j;
    // the split sums first (they depend only on the row), so that their loads overlap the request's lookup
    const int N = n_layers * 2 * nkv * d;
    const int ck = l * 2 * nkv * d + kh * d + i;
    const int cv = ck + nkv * d;
    const int col[4] = {ck, ck + half, cv, cv + half};
    float sum[4];
    split_sums<4>(part + (size_t)j * N, col, (size_t)rows * N, S, sum);
    if (R >= off[batch]) return;  // padding rows: computed, not stored
    int lo = 0, hi = batch - 1;
    while (lo < hi) {  // last r with off[r] <= R
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= R) lo = mid;
        else hi = mid - 1;
    }
    const int r = lo;
    if (off[r] > R || off[r + 1] <= R) {
        if (i == 0 && kh == 0 && l == 0) set_err(err, DFLASH_DEVERR_ROWS);
        return;
    }
    const int pos = start[r] + (R - off[r]);
    const int pi = pos >> 4, slot = pos & 15;
    if (pos < 0 || pi >= max_pages) {
        if (i == 0 && kh == 0 && l == 0) set_err(err, DFLASH_DEVERR_POS);
        return;
    }
    const int page = pt[(size_t)r * max_pages + pi];
    if (page < 0 || page >= n_pages) {
        if (i == 0 && kh == 0 && l == 0) set_err(err, DFLASH_DEVERR_PAGE);
        return;
    }
    float k1 = sum[0], k2 = sum[1];
    const float v1 = sum[2], v2 = sum[3];
    rope_pair(k1, k2, pos, i, rf);
    const size_t pg = ((size_t)(layer0 + l) * n_pages + page) * nkv + kh;
    T* kd = kpool + (pg * 16 + slot) * d;
    kd[i] = Act<T>::from(k1);
    kd[i + half] = Act<T>::from(k2);
    T* vd = vpool + pg * d * 16;
    vd[i * 16 + slot] = Act<T>::from(v1);
    vd[(i + half) * 16 + slot] = Act<T>::from(v2);
}

hipError_t launch_kv_scatter(int bf16, const float* part, int S, int rows, int row0, int layer0, int n_layers,
                             int nkv, int d, int batch, const int32_t* row_offsets, const int32_t* start_pos,
                             const int32_t* page_table, int max_pages, int n_pages, void* kpool, void* vpool,
                             const RopeFreq& rf, uint32_t* err, hipStream_t st) {
    const int n = n_layers * nkv * (d / 2);
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)rows);
    if (bf16)
        hipLaunchKernelGGL(kv_scatter<bf16_t>, grid, dim3(256), 0, st, part, S, rows, row0, layer0, n_layers, nkv, d,
                           batch,
                           row_offsets, start_pos, page_table, max_pages, n_pages, (bf16_t*)kpool, (bf16_t*)vpool, rf,
                           err);
    else
        hipLaunchKernelGGL(kv_scatter<float>, grid, dim3(256), 0, st, part, S, rows, row0, layer0, n_layers, nkv, d,
                           batch,
                           row_offsets, start_pos, page_table, max_pages, n_pages, (float*)kpool, (float*)vpool, rf,
                           err);
    return hipGetLastError();
}

__global__ void clear_err(uint32_t* err) { *err = 0u; }

hipError_t launch_clear_err(uint32_t* err, hipStream_t st) {
    hipLaunchKernelGGL(clear_err, dim3(1), dim3(1), 0, st, err);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// greedy acceptance
// ------------------------------------------------------------------------------------------------------
// tau = 1 + the length of the common prefix of the drafts and the target's tokens: the accepted drafts plus
// the bonus token the target contributes at the first mismatch (or after the block).
__global__ void accept_len(int batch, int n_draft, const int32_t* __restrict__ draft, int64_t ds,
                           const int32_t* __restrict__ target, int64_t ts, int32_t* __restrict__ tau) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= batch) return;
    int k = 0;
    while (k < n_draft && draft[(size_t)r * ds + k] == target[(size_t)r * ts + k]) ++k;
    tau[r] = k + 1;
}

hipError_t launch_accept(int batch, int n_draft, const int32_t* draft, int64_t ds, const int32_t* target, int64_t ts,
                         int32_t* tau, hipStream_t st) {
    hipLaunchKernelGGL(accept_len, dim3((batch + 63) / 64), dim3(64), 0, st, batch, n_draft, draft, ds, target, ts,
                       tau);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// stream copy (bandwidth reference)
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy16(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

hipError_t launch_copy(void* dst, const void* src, size_t n16, hipStream_t st) {
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(copy16, dim3((unsigned)blocks), dim3(256), 0, st, (u32x4*)dst, (const u32x4*)src, n16);
    return hipGetLastError();
}

}  // namespace df
