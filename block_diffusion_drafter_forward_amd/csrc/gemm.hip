// Weight-streaming GEMMs of the drafter pass: part[s][m][n] = sum_{k in split s} x[m][k] * W[n][k].
//
// At batch 1 the block has M = L = 16 rows, so every projection is a "skinny" product whose cost is the
// bytes of W streamed from HBM once (16 multiply-adds per weight).  The skinny kernel therefore keeps each
// weight in registers for exactly one MFMA per m-tile, spreads K over the four waves of a workgroup and
// over a grid-level split so that enough bytes are in flight on all 256 CUs, and reduces the four waves'
// partial tiles in LDS.  Large M (the 16-request serving batch, prefill of long contexts) uses an LDS-tiled
// MFMA kernel.  Float32 drafters use a VALU kernel.  Every kernel writes float32 split partials; the
// consumer of the product (an epilogue kernel) sums the splits in a fixed order, so results are
// deterministic.
#include "common.h"
#include "kernels.h"

namespace df {

// ------------------------------------------------------------------------------------------------------
// skinny MFMA GEMM (bfloat16), M <= 16 * MT
// ------------------------------------------------------------------------------------------------------
// Workgroup = 4 waves on the same 64 output columns (4 n-tiles of 16); wave w takes the k-range
// [k0 + w * kpw, k0 + (w + 1) * kpw) of the workgroup's split.  Per 256-wide k-chunk a lane loads, for each
// n-tile, eight 16-byte pieces of one weight row (A operand: row = lane % 16, k = 32 j + 8 (lane / 16)) and
// the matching eight pieces of its activation row (B operand), then issues 8 MFMAs per (n-tile, m-tile).
template <int MT>
__global__ __launch_bounds__(256) void gemm_skinny_bf16(const bf16_t* __restrict__ x, int ldx, int M, Segs w,
                                                        int N, int K, int kpw, float* __restrict__ part) {
    constexpr int NT = 4;
    __shared__ f32x4 red[4][NT * MT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64;
    const int s = blockIdx.y;
    const int kb = s * 4 * kpw + wave * kpw;
    const int ke = min(K, kb + kpw);

    const bf16_t* wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int n = min(n0 + nt * 16 + r, N - 1);
        wrow[nt] = (const bf16_t*)seg_row(w, n, K, 2) + g * 8;
    }
    const bf16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrow[mt] = x + (size_t)min(mt * 16 + r, M - 1) * ldx + g * 8;

    f32x4 acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kc = kb; kc < ke; kc += 256) {
        u32x4 wf[NT][8];
        u32x4 xf[MT][8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                wf[nt][j] = ld16_nt(wrow[nt] + kc + j * 32);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 8; ++j) xf[mt][j] = ld16(xrow[mt] + kc + j * 32);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = mfma16(wf[nt][j], xf[mt][j], acc[nt][mt]);
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
            f32x4 u = red[q][t][l];
            v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
        }
        const int m = mt * 16 + (l & 15);
        const int n = n0 + nt * 16 + 4 * (l >> 4);
        if (m >= M || n >= N) continue;
        float* dst = part + ((size_t)s * M + m) * N + n;
        if ((N & 3) == 0 && n + 3 < N) {
            *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            for (int i = 0; i < 4 && n + i < N; ++i) dst[i] = v[i];
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// LDS-tiled MFMA GEMM (bfloat16) for large M
// ------------------------------------------------------------------------------------------------------
// Tile 128 (n) x 128 (m) x 64 (k); 4 waves in a 2 x 2 grid, each owning 64 x 64 = 4 x 4 MFMA tiles.  The
// next k-tile is fetched into registers while the current one is consumed from LDS (one barrier pair per
// k-tile).  Rows are padded to 72 elements in LDS to spread the 16-byte reads over the banks.
#define TL_BN 128
#define TL_BM 128
#define TL_BK 64
#define TL_LD (TL_BK + 8)

__global__ __launch_bounds__(256) void gemm_tiled_bf16(const bf16_t* __restrict__ x, int ldx, int M, Segs w,
                                                       int N, int K, int kps, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) bf16_t sw[TL_BN * TL_LD];
    __shared__ __attribute__((aligned(16))) bf16_t sx[TL_BM * TL_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const int n0 = blockIdx.x * TL_BN, m0 = blockIdx.y * TL_BM, s = blockIdx.z;
    const int kb = s * kps, ke = min(K, kb + kps);

    // global -> register staging: each thread moves 4 pieces of 16 bytes of W and of x per k-tile
    const bf16_t* wsrc[4];
    const bf16_t* xsrc[4];
    int lrow[4], lcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = tid + 256 * i;
        lrow[i] = c >> 3;
        lcol[i] = (c & 7) * 8;
        wsrc[i] = (const bf16_t*)seg_row(w, min(n0 + lrow[i], N - 1), K, 2) + lcol[i];
        xsrc[i] = x + (size_t)min(m0 + lrow[i], M - 1) * ldx + lcol[i];
    }
    u32x4 pw[4], px[4];
    auto fetch = [&](int k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = ld16_nt(wsrc[i] + k);
            px[i] = ld16(xsrc[i] + k);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)(sw + lrow[i] * TL_LD + lcol[i]) = pw[i];
            *(u32x4*)(sx + lrow[i] * TL_LD + lcol[i]) = px[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kb < ke) fetch(kb);
    for (int k = kb; k < ke; k += TL_BK) {
        __syncthreads();
        stash();
        __syncthreads();
        if (k + TL_BK < ke) fetch(k + TL_BK);
#pragma unroll
        for (int ks = 0; ks < TL_BK / 32; ++ks) {
            u32x4 af[4], bfr[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = ld16(sw + (wn * 64 + t * 16 + r) * TL_LD + ks * 32 + g * 8);
                bfr[t] = ld16(sx + (wm * 64 + t * 16 + r) * TL_LD + ks * 32 + g * 8);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
        }
    }

    // D lane l: n = 4 (l / 16) + i, m = l % 16 within each 16 x 16 tile
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = n0 + wn * 64 + a * 16 + 4 * g;
            const int m = m0 + wm * 64 + b * 16 + r;
            if (m >= M || n >= N) continue;
            float* dst = part + ((size_t)s * M + m) * N + n;
            f32x4 v = acc[a][b];
            if ((N & 3) == 0 && n + 3 < N) {
                *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                for (int i = 0; i < 4 && n + i < N; ++i) dst[i] = v[i];
            }
        }
}

// ------------------------------------------------------------------------------------------------------
// float32 VALU GEMM (float32 drafters)
// ------------------------------------------------------------------------------------------------------
// One wave per output column n: lanes read 16 contiguous bytes each of the weight row (coalesced), keep
// one partial sum per activation row, and reduce across the wave.
__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ x, int ldx, int M, Segs w, int N, int K,
                                                float* __restrict__ part) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const float* wr = (const float*)seg_row(w, n, K, 4);
    for (int m0 = 0; m0 < M; m0 += 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int k = lane * 4; k < K; k += 256) {
            float4 wv = *(const float4*)(wr + k);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int m = min(m0 + i, M - 1);
                float4 xv = *(const float4*)(x + (size_t)m * ldx + k);
                acc[i] += wv.x * xv.x + wv.y * xv.y + wv.z * xv.z + wv.w * xv.w;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float t = wave_sum(acc[i]);
            if (lane == 0 && m0 + i < M) part[(size_t)(m0 + i) * N + n] = t;
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// launch planning
// ------------------------------------------------------------------------------------------------------

GemmPlan plan_gemm(int dtype_bf16, int M, int N, int K) {
    GemmPlan p{};
    if (!dtype_bf16) {
        p.kind = GEMM_F32;
        p.splits = 1;
        return p;
    }
    if (M <= 32) {
        p.kind = M <= 16 ? GEMM_SKINNY1 : GEMM_SKINNY2;
        const int groups = (N + 63) / 64;
        const int chunks = (K + 255) / 256;             // 256-wide k-chunks
        // aim for >= 512 workgroups (2 per CU, 8 waves per CU) with at least one chunk per wave
        int want = (512 + groups - 1) / groups;
        int max_splits = (chunks + 3) / 4;
        int splits = want < 1 ? 1 : (want > max_splits ? max_splits : want);
        int kpw_chunks = (chunks + 4 * splits - 1) / (4 * splits);
        p.kpw = kpw_chunks * 256;
        p.splits = (K + 4 * p.kpw - 1) / (4 * p.kpw);
        return p;
    }
    p.kind = GEMM_TILED;
    const int tiles = ((N + TL_BN - 1) / TL_BN) * ((M + TL_BM - 1) / TL_BM);
    const int kt = (K + TL_BK - 1) / TL_BK;
    int splits = tiles >= 256 ? 1 : (384 + tiles - 1) / tiles;
    if (splits > kt / 4) splits = kt / 4 > 0 ? kt / 4 : 1;
    int kps_tiles = (kt + splits - 1) / splits;
    p.kps = kps_tiles * TL_BK;
    p.splits = (K + p.kps - 1) / p.kps;
    return p;
}

hipError_t launch_gemm(const GemmPlan& p, const void* x, int ldx, int M, const Segs& w, int N, int K, float* part,
                       hipStream_t st) {
    switch (p.kind) {
        case GEMM_SKINNY1:
            hipLaunchKernelGGL(gemm_skinny_bf16<1>, dim3((N + 63) / 64, p.splits), dim3(256), 0, st,
                               (const bf16_t*)x, ldx, M, w, N, K, p.kpw, part);
            break;
        case GEMM_SKINNY2:
            hipLaunchKernelGGL(gemm_skinny_bf16<2>, dim3((N + 63) / 64, p.splits), dim3(256), 0, st,
                               (const bf16_t*)x, ldx, M, w, N, K, p.kpw, part);
            break;
        case GEMM_TILED:
            hipLaunchKernelGGL(gemm_tiled_bf16, dim3((N + TL_BN - 1) / TL_BN, (M + TL_BM - 1) / TL_BM, p.splits),
                               dim3(256), 0, st, (const bf16_t*)x, ldx, M, w, N, K, p.kps, part);
            break;
        case GEMM_F32:
            hipLaunchKernelGGL(gemm_f32, dim3((N + 3) / 4), dim3(256), 0, st, (const float*)x, ldx, M, w, N, K, part);
            break;
    }
    return hipGetLastError();
}

const char* gemm_kernel_name(const GemmPlan& p) {
    switch (p.kind) {
        case GEMM_SKINNY1: return "gemm_skinny_bf16_m16";
        case GEMM_SKINNY2: return "gemm_skinny_bf16_m32";
        case GEMM_TILED: return "gemm_tiled_bf16";
        default: return "gemm_f32";
    }
}

}  // namespace df
