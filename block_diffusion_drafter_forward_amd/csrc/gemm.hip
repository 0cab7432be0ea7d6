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
#include "gemm_core.h"
#include "kernels.h"

namespace df {

// ------------------------------------------------------------------------------------------------------
// weight packing (once per weight matrix, into the fragment-major layout of gemm_core.h)
// ------------------------------------------------------------------------------------------------------
// One thread per 16-byte lane piece of the packed image: piece c is lane c % 64 of fragment c / 64, whose
// (n-tile, k-step) inverts the chunk-major fragment index.  Row n of the stacked matrix is row n - start[i]
// of segment i; rows past N are zero.
__global__ __launch_bounds__(256) void pack_frag(Segs src, int N, int K, bf16_t* __restrict__ dst, size_t pieces) {
    const size_t G = packed_groups(N);
    for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < pieces; c += (size_t)gridDim.x * 256) {
        const size_t f = c >> 6;
        const int l = (int)(c & 63);
        const size_t rest = f >> 5;  // chunk * G + group
        const size_t t = (rest % G) * 4 + ((f >> 3) & 3);
        const int s = (int)(rest / G) * 8 + (int)(f & 7);
        const size_t n = t * 16 + (l & 15);
        const int k = s * 32 + (l >> 4) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n < (size_t)N) v = ld16((const bf16_t*)seg_row(src, (int)n, K, 2) + k);
        *(u32x4*)(dst + c * 8) = v;
    }
}

hipError_t launch_pack(const Segs& src, int N, int K, void* dst, hipStream_t st) {
    const size_t pieces = packed_elems(N, K) / 8;
    const size_t blocks = (pieces + 255) / 256;
    hipLaunchKernelGGL(pack_frag, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st, src, N, K,
                       (bf16_t*)dst, pieces);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// skinny MFMA GEMM (bfloat16), M <= 16 * MT, packed weights
// ------------------------------------------------------------------------------------------------------
// Workgroup = W waves (4, 8 or 2: see plan_gemm) on the same 64 output columns (4 n-tiles of 16); wave w takes
// the k-range [k0 + w * kpw, k0 + (w + 1) * kpw) of the workgroup's split.  Per 256-wide k-chunk a wave loads, for each
// n-tile, eight packed weight fragments (one coalesced 1 KB load each: the A operand, row = lane % 16,
// k = 32 j + 8 (lane / 16)) and the matching eight 16-byte pieces of its activation row (B operand), then
// issues 8 MFMAs per (n-tile, m-tile).  With SPLIT the activation is a pair of bfloat16 planes (x = hi + lo,
// lo plane at x + xplane) and every weight fragment meets both: two MFMAs, one weight load; at one m-tile
// the hi and lo products go to separate accumulators so that the two MFMAs do not wait on each other.
template <int MT, bool SPLIT, int W>
__global__ __launch_bounds__(64 * W) void gemm_skinny_bf16(const bf16_t* __restrict__ x, int ldx, size_t xplane, int M,
                                                           const bf16_t* __restrict__ wp, int N, int K, int kpw,
                                                           float* __restrict__ part) {
    constexpr int NT = 4;
    constexpr bool SEP = SPLIT && MT == 1;
    __shared__ f32x4 red[W][NT * MT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64;
    const int s = blockIdx.y;
    const int kb = s * W * kpw + wave * kpw;
    const int ke = min(K, kb + kpw);
    // this workgroup's four n-tiles are group blockIdx.x of the chunk-major packed matrix: per k-chunk one
    // contiguous 32 KB block, n-tile nt at fragment 8 nt of it
    const size_t chunk_stride = packed_groups(N) * 32 * DF_FRAG;
    const bf16_t* wt = wp + (size_t)blockIdx.x * 32 * DF_FRAG + lane * 8;
    const bf16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrow[mt] = x + (size_t)min(mt * 16 + r, M - 1) * ldx + g * 8;

    f32x4 acc[NT][MT], acl[SEP ? NT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (SEP) acl[SEP ? nt : 0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int kc = kb; kc < ke; kc += 256) {
        u32x4 wf[NT][8];
        u32x4 xf[MT][8];
        u32x4 xl[SPLIT ? MT : 1][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wf[nt][j] = ld16_nt(wt + (size_t)(kc / 256) * chunk_stride + (nt * 8 + j) * DF_FRAG);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                xf[mt][j] = ld16(xrow[mt] + kc + j * 32);
                if (SPLIT) xl[SPLIT ? mt : 0][j] = ld16(xrow[mt] + xplane + kc + j * 32);
            }
        }
        // issue every load of the chunk before the first MFMA: 32 KB of weights in flight per wave
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[nt][mt] = mfma16(wf[nt][j], xf[mt][j], acc[nt][mt]);
                    if (SEP) acl[SEP ? nt : 0] = mfma16(wf[nt][j], xl[0][j], acl[SEP ? nt : 0]);
                    else if (SPLIT) acc[nt][mt] = mfma16(wf[nt][j], xl[SPLIT ? mt : 0][j], acc[nt][mt]);
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

    for (int e = threadIdx.x; e < NT * MT * 64; e += 64 * W) {
        const int t = e >> 6, l = e & 63;
        const int nt = t / MT, mt = t % MT;
        f32x4 v = red[0][t][l];
#pragma unroll
        for (int q = 1; q < W; ++q) {
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
// wide-tile MFMA GEMM (bfloat16) for large M: the main loop of gemm_core.h, split-K partials out
// ------------------------------------------------------------------------------------------------------
template <bool SPLIT, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_wide_bf16(
    const bf16_t* __restrict__ x, int ldx, size_t xplane, int M, const bf16_t* __restrict__ wp, int N, int K,
    int kps, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) bf16_t lds[wd_lds_elems(NT, SPLIT)];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    int tx, ty;
    if (!xcd_tile(blockIdx.x, (N + wd_bn(NT) - 1) / wd_bn(NT), (M + WD_BM - 1) / WD_BM, tx, ty)) return;
    const int n0 = tx * wd_bn(NT), m0 = ty * WD_BM, sp = blockIdx.y;
    const int kb = sp * kps, ke = min(K, kb + kps);
    f32x4 acc[NT][4];
    wide_mainloop<SPLIT, NT>(x, ldx, xplane, M, wp, N, n0, m0, kb, ke, lds, acc);
    // D lane l: n = 4 (l / 16) + i, m = l % 16 within each 16 x 16 tile
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = n0 + wn * 16 * NT + a * 16 + 4 * g;
            const int m = m0 + wm * 64 + b * 16 + r;
            if (m >= M || n >= N) continue;
            float* dst = part + ((size_t)sp * M + m) * N + n;
            const f32x4 v = acc[a][b];
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

GemmPlan plan_gemm(int dtype_bf16, int M, int N, int K, bool few_splits) {
    GemmPlan p{};
    if (!dtype_bf16) {
        p.kind = GEMM_F32;
        p.splits = 1;
        return p;
    }
    if (M <= 32) {
        p.kind = M <= 16 ? GEMM_SKINNY1 : GEMM_SKINNY2;
        // Each wave streams kpw of K for 64 columns (32 KB of packed weights per 256-wide chunk), one chunk in
        // flight at a time.  Longer ranges mean fewer waves in flight but fewer split partials for the
        // consumer.  Measured on MI355X: one chunk per wave is best for the GEMM alone; vocabulary-sized N
        // (>= ~2000 workgroups even with four chunks) gains from four.  With few_splits (the drafter layer's
        // GEMMs, whose consumers are the row norms, the QKV epilogue and SwiGLU) the longest range of at
        // most three chunks that splits K evenly and still gives 256 or more workgroups is best:
        // gate/up 2 chunks, down 3, QKV and O 1, 7.8 us per drafter pass less than one chunk everywhere.  The
        // injection GEMMs, whose consumers are elementwise, lose 3-5 us each with longer ranges.
        const int groups = (N + 63) / 64;
        auto wgs = [&](int kpw) { return groups * ((K + 4 * kpw - 1) / (4 * kpw)); };
        p.kpw = 256;
        if (K % 1024 == 0 && wgs(1024) >= 2000) {
            p.kpw = 1024;
        } else if (few_splits) {
            for (int kpw : {768, 512}) {
                if (K % (4 * kpw) == 0 && wgs(kpw) >= 256) {
                    p.kpw = kpw;
                    break;
                }
            }
        }
        p.splits = (K + 4 * p.kpw - 1) / (4 * p.kpw);
        p.waves = 4;
        // Eight-wave workgroups, one chunk per wave, where that gives one generation of 192 to 256
        // workgroups (at most one per CU) and four-wave ones would leave some CUs with two: measured on
        // MI355X for the QKV shape (6144 x 4096: 192 instead of 384 workgroups), 11.4 us instead of 12.0 in
        // isolation, and half the split partials for its epilogue.
        if (few_splits && M <= 16 && p.kpw == 256 && K % 2048 == 0) {  // (two m-tiles would spill)
            const int w8 = groups * (K / 2048);
            if (w8 >= 192 && w8 <= 256 && wgs(256) % 256 != 0) {
                p.waves = 8;
                p.splits = K / 2048;
            }
        }
        // K a whole number of 512-wide pairs of chunks but not of 1024-wide four-wave splits (whose last split
        // leaves waves idle), and one generation of waves (eight per CU) covering every chunk: two-wave
        // workgroups, one chunk per wave, keep every wave busy and spread the workgroups over all CUs.  Where
        // that would give more than eight splits (more than one batch of the consumer's split loads), eight-wave
        // workgroups halve the splits instead.  Measured on MI355X with cold weights: QKV 6144 x 2560 8.2 us
        // with two waves instead of 9.7; down 2560 x 9728 10.9 with two waves (19 splits, its row norm +1.1)
        // or 11.7 with eight (5 splits) instead of 12.3 (10 splits); gate/up 19456 x 2560 (3040 chunks, more
        // than one generation) stays faster with four waves.
        if (few_splits && M <= 16 && p.kpw == 256 && p.waves == 4 && K % 1024 != 0 && K % 512 == 0 &&
            groups * (K / 256) <= 2048) {
            if (K / 512 <= 8) {
                p.waves = 2;
                p.splits = K / 512;
            } else {
                p.waves = 8;
                p.splits = (K + 2047) / 2048;
            }
        }
        return p;
    }
    p.kind = GEMM_TILED;
    // Wide tiles, one workgroup per CU: pick the tile width (256 or 192 columns) and the split of K by an
    // estimate of time = generations of workgroups over the 256 CUs x k-tiles per split x the k-tile time
    // (measured on MI355X with both activation planes: 2.2 us for a 256 x 128 x 64 k-tile, 1.8 us for a
    // 192-wide one) + the float32 partials written and read back by the consumer at ~5 TB/s.  At M = 256
    // (Qwen3-8B shapes) this picks gate/up 192 wide x 1 split (256 workgroups), QKV 192 x 4, O 256 x 8,
    // down 256 x 8.
    double best_us = 1e30;
    p.nt = 8;
    p.kps = K;
    for (int nt : {8, 6}) {
        const int tiles = ((N + 32 * nt - 1) / (32 * nt)) * ((M + WD_BM - 1) / WD_BM);
        const int kt = (K + WD_BK - 1) / WD_BK;
        const double ktile_us = nt == 8 ? 2.2 : 1.8;
        for (int sp = 1; sp <= 16 && sp <= kt; ++sp) {
            const int per = (kt + sp - 1) / sp;
            const int used = (kt + per - 1) / per;  // splits actually launched
            const double gens = (double)((tiles * used + 255) / 256);
            const double us = gens * per * ktile_us + (double)used * M * N * 4.0 * 2.0 / 5.0e6;
            if (us < best_us - 1e-9) {
                best_us = us;
                p.nt = nt;
                p.kps = per * WD_BK;
            }
        }
    }
    p.splits = (K + p.kps - 1) / p.kps;
    return p;
}

hipError_t launch_gemm_bf16(const GemmPlan& p, const void* x, int ldx, size_t xplane, int M, const void* wpacked,
                            int N, int K, float* part, hipStream_t st) {
    const bool split = xplane != 0;
    const dim3 gs((N + 63) / 64, p.splits);
    const bf16_t* xb = (const bf16_t*)x;
    const bf16_t* wp = (const bf16_t*)wpacked;
    switch (p.kind) {
        case GEMM_SKINNY1:
        case GEMM_SKINNY2: {
            const dim3 block(64 * p.waves);
#define DF_SKINNY(MT, SP, W) DF_LAUNCH((gemm_skinny_bf16<MT, SP, W>), gs, block, 0, st, xb, ldx, xplane, M, wp, N, K, p.kpw, part)
            const int mt = p.kind == GEMM_SKINNY1 ? 1 : 2;
            if (p.waves == 8 || p.waves == 2) {
                if (mt != 1) return hipErrorInvalidValue;
                if (p.waves == 8) { if (split) DF_SKINNY(1, true, 8); else DF_SKINNY(1, false, 8); }
                else { if (split) DF_SKINNY(1, true, 2); else DF_SKINNY(1, false, 2); }
            } else {
                if (mt == 1) { if (split) DF_SKINNY(1, true, 4); else DF_SKINNY(1, false, 4); }
                else { if (split) DF_SKINNY(2, true, 4); else DF_SKINNY(2, false, 4); }
            }
#undef DF_SKINNY
            break;
        }
        case GEMM_TILED: {
            if (p.nt != 6 && p.nt != 8) return hipErrorInvalidValue;
            const dim3 gt(xcd_tile_count((N + 32 * p.nt - 1) / (32 * p.nt), (M + WD_BM - 1) / WD_BM), p.splits);
#define DF_WIDE(SP, NT) DF_LAUNCH((gemm_wide_bf16<SP, NT>), gt, dim3(256), 0, st, xb, ldx, xplane, M, wp, N, K, p.kps, part)
            if (p.nt == 6) {
                if (split) DF_WIDE(true, 6); else DF_WIDE(false, 6);
            } else {
                if (split) DF_WIDE(true, 8); else DF_WIDE(false, 8);
            }
#undef DF_WIDE
            break;
        }
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* x, int ldx, int M, const Segs& w, int N, int K, float* part, hipStream_t st) {
    hipLaunchKernelGGL(gemm_f32, dim3((N + 3) / 4), dim3(256), 0, st, x, ldx, M, w, N, K, part);
    return hipGetLastError();
}

const char* gemm_kernel_name(const GemmPlan& p, bool pair) {
    switch (p.kind) {
        case GEMM_SKINNY1: return pair ? "gemm_skinny_bf16_m16_pair" : "gemm_skinny_bf16_m16";
        case GEMM_SKINNY2: return pair ? "gemm_skinny_bf16_m32_pair" : "gemm_skinny_bf16_m32";
        case GEMM_TILED: return pair ? "gemm_wide_bf16_pair" : "gemm_wide_bf16";
        default: return "gemm_f32";
    }
}

}  // namespace df
