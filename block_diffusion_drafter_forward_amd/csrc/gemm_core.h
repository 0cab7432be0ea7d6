// Packed weight layout and the main loop of the LDS-tiled MFMA GEMM, shared by the large-M projection
// kernel and the large-M LM head.
#pragma once

#include "common.h"

// ------------------------------------------------------------------------------------------------------
// packed ("fragment-major") weights
// ------------------------------------------------------------------------------------------------------
// A bfloat16 matrix W[N][K] (K a multiple of 256) is stored as fragments of 16 rows x 32 k-values.  Inside a
// fragment, lane l of a wave owns the 16 bytes at offset 8 l: row 16 t + (l % 16), k = 32 s + 8 (l / 16) ..
// + 7 -- exactly the A operand of one 16x16x32 MFMA, so a wave fetches a whole fragment with one fully
// coalesced 1 KB load.  The fragments are ordered chunk-major: the n-tiles are taken four at a time (group
// g = t / 4 of 64 rows; N is padded with zero rows to whole groups) and K in chunks of 256 (eight
// fragments), and fragment (t, s) sits at fragment index ((s / 8) * G + t / 4) * 32 + (t % 4) * 8 + s % 8,
// G = ceil(N / 64).  The 32 KB one wave streams per k-chunk (four n-tiles x eight fragments) is then one
// contiguous block, and the waves of neighbouring workgroups at the same chunk read neighbouring blocks:
// measured on MI355X, this streams 6-37% faster than an n-tile-major order (the gain is largest for the
// smallest matrices).  Matrices that one GEMM stacks along N are packed together as one matrix.
#define DF_FRAG 512  // elements per fragment
__host__ __device__ inline size_t packed_groups(int N) { return (size_t)((N + 63) / 64); }
__host__ __device__ inline size_t packed_elems(int N, int K) { return packed_groups(N) * 64 * (size_t)K; }
// fragment index of n-tile t, k-step s in a matrix of G groups
__host__ __device__ inline size_t frag_index(size_t t, int s, size_t G) {
    return (((size_t)(s >> 3) * G + (t >> 2)) * 4 + (t & 3)) * 8 + (s & 7);
}

// ------------------------------------------------------------------------------------------------------
// LDS-tiled MFMA GEMM (bfloat16) for large M
// ------------------------------------------------------------------------------------------------------
// Tile 128 (n) x 128 (m) x 64 (k); 4 waves in a 2 x 2 grid, each owning 64 x 64 = 4 x 4 MFMA tiles.  The
// next k-tile is fetched into registers while the current one is consumed from LDS (one barrier pair per
// k-tile).  The weight tile is 16 packed fragments, copied to LDS as they are (conflict-free 1 KB reads per
// MFMA operand); activation rows are padded to 72 elements in LDS to spread the 16-byte reads over the banks.
// Tile (x = n-tile, y = m-tile) of workgroup `bid` of a one-dimensional grid of xcd_tile_count(gx, gy)
// workgroups.  Workgroups are dispatched to the eight XCDs round-robin, so workgroups i and i + 8 run on the
// same XCD at about the same time: the m-tiles of one n-tile are placed 8 apart, and the second one finds the
// weight tile in that XCD's L2 instead of reading it from HBM again.  Returns false for the padding
// workgroups of the last column of eight.
__device__ __forceinline__ bool xcd_tile(int bid, int gx, int gy, int& x, int& y) {
    const int rest = bid >> 3;
    y = rest % gy;
    x = (rest / gy) * 8 + (bid & 7);
    return x < gx;
}
__host__ __device__ inline int xcd_tile_count(int gx, int gy) { return (gx + 7) / 8 * 8 * gy; }

#define TL_BN 128
#define TL_BM 128
#define TL_BK 64
#define TL_LD (TL_BK + 8)
#define TL_SW (16 * DF_FRAG)  // elements of the LDS weight tile

// Main loop of the tiled kernel: acc[a][b] (n-tile a, m-tile b of this wave's 64 x 64 block) for the k-range
// [kb, ke).  wp is the packed weight matrix (N x K); sw / sx are LDS staging buffers of TL_SW and
// TL_BM * TL_LD elements.  With SPLIT the activation is a pair of bfloat16 planes (lo plane at x + xplane):
// sx holds both planes (2 * TL_BM * TL_LD elements) and every weight fragment meets hi and lo.
template <bool SPLIT>
static __device__ __forceinline__ void tiled_mainloop(const bf16_t* __restrict__ x, int ldx, size_t xplane, int M,
                                                      const bf16_t* __restrict__ wp, int N, int K, int n0, int m0,
                                                      int kb, int ke, bf16_t* sw, bf16_t* sx, f32x4 (&acc)[4][4]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const size_t G = packed_groups(N);
    // global -> register staging: each thread moves 4 pieces of 16 bytes of W and of x per k-tile.  Weight
    // piece c = tid + 256 i is lane (c % 64) of fragment c / 64 = (n-tile, k-step) = ((c / 64) / 2, (c / 64) % 2)
    // of the tile; n-tiles past the padded groups read the last padded tile (their columns are discarded).
    const bf16_t* wsrc[4];
    const bf16_t* xsrc[4];
    int lrow[4], lcol[4], wks[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, f = c >> 6;
        const size_t t = min((size_t)(n0 / 16 + (f >> 1)), 4 * G - 1);
        wsrc[i] = wp + frag_index(t, 0, G) * DF_FRAG + (c & 63) * 8;  // k-step 0; add the k-step part below
        wks[i] = f & 1;
        lrow[i] = c >> 3;
        lcol[i] = (c & 7) * 8;
        xsrc[i] = x + (size_t)min(m0 + lrow[i], M - 1) * ldx + lcol[i];
    }
    constexpr int XP = SPLIT ? 2 : 1;
    u32x4 pw[4], px[XP][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb < ke) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = ld16_nt(wsrc[i] + frag_index(0, kb / 32 + wks[i], G) * DF_FRAG);
#pragma unroll
            for (int pl = 0; pl < XP; ++pl) px[pl][i] = ld16(xsrc[i] + pl * xplane + kb);
        }
    }
    for (int k = kb; k < ke; k += TL_BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4*)(sw + (tid + 256 * i) * 8) = pw[i];
#pragma unroll
            for (int pl = 0; pl < XP; ++pl) *(u32x4*)(sx + (pl * TL_BM + lrow[i]) * TL_LD + lcol[i]) = px[pl][i];
        }
        __syncthreads();
        if (k + TL_BK < ke) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[i] = ld16_nt(wsrc[i] + frag_index(0, (k + TL_BK) / 32 + wks[i], G) * DF_FRAG);
#pragma unroll
                for (int pl = 0; pl < XP; ++pl) px[pl][i] = ld16(xsrc[i] + pl * xplane + k + TL_BK);
            }
        }
#pragma unroll
        for (int ks = 0; ks < TL_BK / 32; ++ks) {
            u32x4 af[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) af[t] = ld16(sw + (((wn * 4 + t) * 2 + ks) * 64 + lane) * 8);
#pragma unroll
            for (int pl = 0; pl < XP; ++pl) {
                u32x4 bfr[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    bfr[t] = ld16(sx + (pl * TL_BM + wm * 64 + t * 16 + r) * TL_LD + ks * 32 + g * 8);
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
            }
        }
    }
}
