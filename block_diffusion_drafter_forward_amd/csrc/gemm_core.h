// Packed weight layout and the main loops of the large-M MFMA kernels: the wide-tile projection GEMM and the
// LDS-tiled LM head.
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
// workgroup -> tile order
// ------------------------------------------------------------------------------------------------------
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

// ------------------------------------------------------------------------------------------------------
// LDS-tiled MFMA main loop (bfloat16) of the large-M LM head
// ------------------------------------------------------------------------------------------------------
// Tile 128 (n) x 128 (m) x 64 (k); 4 waves in a 2 x 2 grid, each owning 64 x 64 = 4 x 4 MFMA tiles.  The
// next k-tile is fetched into registers while the current one is consumed from LDS (one barrier pair per
// k-tile).  The weight tile is 16 packed fragments, copied to LDS as they are (conflict-free 1 KB reads per
// MFMA operand); activation rows are padded to 72 elements in LDS to spread the 16-byte reads over the banks.
// Three workgroups share a CU, so one workgroup's row reductions overlap the others' MFMAs (the head's
// epilogue is too long to leave exposed, as it would be with one wide workgroup per CU).
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

// ------------------------------------------------------------------------------------------------------
// wide-tile MFMA main loop (bfloat16), one workgroup of four waves per CU
// ------------------------------------------------------------------------------------------------------
// Workgroup tile 32 NT (n) x 128 (m) x 64 (k); 4 waves in a 2 x 2 grid, each owning 16 NT x 64 = NT x 4
// MFMA tiles (NT = 8: 256-wide tiles; NT = 6: 192-wide, for widths that then fill whole generations of
// workgroups).  A k-step reads NT weight and 4 activation fragments (per plane) from LDS for 4 NT MFMAs
// (8 NT with both planes): 256 bytes of LDS per MFMA at NT = 8, against 384 for 64 x 64 wave tiles, which
// kept the 128 x 128 tile LDS-bound.  Both activation planes accumulate into the same accumulators.  LDS is
// double-buffered and the registers hold two staging sets: while tile k is consumed, tile k + 1 waits in the
// other LDS buffer and tile k + 2's loads are in flight, one barrier per k-tile.  The buffers take
// 2 * (4 NT fragments + one 128 x 72 activation tile per plane): 139 KB at NT = 8 with both planes, so one
// workgroup per CU with the registers of a whole SIMD per wave (the accumulators live in AGPRs).
#define WD_BM 128
#define WD_BK 64
#define WD_LD (WD_BK + 8)
#define WD_SX (WD_BM * WD_LD)  // activation tile of one plane, rows padded to 72 elements
__host__ __device__ constexpr int wd_bn(int nt) { return 32 * nt; }
__host__ __device__ constexpr int wd_sw(int nt) { return 4 * nt * DF_FRAG; }  // 2 NT n-tiles x 2 k-steps
__host__ __device__ constexpr int wd_lds_elems(int nt, bool split) {
    return 2 * (wd_sw(nt) + (split ? 2 : 1) * WD_SX);
}

// acc[a][b]: n-tile a, m-tile b of this wave's block, for the k-range [kb, ke) of the tile at (n0, m0).  lds
// holds wd_lds_elems(NT, SPLIT) elements.  With SPLIT the activation is a pair of bfloat16 planes (lo plane
// at x + xplane) and every weight fragment meets hi and lo.
template <bool SPLIT, int NT>
static __device__ __forceinline__ void wide_mainloop(const bf16_t* __restrict__ x, int ldx, size_t xplane, int M,
                                                     const bf16_t* __restrict__ wp, int N, int n0, int m0, int kb,
                                                     int ke, bf16_t* lds, f32x4 (&acc)[NT][4]) {
    constexpr int XP = SPLIT ? 2 : 1;
    constexpr int SW = wd_sw(NT), SXB = XP * WD_SX;
    bf16_t* const sw[2] = {lds, lds + SW};
    bf16_t* const sx[2] = {lds + 2 * SW, lds + 2 * SW + SXB};
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const size_t G = packed_groups(N);
    // Weight piece c = tid + 256 i (i < NT) is lane c % 64 of fragment c / 64 = (n-tile, k-step) =
    // ((c / 64) / 2, (c / 64) % 2) = (wave / 2 + 2 i, wave % 2); n-tiles past the padded groups read the last
    // padded tile (their columns are discarded).  Activation piece c = tid + 256 i (i < 4): row c / 8 =
    // tid / 8 + 32 i, k (c % 8) * 8 = (tid % 8) * 8.  Addresses are formed per load.
    const size_t tlast = 4 * G - 1;
    const int t0 = n0 / 16 + (wave >> 1), wk = wave & 1;
    const bf16_t* wlane = wp + (size_t)lane * 8;
    const int xrow = tid >> 3, xcol = (tid & 7) * 8;
    u32x4 pwa[NT], pxa[XP][4], pwb[NT], pxb[XP][4];
#define WD_FETCH(k, PW, PX)                                                                                    \
    do {                                                                                                       \
        const size_t fk = frag_index(0, (k) / 32 + wk, G);                                                     \
        _Pragma("unroll") for (int i = 0; i < NT; ++i) PW[i] =                                                \
            ld16_nt(wlane + (frag_index(min((size_t)(t0 + 2 * i), tlast), 0, G) + fk) * DF_FRAG);              \
        _Pragma("unroll") for (int pl = 0; pl < XP; ++pl)                                                      \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) PX[pl][i] =                                          \
                ld16(x + (size_t)min(m0 + xrow + 32 * i, M - 1) * ldx + pl * xplane + xcol + (k));            \
    } while (0)
#define WD_STASH(b, PW, PX)                                                                                    \
    do {                                                                                                       \
        _Pragma("unroll") for (int i = 0; i < NT; ++i) * (u32x4*)(sw[b] + (tid + 256 * i) * 8) = PW[i];        \
        _Pragma("unroll") for (int pl = 0; pl < XP; ++pl)                                                      \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) *                                                    \
                (u32x4*)(sx[b] + pl * WD_SX + (xrow + 32 * i) * WD_LD + xcol) = PX[pl][i];                     \
    } while (0)
#define WD_COMPUTE(b)                                                                                          \
    do {                                                                                                       \
        const bf16_t* cw = sw[b];                                                                              \
        const bf16_t* cx = sx[b];                                                                              \
        _Pragma("unroll") for (int ks = 0; ks < WD_BK / 32; ++ks) {                                            \
            u32x4 af[NT];                                                                                      \
            _Pragma("unroll") for (int a = 0; a < NT; ++a) af[a] =                                            \
                ld16(cw + (((wn * NT + a) * 2 + ks) * 64 + lane) * 8);                                         \
            _Pragma("unroll") for (int pl = 0; pl < XP; ++pl) {                                                \
                u32x4 bfr[4];                                                                                  \
                _Pragma("unroll") for (int q = 0; q < 4; ++q) bfr[q] =                                         \
                    ld16(cx + pl * WD_SX + (wm * 64 + q * 16 + r) * WD_LD + ks * 32 + g * 8);                   \
                _Pragma("unroll") for (int a = 0; a < NT; ++a)                                                 \
                    _Pragma("unroll") for (int q = 0; q < 4; ++q) acc[a][q] = mfma16(af[a], bfr[q], acc[a][q]); \
            }                                                                                                  \
        }                                                                                                      \
    } while (0)
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // tile j of the range sits in LDS buffer j % 2 and is staged in register set j % 2
    if (kb < ke) WD_FETCH(kb, pwa, pxa);
    if (kb + WD_BK < ke) WD_FETCH(kb + WD_BK, pwb, pxb);
    if (kb < ke) WD_STASH(0, pwa, pxa);
    __syncthreads();
    int k = kb;
    for (; k + WD_BK < ke; k += 2 * WD_BK) {
        // tile k in buffer 0, tile k + 64 in set b, set a free
        if (k + 2 * WD_BK < ke) WD_FETCH(k + 2 * WD_BK, pwa, pxa);
        WD_COMPUTE(0);
        WD_STASH(1, pwb, pxb);
        __syncthreads();
        // tile k + 64 in buffer 1, tile k + 128 (if any) in set a
        if (k + 3 * WD_BK < ke) WD_FETCH(k + 3 * WD_BK, pwb, pxb);
        WD_COMPUTE(1);
        if (k + 2 * WD_BK < ke) WD_STASH(0, pwa, pxa);
        __syncthreads();
    }
    if (k < ke) WD_COMPUTE(0);  // an odd last tile, already in buffer 0
#undef WD_FETCH
#undef WD_STASH
#undef WD_COMPUTE
}
