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
// Two workgroups share a CU (the head's 66 KB logits tile sets the LDS per workgroup), so one workgroup's
// row reductions overlap the other's MFMAs (the head's epilogue is too long to leave exposed, as it would be
// with one wide workgroup per CU).  With two workgroups per CU the register staging stays: the wide loop's
// direct-to-LDS stages, with the one or two tiles in flight that fit in this LDS, measured slower here.
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
// Workgroup tile 32 NT (n) x 128 (m); 4 waves in a 2 x 2 grid, each owning 16 NT x 64 = NT x 4 MFMA tiles
// (NT = 8: 256-wide tiles; NT = 6: 192-wide, for widths that then fill whole generations of workgroups).  Both
// activation planes accumulate into the same accumulators.
//
// K is consumed in k-tiles of 32 (one MFMA k-step) through WD_STAGES LDS stages, filled by direct
// global -> LDS loads (`global_load_lds_dwordx4`: each lane's 16 bytes land at the wave's LDS base + 16 lane),
// with no staging registers and no LDS store instructions.  A stage holds the k-tile's 2 NT weight fragments as
// packed (1 KB each, lane-linear) and its activation fragments, loaded directly in MFMA B-operand order (lane
// l: row l % 16 of the m-tile, k 8 (l / 16) .. + 7), so that every operand read is one conflict-free 1 KB
// read.  Each k-tile step issues the loads of the tile WD_STAGES - 1 ahead, so two tiles stay in flight
// behind the one waited for; steps past the last tile re-load it into a stage nobody reads, which keeps that
// count fixed (one wait constant) and is drained before the workgroup exits.  The waits are explicit
// (`s_waitcnt vmcnt`, then `s_barrier`): __syncthreads would wait for every load in flight.
//
// Within a k-tile the second plane's fragments are read during the first plane's MFMAs, and the next tile's
// first fragments during the second plane's MFMAs (after the barrier that publishes that tile).
//
// Measured at M = 256 (Qwen3-8B shapes; cold weights, per launch): gate/up 127 -> 111 us, down 65 -> 55,
// QKV 38 -> 32, O 30 -> 25 against the same tiles staged through registers and LDS stores.  Isolated,
// those stores and their waits on the global loads cost about a third of the old main loop.
#define WD_BM 128
#define WD_BK 64  // granularity of a split's k-range (two k-tiles)
#define WD_KT 32  // k-tile of the main loop
#define WD_STAGES 4
__host__ __device__ constexpr int wd_bn(int nt) { return 32 * nt; }
// LDS elements of one stage: 2 NT weight fragments + 8 activation fragments per plane
__host__ __device__ constexpr int wd_stage(int nt, bool split) { return (2 * nt + (split ? 16 : 8)) * DF_FRAG; }
__host__ __device__ constexpr int wd_lds_elems(int nt, bool split) { return WD_STAGES * wd_stage(nt, split); }

typedef __attribute__((address_space(3))) void df_lds_void;
typedef __attribute__((address_space(1))) void df_global_void;
// 16 bytes per lane from global memory straight into LDS at (wave-uniform) l + 16 * lane
__device__ __forceinline__ void dma16(const bf16_t* g, bf16_t* l) {
    __builtin_amdgcn_global_load_lds((df_global_void*)g, (df_lds_void*)l, 16, 0, 0);
}
// s_waitcnt: vector-memory count <= n and LDS count 0 (gfx9 encoding; export count not waited on)
#define WD_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

// acc[a][b]: n-tile a, m-tile b of this wave's block, for the k-range [kb, ke) (a multiple of WD_BK) of the
// tile at (n0, m0).  lds holds wd_lds_elems(NT, SPLIT) elements.  With SPLIT the activation is a pair of
// bfloat16 planes (lo plane at x + xplane) and every weight fragment meets hi and lo.
template <bool SPLIT, int NT>
static __device__ __forceinline__ void wide_mainloop(const bf16_t* __restrict__ x, int ldx, size_t xplane, int M,
                                                     const bf16_t* __restrict__ wp, int N, int n0, int m0, int kb,
                                                     int ke, bf16_t* lds, f32x4 (&acc)[NT][4]) {
    constexpr int XP = SPLIT ? 2 : 1;
    constexpr int NWF = 2 * NT, NXF = 8 * XP;                      // fragments per k-tile
    constexpr int STAGE = wd_stage(NT, SPLIT);
    constexpr int WPW = NWF / 4, XPW = NXF / 4, DPT = WPW + XPW;  // loads per wave per k-tile
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    const size_t G = packed_groups(N), tlast = 4 * G - 1;
    // This wave loads weight fragments (n-tiles) wave * WPW + i of the tile (n-tiles past the padded groups
    // read the last padded tile; their columns are discarded) and activation fragments f = wave * XPW + i:
    // plane f / 8, m-tile f % 8 (rows past M read row M - 1; their results are discarded).
    const bf16_t* wsrc[WPW];
    const bf16_t* xsrc[XPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i)
        wsrc[i] = wp + frag_index(min((size_t)(n0 / 16 + wave * WPW + i), tlast), 0, G) * DF_FRAG + lane * 8;
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int f = wave * XPW + i;
        xsrc[i] = x + (size_t)min(m0 + (f & 7) * 16 + r, M - 1) * ldx + (f >> 3) * xplane + g * 8;
    }
    const int T = (ke - kb) / WD_KT;
    auto issue = [&](int t, int st) {  // the loads of k-tile t into stage st
        const int k = kb + WD_KT * min(t, T - 1);
        bf16_t* sb = lds + st * STAGE;
        const size_t fk = frag_index(0, k / 32, G) * DF_FRAG;
#pragma unroll
        for (int i = 0; i < WPW; ++i) dma16(wsrc[i] + fk, sb + (wave * WPW + i) * DF_FRAG);
#pragma unroll
        for (int i = 0; i < XPW; ++i) dma16(xsrc[i] + k, sb + (NWF + wave * XPW + i) * DF_FRAG);
        asm volatile("" ::: "memory");  // issued before the next wait counts them
    };
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (T <= 0) return;
    u32x4 Aa[NT], Ab[NT], B0a[4], B0b[4], B1[4];
#define WD_RA(st, A)                                                                                           \
    _Pragma("unroll") for (int a = 0; a < NT; ++a) A[a] = ld16(lds + (st) * STAGE + (wn * NT + a) * DF_FRAG + lane * 8)
#define WD_RB(st, pl, B)                                                                                       \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) B[q] =                                                       \
        ld16(lds + (st) * STAGE + (NWF + (pl) * 8 + wm * 4 + q) * DF_FRAG + lane * 8)
#define WD_MM(A, B)                                                                                            \
    _Pragma("unroll") for (int a = 0; a < NT; ++a) _Pragma("unroll") for (int q = 0; q < 4; ++q) acc[a][q] =  \
        mfma16(A[a], B[q], acc[a][q])
// n_ds LDS reads, each followed by n_mm MFMAs
#define WD_INTERLEAVE(n_ds, n_mm)                                                                              \
    do {                                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < (n_ds); ++i_) {                                                \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                 \
            __builtin_amdgcn_sched_group_barrier(0x008, (n_mm), 0);                                            \
        }                                                                                                      \
    } while (0)
// the next tile's loads done (two tiles stay in flight), this wave's LDS reads done, then the barrier
#define WD_PUBLISH()                                                                                           \
    do {                                                                                                       \
        WD_WAIT_VM((WD_STAGES - 2) * DPT);                                                                     \
        asm volatile("" ::: "memory");                                                                         \
        __builtin_amdgcn_s_barrier();                                                                          \
        asm volatile("" ::: "memory");                                                                         \
    } while (0)
// k-tile t in stage ST (a constant: a run-time stage index made the compiler copy the accumulators around
// every MFMA).  Entering, A / B0 hold its weight and first-plane fragments; leaving, An / B0n hold the next
// tile's (after the last tile they are read from a stale stage and not used).
#define WD_TILE(t, ST, A, B0, An, B0n)                                                                         \
    do {                                                                                                       \
        issue((t) + WD_STAGES - 1, ((ST) + WD_STAGES - 1) % WD_STAGES);                                        \
        if constexpr (SPLIT) {                                                                                 \
            WD_RB(ST, 1, B1);                                                                                  \
            WD_MM(A, B0);                                                                                      \
            WD_INTERLEAVE(4, 8);                                                                               \
            WD_PUBLISH();                                                                                      \
            WD_RA(((ST) + 1) % WD_STAGES, An);                                                                 \
            WD_RB(((ST) + 1) % WD_STAGES, 0, B0n);                                                             \
            WD_MM(A, B1);                                                                                      \
            WD_INTERLEAVE(NT + 4, 2);                                                                          \
        } else {                                                                                               \
            WD_PUBLISH();                                                                                      \
            WD_RA(((ST) + 1) % WD_STAGES, An);                                                                 \
            WD_RB(((ST) + 1) % WD_STAGES, 0, B0n);                                                             \
            WD_MM(A, B0);                                                                                      \
            WD_INTERLEAVE(NT + 4, 2);                                                                          \
        }                                                                                                      \
    } while (0)
    static_assert(WD_STAGES == 4, "the k-tile loop below is unrolled over four stages");
#pragma unroll
    for (int j = 0; j < WD_STAGES - 1; ++j) issue(j, j);
    WD_PUBLISH();
    WD_RA(0, Aa);
    WD_RB(0, 0, B0a);
    // (tiles guarded one by one inside the four-stage loop: a remainder after the loop, or one guard around a
    // pair of tiles, also brought back the accumulator copies)
    for (int t = 0; t < T; t += 4) {
        WD_TILE(t, 0, Aa, B0a, Ab, B0b);
        if (t + 1 < T) WD_TILE(t + 1, 1, Ab, B0b, Aa, B0a);
        if (t + 2 < T) WD_TILE(t + 2, 2, Aa, B0a, Ab, B0b);
        if (t + 3 < T) WD_TILE(t + 3, 3, Ab, B0b, Aa, B0a);
    }
    WD_WAIT_VM(0);  // the re-loads past the last tile land before the workgroup exits
#undef WD_TILE
#undef WD_PUBLISH
#undef WD_INTERLEAVE
#undef WD_MM
#undef WD_RB
#undef WD_RA
}
