// Shared LM head fused with the per-row reductions the drafter needs: max, sum of exponentials (for the
// log-sum-exp over the full vocabulary) and the top-8 (logit, id) list, ordered by logit then id; at
// temperature 1 also the row's Gumbel-max sample (best logit + Gumbel noise, drawn per logit from a
// counter-based generator).  Logits live only in registers and LDS.  Stage 1 (lm_head): one workgroup per 64 vocabulary rows, four waves
// splitting K, writes one (max, sumexp, top-8) record per block row.  Stage 2 (head_merge): one workgroup
// per block row combines the records and emits the greedy token, the top-k ids and their log-probabilities.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"
#include "philox.h"

namespace df {

#define HEAD_REC 20  // max, sumexp, 8 values, 8 ids (as int bits), sampled score and id (temperature 1 only)
// Field order: the first 16-byte word holds what the merge's first pass needs, (max, sumexp, 8th value,
// sampled score); then values 1..7 and the sampled id; then the 8 ids.
__host__ __device__ constexpr int hr_val(int j) { return j == DF_TOPK - 1 ? 2 : 4 + j; }  // value j (best first)
__host__ __device__ constexpr int hr_id(int j) { return 12 + j; }                          // id j
#define HR_SSC 3   // sampled score
#define HR_SID 11  // sampled id
// Records are stored per group, hpart[(group * rows + row) * HEAD_REC + field]: the records a workgroup of the
// LM head writes are one contiguous block (80 bytes per block row), so its stores fill whole cache lines.

// Vocabulary columns per record group: 64 for the skinny head (block rows <= 32), 128 for the tiled head.
int head_group_width(int bf16, int M) { return (bf16 && M > 32) ? 128 : 64; }
int head_groups(int V, int width) { return (V + width - 1) / width; }
size_t head_partial_floats(int bf16, int V, int M) {
    return (size_t)head_groups(V, head_group_width(bf16, M)) * M * HEAD_REC;
}

// Top-8 lists: (value, id) entries sorted best-first by df_better; empty slots hold (-inf, INT_MAX).
struct Top8 {
    float v[DF_TOPK];
    int id[DF_TOPK];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) { v[j] = -INFINITY; id[j] = 0x7FFFFFFF; }
    }
    // insertion of one entry, branch-free over the fixed length
    __device__ __forceinline__ void insert(float x, int xid) {
        float cv = x;
        int ci = xid;
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {
            const bool b = df_better(cv, ci, v[j], id[j]);
            const float tv = v[j];
            const int ti = id[j];
            v[j] = b ? cv : tv;
            id[j] = b ? ci : ti;
            cv = b ? tv : cv;
            ci = b ? ti : ci;
        }
    }
    // this := best 8 of this and o (both sorted).  Bitonic merge: the better of v[i] and o[7 - i] for every i
    // is a bitonic sequence holding the best 8 of the union; three half-cleaner stages sort it.
    __device__ __forceinline__ void merge(const float (&ov)[DF_TOPK], const int (&oid)[DF_TOPK]) {
#pragma unroll
        for (int i = 0; i < DF_TOPK; ++i) {
            const bool t = df_better(ov[DF_TOPK - 1 - i], oid[DF_TOPK - 1 - i], v[i], id[i]);
            v[i] = t ? ov[DF_TOPK - 1 - i] : v[i];
            id[i] = t ? oid[DF_TOPK - 1 - i] : id[i];
        }
#pragma unroll
        for (int d = DF_TOPK / 2; d > 0; d >>= 1)
#pragma unroll
            for (int i = 0; i < DF_TOPK; ++i)
                if ((i & d) == 0) {
                    const bool sw = df_better(v[i + d], id[i + d], v[i], id[i]);
                    const float a = v[i], b = v[i + d];
                    const int ia = id[i], ib = id[i + d];
                    v[i] = sw ? b : a;
                    id[i] = sw ? ib : ia;
                    v[i + d] = sw ? a : b;
                    id[i + d] = sw ? ia : ib;
                }
    }
    // merge with the list held by lane (lane ^ o) of the wave
    __device__ __forceinline__ void merge_lane_xor(int o) {
        float ov[DF_TOPK];
        int oid[DF_TOPK];
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {
            ov[j] = __shfl_xor(v[j], o, DF_WAVE);
            oid[j] = __shfl_xor(id[j], o, DF_WAVE);
        }
        merge(ov, oid);
    }
};

// Row reductions over a logits tile lg[R][C] held in LDS (vocabulary columns n0 .. n0+C-1, block rows
// row0 .. row0+R-1, of which `rows` are valid).  The TPR = 256 / R threads of a row are consecutive lanes of
// one wave; each takes C / TPR columns, and the row's max, sum of exponentials and top-8 list are combined
// by a butterfly over those lanes (xor shuffles: every lane ends with the same, order-independent result).
// The first thread of the row writes the record of (group, row).
template <int R, int C>
__device__ void head_epilogue(const float (*lg)[C + 1], int rows, int row0, int Mtot, int n0, int V, int group,
                              float* __restrict__ hpart, float* __restrict__ logits_dbg, RngKey key, int sample) {
    constexpr int TPR = 256 / R, CPT = C / TPR;
    static_assert(TPR <= DF_WAVE && (TPR & (TPR - 1)) == 0, "a row's threads must share a wave");
    const int t = threadIdx.x;
    const int m = t / TPR, piece = t % TPR, c0 = piece * CPT;
    const bool live = m < rows;
    const int ncol = live ? min(CPT, V - (n0 + c0)) : 0;  // valid columns of this thread (may be <= 0)
    float mx = -INFINITY;
    for (int c = 0; c < ncol; ++c) {
        const float x = lg[m][c0 + c];
        mx = fmaxf(mx, x);
        if (logits_dbg) logits_dbg[(size_t)(row0 + m) * V + n0 + c0 + c] = x;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, DF_WAVE));
    float se = 0.f;
    Top8 s;
    s.clear();
    for (int c = 0; c < ncol; ++c) {
        const float x = lg[m][c0 + c];
        se += expf(x - mx);
        s.insert(x, n0 + c0 + c);
    }
    // (kept rolled: one copy of the merge network keeps the compiler's work linear)
#pragma unroll 1
    for (int o = 1; o < TPR; o <<= 1) {
        se += __shfl_xor(se, o, DF_WAVE);
        s.merge_lane_xor(o);
    }
    // Temperature 1: the row's Gumbel-max candidate over these columns.  A thread's columns start at a
    // multiple of 4, so each generator block serves four consecutive logits.
    float bs = -INFINITY;
    int bi = 0x7FFFFFFF;
    if (sample) {
        for (int c = 0; c < ncol; c += 4) {
            const int j0 = n0 + c0 + c;
            uint32_t w[4];
            philox_block(key, (uint32_t)j0 >> 2, (uint32_t)(row0 + m), RNG_TAG_DRAFT, w);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c + e < ncol) {
                    const float sc = lg[m][c0 + c + e] + rng_gumbel(w[e]);
                    if (sc > bs) {  // columns ascend: a tie keeps the smaller id
                        bs = sc;
                        bi = j0 + e;
                    }
                }
        }
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) {
            const float os = __shfl_xor(bs, o, DF_WAVE);
            const int oi = __shfl_xor(bi, o, DF_WAVE);
            if (df_better(os, oi, bs, bi)) {
                bs = os;
                bi = oi;
            }
        }
    }
    if (live && piece == 0) {
        float* dst = hpart + ((size_t)group * Mtot + row0 + m) * HEAD_REC;
        dst[0] = mx;
        dst[1] = se;
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {
            dst[hr_val(j)] = s.v[j];
            dst[hr_id(j)] = __int_as_float(s.id[j]);
        }
        if (sample) {
            dst[HR_SSC] = bs;
            dst[HR_SID] = __int_as_float(bi);
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// bfloat16 MFMA LM head: the GEMM core of the skinny kernel with the reductions as epilogue
// ------------------------------------------------------------------------------------------------------
// W is the packed (chunk-major) V x K matrix; z is an activation pair of bfloat16 planes (lo plane at
// z + zplane): two MFMAs per weight fragment.  NW waves split K.  Four waves per workgroup keep two
// workgroups resident per CU, so one streams weights while the other runs its reduction epilogue (measured
// on MI355X: eight waves per workgroup, one workgroup per CU, is ~20% slower end to end).
template <int MT, int NW>
__global__ __launch_bounds__(64 * NW) void lm_head_bf16(const bf16_t* __restrict__ z, size_t zplane, int M,
                                                        const bf16_t* __restrict__ W, int V, int K,
                                                        float* __restrict__ hpart, float* __restrict__ logits_dbg,
                                                        RngKey key, int sample) {
    constexpr int NT = 4;
    __shared__ f32x4 red[NW][NT * MT][64];
    __shared__ float lg[16 * MT][65];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 64;
    const int chunks = K / 256;
    const int kb = (wave * chunks / NW) * 256, ke = ((wave + 1) * chunks / NW) * 256;

    // group blockIdx.x of the chunk-major packed matrix: one contiguous 32 KB block per k-chunk
    const size_t chunk_stride = packed_groups(V) * 32 * DF_FRAG;
    const bf16_t* wt = W + (size_t)blockIdx.x * 32 * DF_FRAG + lane * 8;
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
            for (int nt = 0; nt < NT; ++nt) wf[nt][j] = ld16_nt(wt + (size_t)(kc / 256) * chunk_stride + (nt * 8 + j) * DF_FRAG);
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
    for (int e = threadIdx.x; e < NT * MT * 64; e += 64 * NW) {
        const int t = e >> 6, l = e & 63;
        const int nt = t / MT, mt = t % MT;
        f32x4 v = red[0][t][l];
#pragma unroll
        for (int q = 1; q < NW; ++q) {
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
    if (threadIdx.x < 256)
        head_epilogue<16 * MT, 64>(lg, M, 0, M, n0, V, blockIdx.x, hpart, logits_dbg, key, sample);
}

// ------------------------------------------------------------------------------------------------------
// float32 LM head (float32 drafters, M <= 32)
// ------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lm_head_f32(const float* __restrict__ z, int M, const float* __restrict__ W,
                                                   int V, int K, float* __restrict__ hpart,
                                                   float* __restrict__ logits_dbg, RngKey key, int sample) {
    __shared__ float lg[32][65];
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
    head_epilogue<32, 64>(lg, M, 0, M, n0, V, blockIdx.x, hpart, logits_dbg, key, sample);
}

// ------------------------------------------------------------------------------------------------------
// LDS-tiled MFMA LM head for many block rows (serving batches): tile 128 vocabulary x 128 rows
// ------------------------------------------------------------------------------------------------------
// The tiled GEMM main loop leaves each wave a 64 x 64 block of logits in registers; the tile is parked in
// LDS (over the staging buffers, which are free after the loop) and the row reductions run on it.
#define TH_LG_BYTES (128 * 129 * 4)
__global__ __launch_bounds__(256) void lm_head_tiled_bf16(const bf16_t* __restrict__ z, size_t zplane, int M,
                                                          const bf16_t* __restrict__ W, int V, int K,
                                                          float* __restrict__ hpart, float* __restrict__ logits_dbg,
                                                          RngKey key, int sample) {
    static_assert(TH_LG_BYTES >= (TL_SW + 2 * TL_BM * TL_LD) * 2, "logits tile must cover the staging buffers");
    __shared__ __attribute__((aligned(16))) char smem[TH_LG_BYTES];
    bf16_t* sw = (bf16_t*)smem;
    bf16_t* sx = sw + TL_SW;
    float(*lg)[129] = (float(*)[129])smem;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave >> 1, wm = wave & 1;
    int tx, ty;
    if (!xcd_tile(blockIdx.x, (V + TL_BN - 1) / TL_BN, (M + TL_BM - 1) / TL_BM, tx, ty)) return;
    const int n0 = tx * TL_BN, m0 = ty * TL_BM;
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
    head_epilogue<128, 128>(lg, min(128, M - m0), m0, M, n0, V, tx, hpart, logits_dbg, key, sample);
}

hipError_t launch_lm_head(int bf16, const void* z, int M, const void* wlm, int V, int K, float* hpart,
                          float* logits_dbg, int sample, uint64_t seed, hipStream_t st) {
    const dim3 grid(head_groups(V, head_group_width(bf16, M)));
    const RngKey key{(uint32_t)seed, (uint32_t)(seed >> 32)};
    const size_t zplane = (size_t)M * K;
    if (bf16 && M > 32)
        DF_LAUNCH(lm_head_tiled_bf16, dim3(xcd_tile_count(grid.x, (M + TL_BM - 1) / TL_BM)), dim3(256), 0, st,
                           (const bf16_t*)z, zplane, M, (const bf16_t*)wlm, V, K, hpart, logits_dbg, key, sample);
    else if (!bf16)
        hipLaunchKernelGGL(lm_head_f32, grid, dim3(256), 0, st, (const float*)z, M, (const float*)wlm, V, K, hpart,
                           logits_dbg, key, sample);
    else if (M <= 16)
        DF_LAUNCH((lm_head_bf16<1, 4>), grid, dim3(256), 0, st, (const bf16_t*)z, zplane, M,
                           (const bf16_t*)wlm, V, K, hpart, logits_dbg, key, sample);
    else
        DF_LAUNCH((lm_head_bf16<2, 4>), grid, dim3(256), 0, st, (const bf16_t*)z, zplane, M,
                           (const bf16_t*)wlm, V, K, hpart, logits_dbg, key, sample);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// stage 2: merge the per-group records of one block row
// ------------------------------------------------------------------------------------------------------
// One workgroup per block row.  The log-sum-exp needs only the records' (max, sumexp).  For the top-8, a
// lower bound T of the row's 8th best logit: (a) the largest 8th entry of any record (that record alone has
// 8 entries >= it), and (b) the 8th largest of the 16 waves' maxima over their records' maxima (8 distinct
// records reach it).  Every entry of the row's top 8 is then among the record entries >= T -- about a dozen
// for continuous logits -- which are gathered in LDS and placed by rank (number of better candidates; ranks
// are unique because ids are).  If ties push the candidate count past the buffer, a tree of bitonic merges
// over all records takes over.  The result does not depend on the gathering order: deterministic.
#define MERGE_THREADS 1024
#define MERGE_CAP 1024
__global__ __launch_bounds__(MERGE_THREADS) void head_merge(int M, int V, int n_groups, int top_k, int sample,
                                                            const float* __restrict__ hpart,
                                                            const int32_t* __restrict__ btok,
                                                            int32_t* __restrict__ tokens, int32_t* __restrict__ topk_ids,
                                                            float* __restrict__ topk_lp, uint32_t* err) {
    __shared__ float cv[MERGE_CAP];
    __shared__ int cid[MERGE_CAP];
    __shared__ float red[MERGE_THREADS / 64];
    __shared__ float rmx[MERGE_THREADS / 64], rth[MERGE_THREADS / 64];
    __shared__ float outv[DF_TOPK];
    __shared__ int outi[DF_TOPK];
    __shared__ float sbest[MERGE_THREADS / 64];
    __shared__ int sbid[MERGE_THREADS / 64];
    __shared__ int cnt;
    const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
    if (t == 0) {
        cnt = 0;
        if (btok[m] < 0 || btok[m] >= V) set_err(err, DFLASH_DEVERR_TOKEN);
    }
    const size_t RS = (size_t)M * HEAD_REC;               // record stride between groups
    const float* row = hpart + (size_t)m * HEAD_REC;      // field f of group gi at row[gi * RS + f]
    float mx = -INFINITY, th = -INFINITY;
    float sb = -INFINITY;  // temperature 1: best (perturbed score, id) over the records
    int sbi = 0x7FFFFFFF;
    // A record is five 16-byte words (80 bytes, 16-byte aligned); word 0 holds (max, sumexp, 8th value, sampled
    // score) and word 2 ends with the sampled id.  The first MERGE_GROUPS of a thread's groups are fetched with
    // their loads in flight together (one word each, two at temperature 1), and their (max, sumexp) kept for the
    // second pass.
    constexpr int MERGE_GROUPS = 4;
    // (every load is issued, a thread past the last group reading group 0, so that all are in flight before the
    // first is used)
    float4 w0[MERGE_GROUPS];
    int sid[MERGE_GROUPS];
#pragma unroll
    for (int u = 0; u < MERGE_GROUPS; ++u) {
        const int gi = t + u * MERGE_THREADS;
        w0[u] = *(const float4*)(row + (size_t)(gi < n_groups ? gi : 0) * RS);
    }
    if (sample) {
#pragma unroll
        for (int u = 0; u < MERGE_GROUPS; ++u) {
            const int gi = t + u * MERGE_THREADS;
            sid[u] = __float_as_int(row[(size_t)(gi < n_groups ? gi : 0) * RS + HR_SID]);
        }
    }
#pragma unroll
    for (int u = 0; u < MERGE_GROUPS; ++u) {
        const bool ok = t + u * MERGE_THREADS < n_groups;
        if (!ok) w0[u] = make_float4(-INFINITY, 0.f, -INFINITY, -INFINITY);
        mx = fmaxf(mx, w0[u].x);
        th = fmaxf(th, w0[u].z);  // the record's 8th value
        if (sample && ok && df_better(w0[u].w, sid[u], sb, sbi)) {
            sb = w0[u].w;
            sbi = sid[u];
        }
    }
    for (int gi = t + MERGE_GROUPS * MERGE_THREADS; gi < n_groups; gi += MERGE_THREADS) {  // very large vocabularies
        mx = fmaxf(mx, row[gi * RS]);
        th = fmaxf(th, row[gi * RS + hr_val(DF_TOPK - 1)]);
        if (sample) {
            const float v = row[gi * RS + HR_SSC];
            const int id = __float_as_int(row[gi * RS + HR_SID]);
            if (df_better(v, id, sb, sbi)) {
                sb = v;
                sbi = id;
            }
        }
    }
    if (sample) {  // (score, id) is a total order: the winner does not depend on the reduction order
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(sb, o, DF_WAVE);
            const int oi = __shfl_xor(sbi, o, DF_WAVE);
            if (df_better(ov, oi, sb, sbi)) {
                sb = ov;
                sbi = oi;
            }
        }
        if ((t & 63) == 0) {  // read by thread 0 after the barriers below
            sbest[t >> 6] = sb;
            sbid[t >> 6] = sbi;
        }
    }
    // One block reduction (one barrier) for the maximum and bound (a); every wave then finds bound (b), the
    // 8th largest wave maximum (ties by wave index), on its first sixteen lanes.
    constexpr int NW = MERGE_THREADS / 64;
    float wm = mx, wt = th;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        wm = fmaxf(wm, __shfl_xor(wm, o, DF_WAVE));
        wt = fmaxf(wt, __shfl_xor(wt, o, DF_WAVE));
    }
    if (lane == 0) {
        rmx[wv] = wm;
        rth[wv] = wt;
    }
    __syncthreads();
    mx = rmx[0];
    float ta = rth[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        mx = fmaxf(mx, rmx[i]);
        ta = fmaxf(ta, rth[i]);
    }
    float t8 = -INFINITY;
    if (lane < NW) {
        const float x = rmx[lane];
        int rank = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) rank += (rmx[j] > x || (rmx[j] == x && j < lane)) ? 1 : 0;
        if (rank == DF_TOPK - 1) t8 = x;
    }
    th = fmaxf(ta, wave_max(t8));
    float se = 0.f;
    for (int gi = t; gi < n_groups; gi += MERGE_THREADS) {
        const int u = (gi - t) / MERGE_THREADS;
        float r0, r1;
        if (u < MERGE_GROUPS) {  // cached from the first pass (u is uniform per iteration)
            float4 c = w0[0];
#pragma unroll
            for (int q = 1; q < MERGE_GROUPS; ++q) c = u == q ? w0[q] : c;
            r0 = c.x;
            r1 = c.y;
        } else {
            r0 = row[gi * RS];
            r1 = row[gi * RS + 1];
        }
        if (r0 != -INFINITY) se += r1 * expf(r0 - mx);
        if (r0 >= th) {  // the record's best entry reaches the threshold: scan its list
            for (int j = 0; j < DF_TOPK; ++j) {
                const float v = row[gi * RS + hr_val(j)];
                const int id = __float_as_int(row[gi * RS + hr_id(j)]);
                if (v < th) break;
                if (id < V) {
                    const int k = atomicAdd(&cnt, 1);
                    if (k < MERGE_CAP) {
                        cv[k] = v;
                        cid[k] = id;
                    }
                }
            }
        }
    }
    se = block_sum(se, red);  // ends with a barrier: cnt and the candidates are complete
    const int n = cnt;
    if (n <= MERGE_CAP) {
        for (int i = t; i < n; i += MERGE_THREADS) {
            const float vi = cv[i];
            const int ii = cid[i];
            int rank = 0;
            for (int k = 0; k < n; ++k) rank += df_better(cv[k], cid[k], vi, ii) ? 1 : 0;
            if (rank < DF_TOPK) {
                outv[rank] = vi;
                outi[rank] = ii;
            }
        }
    } else {
        // fallback: bitonic-merge tree over all records (cv / cid reused as list storage)
        Top8 s;
        s.clear();
#pragma unroll 1
        for (int gi = t; gi < n_groups; gi += MERGE_THREADS) {
            float ov[DF_TOPK];
            int oid[DF_TOPK];
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) {
                ov[j] = row[gi * RS + hr_val(j)];
                oid[j] = __float_as_int(row[gi * RS + hr_id(j)]);
            }
            s.merge(ov, oid);
        }
#pragma unroll 1
        for (int o = 1; o < DF_WAVE; o <<= 1) s.merge_lane_xor(o);
        __syncthreads();
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) {
                cv[wv * DF_TOPK + j] = s.v[j];
                cid[wv * DF_TOPK + j] = s.id[j];
            }
        }
        __syncthreads();
        if (t == 0) {
#pragma unroll 1
            for (int q = 1; q < MERGE_THREADS / 64; ++q) {
                float ov[DF_TOPK];
                int oid[DF_TOPK];
#pragma unroll
                for (int j = 0; j < DF_TOPK; ++j) {
                    ov[j] = cv[q * DF_TOPK + j];
                    oid[j] = cid[q * DF_TOPK + j];
                }
                s.merge(ov, oid);
            }
#pragma unroll
            for (int j = 0; j < DF_TOPK; ++j) {
                outv[j] = s.v[j];
                outi[j] = s.id[j];
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        const float lse = mx + logf(se);
        int tok = outi[0];
        if (sample) {
            float b = sbest[0];
            tok = sbid[0];
            for (int w = 1; w < MERGE_THREADS / 64; ++w)
                if (df_better(sbest[w], sbid[w], b, tok)) {
                    b = sbest[w];
                    tok = sbid[w];
                }
        }
        tokens[m] = tok;
#pragma unroll
        for (int j = 0; j < DF_TOPK; ++j) {  // static indices keep the state in registers
            if (j < top_k) {
                topk_ids[(size_t)m * top_k + j] = outi[j];
                topk_lp[(size_t)m * top_k + j] = outv[j] - lse;
            }
        }
    }
}

hipError_t launch_head_merge(int bf16, int M, int V, int top_k, int sample, const float* hpart,
                             const int32_t* block_tokens, int32_t* tokens, int32_t* topk_ids, float* topk_lp,
                             uint32_t* err, hipStream_t st) {
    const int groups = head_groups(V, head_group_width(bf16, M));
    hipLaunchKernelGGL(head_merge, dim3(M), dim3(MERGE_THREADS), 0, st, M, V, groups, top_k, sample, hpart,
                       block_tokens, tokens, topk_ids, topk_lp, err);
    return hipGetLastError();
}

}  // namespace df
