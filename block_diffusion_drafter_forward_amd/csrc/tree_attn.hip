// Tree attention for verifying a draft tree in one target-layer pass ("Accelerating Speculative Decoding with
// Block Diffusion Draft Trees", section 3.4.5 "Verification: Tree Attention and the Verifier Walk"): the
// flattened tree tokens (token 0 = the root / bonus token, every parent before its children) attend to the
// whole cached context and, inside the tree, only to their ancestors and themselves; a token's position id
// is its depth, i.e. absolute position ctx_len + depth.
//
// Three launches:
//   tree_prep       per 16 tokens and group of eight heads: depth and (first group) root-to-token ancestor
//                   list from the parent links (walked in LDS), and RoPE of the group's q / k rows at
//                   ctx_len + depth (cos / sin per depth from an LDS table), rounded to bfloat16
//   tree_ctx_bf16   the context part, MFMA: one workgroup per (16-token tile, KV head, context chunk,
//                   request), one wave per query head of the KV group; 64-key rounds staged in LDS as in the
//                   drafter's attention.  The KV head is the fastest grid index, so with 8 KV heads (or a
//                   multiple) workgroup i lands on XCD i % 8 = KV head: each XCD's L2 holds one head's K/V
//                   for every tile.  Writes (m, l, O) partials.
//   tree_merge      one wave per (token, KV head): the token's ancestor keys (at most depth + 1, a short list)
//                   by vector dot products, merged with the context partials by log-sum-exp; bfloat16 out.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace df {

#define TA_D 128
#define TA_SUB 64         // keys per LDS round
#define TA_MAX_PAGES 256  // pages of one context chunk
#define TA_KLD (128 + 16)
// Values in LDS: one row per (32-key slice hk, d) holding the slice's two pages interleaved by groups of four
// slots, [g][page 2 hk + pp][4 slots] (g = slot / 4), so that a lane's V^T operand (slots 4g..4g+3 of both
// pages) is one aligned 16-byte read; rows padded to 80 bytes.
#define TA_SVLD (32 + 8)
#define TA_RESCALE 8.0f  // log2 growth of a row maximum before the running reference is raised
#define TP_HEADS 8        // heads whose rows one tree_prep workgroup rotates (16 tokens x 8 heads: one round trip)
#define TM_BATCH 8        // context chunks (and ancestor keys) whose loads tree_merge keeps in flight together

static size_t ta_align(size_t x) { return (x + 255) & ~(size_t)255; }

// x / d for 0 <= x < 2^31 and a divisor d fixed for the call, as a multiply-high and a shift (Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", PLDI 1994, Theorem 4.2 with N = 31):
// l = ceil(log2 d), m = floor(2^(31 + l) / d) + 1 < 2^32.  The kernels' segment and slot indices use it in
// place of a run-time division (a long reciprocal-and-correct sequence) ahead of their first loads.
struct FastDiv {
    uint32_t m, s;
};
static FastDiv fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    return FastDiv{(uint32_t)((1ull << (31 + l)) / d + 1), 31 + l};
}
__device__ __forceinline__ int fdiv(int x, FastDiv f) { return (int)(((uint64_t)(uint32_t)x * f.m) >> f.s); }

// Waves per context workgroup: the G query heads of a KV head times TA_WAVES / G wave slots, each slot
// TA_QT token tiles, all served by the same staged K/V.  Two tiles per wave make every K (V) fragment read
// from LDS feed two MFMAs (with one tile per wave, LDS reads bounded the kernel).
#define TA_WAVES 8
#define TA_QT 2

TreePlan plan_tree(int batch, int max_tokens, int nq, int nkv, int max_ctx) {
    TreePlan p{};
    p.tiles = (max_tokens + 15) / 16;
    const int tw = TA_WAVES / (nq / nkv) * TA_QT;  // tiles per workgroup
    p.stiles = (p.tiles + tw - 1) / tw;
    p.rpu = p.rpw = p.wgs = p.slots = 0;
    if (max_ctx > 0) {
        // One eight-wave workgroup per CU (the kernel's registers allow no second), so a grid runs in
        // generations of 256 workgroups.  Pick the rounds per workgroup (and the mode) that minimise the
        // estimated time (measured on MI355X): generations x (rounds + about one round of start-up per unit
        // segment) x 2.8 us, plus the float32 (m, l, O) partials written and read back by the merge at ~5 TB/s,
        // plus one merge round trip (~1.5 us) per TM_BATCH slots.  Two modes:
        //  - padded: each unit's sequence is padded to whole workgroups (the padding rounds are empty), so every
        //    workgroup serves one unit: equal chunks of each unit's context;
        //  - streamed: no padding, so that the workgroups share the rounds evenly, at the price of a second
        //    start-up where a workgroup's rounds run into the next unit.  Equal chunks leave the last generation
        //    part-empty when the unit count does not divide into 256s (at 1025 tree tokens of one request: 136
        //    units).
        const int units = batch * p.stiles;  // per KV head
        const int rounds = (max_ctx + TA_SUB - 1) / TA_SUB;
        const double part_us = (double)batch * p.tiles * nq * 16 * (TA_D + 2) * 4 * 2 / 5.0e6;  // per slot
        const int max_rpw = std::min(TA_MAX_PAGES / 4, rounds);  // a segment's page ids fit in LDS
        double best = 1e30;
        for (int rpw = 1; rpw <= max_rpw; ++rpw) {
            for (int streamed = 0; streamed < 2; ++streamed) {
                const int chunks = (rounds + rpw - 1) / rpw;
                const int seq = streamed ? rounds : chunks * rpw;  // the unit's rounds in the sequence
                if (streamed && seq % rpw == 0) continue;          // same as padded
                const long wgs = ((long)units * seq + rpw - 1) / rpw;
                const long gens = (wgs * nkv + 255) / 256;
                const int segs = streamed ? (rpw + seq - 1) / seq + 1 : 1;
                const int slots = streamed ? (seq - 1) / rpw + 2 : chunks;
                const double per_unit = streamed ? (double)seq / rpw + 1.0 : chunks;
                const double cost = 2.8 * (double)gens * (rpw + 1.2 * segs) + per_unit * part_us +
                                    1.5 * ((slots + TM_BATCH - 1) / TM_BATCH);
                if (cost < best - 1e-9) {
                    best = cost;
                    p.rpu = seq;
                    p.rpw = rpw;
                    p.wgs = (int)wgs;
                }
            }
        }
        // slots: the most workgroups any unit's rounds [u rpu, (u + 1) rpu) meet (a function of u rpu mod rpw,
        // whose values repeat within rpw units)
        for (int u = 0; u < std::min(units, p.rpw); ++u) {
            const long f = (long)u * p.rpu / p.rpw, l = ((long)u * p.rpu + p.rpu - 1) / p.rpw;
            p.slots = std::max(p.slots, (int)(l - f + 1));
        }
    }
    const size_t T = (size_t)p.tiles * 16;
    size_t off = 256;  // error word
    p.q_off = off;
    off += ta_align((size_t)batch * T * nq * TA_D * 2);
    p.k_off = off;
    off += ta_align((size_t)batch * T * nkv * TA_D * 2);
    p.anc_off = off;
    off += ta_align((size_t)batch * T * TREE_MAX_ANC * 4);
    p.o_off = off;
    off += ta_align((size_t)batch * p.tiles * nq * p.slots * 16 * TA_D * 4);
    p.ml_off = off;
    off += ta_align((size_t)batch * p.tiles * nq * p.slots * 16 * 2 * 4);
    p.total = off;
    return p;
}

// ------------------------------------------------------------------------------------------------------
// tree_prep
// ------------------------------------------------------------------------------------------------------
// anc[b][i][0] = depth d of token i, anc[b][i][1 + j] = its ancestor at depth j (j = 0: the root, j = d:
// itself); a token past n_tokens has anc[..][0] = -1.  Parent links that are not < the token's own index
// are flagged and treated as the root.
__global__ __launch_bounds__(256) void tree_prep(int T, const int32_t* __restrict__ n_tokens,
                                                 const int32_t* __restrict__ parent, int nq, int nkv,
                                                 const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                 const int32_t* __restrict__ ctx_len, int max_ctx, RopeFreq rf,
                                                 bf16_t* __restrict__ qr, bf16_t* __restrict__ kr,
                                                 int32_t* __restrict__ anc, int Tpad, uint32_t* err) {
    __shared__ int spar[TREE_MAX_TOKENS];
    __shared__ int sdep[16];
    __shared__ int smaxdep;
    __shared__ float scs[TREE_MAX_ANC][TA_D / 2][2];
    const int b = blockIdx.y, tile = blockIdx.x, t = threadIdx.x;
    const int n = min(max(n_tokens[b], 0), T);
    int C = ctx_len[b];
    if (C < 0 || C > max_ctx) {
        if (tile == 0 && t == 0) set_err(err, DFLASH_DEVERR_POS);
        C = C < 0 ? 0 : max_ctx;
    }
    const int i0 = tile * 16;
    const int need = min(n, i0 + 16);  // parents of tokens below this tile's end
    for (int j = t; j < need; j += 256) spar[j] = parent[(size_t)b * T + j];
    if (t == 0) smaxdep = 0;
    __syncthreads();
    if (t < 16) {
        const int i = i0 + t;
        int32_t* a = anc + ((size_t)b * Tpad + i) * TREE_MAX_ANC;
        int depth = -1;
        if (i < n) {
            // first walk: the depth (a link that does not point to an earlier token, or a path deeper than
            // TREE_MAX_ANC - 2, is flagged and cut at the root)
            int cur = i, len = 0;
            bool bad = false;
            while (cur != 0) {
                int p = spar[cur];
                if (p < 0 || p >= cur || (len == TREE_MAX_ANC - 3 && p != 0)) {  // depth stays <= TREE_MAX_ANC - 2
                    bad = true;
                    p = 0;
                }
                ++len;
                cur = p;
            }
            if (bad) set_err(err, DFLASH_DEVERR_TREE);
            depth = len;
            // second walk (head group 0 only): the path from the token up, stored root first
            if (blockIdx.z == 0) {
                a[1] = 0;
                cur = i;
                for (int j = len; j >= 1; --j) {
                    a[1 + j] = cur;
                    int p = spar[cur];
                    cur = (p < 0 || p >= cur) ? 0 : p;
                }
            }
            atomicMax(&smaxdep, depth);
        }
        if (blockIdx.z == 0) a[0] = depth;
        sdep[t] = depth;
    }
    __syncthreads();
    // cos / sin of the angles float32(float32(C + depth) * inv_freq) of the depths present in the tile
    const int nd = smaxdep + 1;
    for (int e = t; e < nd * (TA_D / 2); e += 256) {
        const int dep = e >> 6, pr = e & 63;
        float s = 0.f, c = 1.f;  // rotary embedding off: identity
        if (rf.on) sincosf((float)(C + dep) * rf.inv[pr], &s, &c);
        scs[dep][pr][0] = c;
        scs[dep][pr][1] = s;
    }
    __syncthreads();
    // RoPE of the tile's rows for this workgroup's group of TP_HEADS heads (16 tokens x up to TP_HEADS heads):
    // eight lanes per row, lane j rotating the pairs (8j + e, 64 + 8j + e), e < 8, from two 16-byte loads;
    // four rows in flight per lane, i.e. every row of the group in one round trip
    const int hh = nq + nkv, h0 = blockIdx.z * TP_HEADS, nh = min(TP_HEADS, hh - h0), rows = 16 * nh;
    const int sub = t & 7, slot = t >> 3;  // 32 row slots per pass
    for (int r0 = 0; r0 < rows; r0 += 32 * 4) {
        u32x4 x1[4], x2[4];
        int rr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = r0 + u * 32 + slot;
            rr[u] = row;
            const int tok = row / nh, h = h0 + row - tok * nh;
            const bool ok = row < rows && sdep[min(tok, 15)] >= 0;
            const bool isq = h < nq;
            const bf16_t* src = isq ? q + (((size_t)b * T + i0 + tok) * nq + h) * TA_D
                                    : k + (((size_t)b * T + i0 + tok) * nkv + (h - nq)) * TA_D;
            x1[u] = ok ? ld16(src + 8 * sub) : u32x4{0u, 0u, 0u, 0u};
            x2[u] = ok ? ld16(src + 64 + 8 * sub) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = rr[u];
            if (row >= rows) break;
            const int tok = row / nh, h = h0 + row - tok * nh;
            const int dep = sdep[tok];
            const bool isq = h < nq;
            bf16_t* dst = isq ? qr + (((size_t)b * Tpad + i0 + tok) * nq + h) * TA_D
                              : kr + (((size_t)b * Tpad + i0 + tok) * nkv + (h - nq)) * TA_D;
            u32x4 y1, y2;
            if (dep < 0) {  // outside the tree: zeros, so that the context kernel's rows stay finite
                y1 = u32x4{0u, 0u, 0u, 0u};
                y2 = y1;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float o1[2], o2[2];
#pragma unroll
                    for (int hw = 0; hw < 2; ++hw) {
                        const int pr = 8 * sub + 2 * j + hw;
                        const float a1 = __uint_as_float(hw ? (x1[u][j] & 0xFFFF0000u) : (x1[u][j] << 16));
                        const float a2 = __uint_as_float(hw ? (x2[u][j] & 0xFFFF0000u) : (x2[u][j] << 16));
                        const float c = scs[dep][pr][0], s = scs[dep][pr][1];
                        o1[hw] = a1 * c - a2 * s;
                        o2[hw] = a2 * c + a1 * s;
                    }
                    y1[j] = f2bf2(o1[0], o1[1]);
                    y2[j] = f2bf2(o2[0], o2[1]);
                }
            }
            *(u32x4*)(dst + 8 * sub) = y1;
            *(u32x4*)(dst + 64 + 8 * sub) = y2;
        }
    }
}

// ------------------------------------------------------------------------------------------------------
// tree_ctx_bf16: the context part (MFMA)
// ------------------------------------------------------------------------------------------------------
// Wave w serves query head kv_head * G + w % G for the TA_QT token tiles (super_tile * TW + w / G) * TA_QT + i.
template <int G>
__global__ __launch_bounds__(64 * TA_WAVES) void tree_ctx_bf16(const bf16_t* __restrict__ qr, int Tpad, int tiles, int nq,
                                                        int nkv, const bf16_t* __restrict__ kpool,
                                                        const bf16_t* __restrict__ vpool, int n_pages,
                                                        const int32_t* __restrict__ pt, int max_pages,
                                                        const int32_t* __restrict__ ctx_len, int max_ctx,
                                                        int units, int rpu, int rpw, FastDiv div_rpu,
                                                        FastDiv div_rpw, FastDiv div_stiles, int n_slots,
                                                        float* __restrict__ opart, float* __restrict__ mlpart,
                                                        uint32_t* err) {
    constexpr int D = TA_D;
    constexpr int TW = TA_WAVES / G;
    constexpr int QT = TA_QT;
    constexpr int NT = 64 * TA_WAVES;
    constexpr int NPG = TA_SUB / 16;
    constexpr int PIECES = NPG * 512;
    constexpr int PPT = PIECES / NT;
    constexpr int PPP = 512 / NT;
    __shared__ __attribute__((aligned(16))) bf16_t sk[TA_SUB * TA_KLD];
    __shared__ __attribute__((aligned(16))) bf16_t sv[(NPG / 2) * D * TA_SVLD];
    __shared__ int spg[TA_MAX_PAGES];
    // grid: KV head fastest (one head per XCD's L2 when there are eight), then the head's workgroups in order;
    // workgroup wl of a head takes rounds [wl rpw, (wl + 1) rpw) of the sequence unit u = request * stiles +
    // super tile, rounds 0 .. rpu - 1 of each
    const int stiles = (tiles + TW * QT - 1) / (TW * QT);
    const int kvh = blockIdx.x % nkv;
    const int wl = blockIdx.x / nkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int h = kvh * G + w % G;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const size_t page_elems = (size_t)16 * D;
    // (units * rpu < 2^31: the API bounds batch x tiles x rounds)
    const int gend = min(units * rpu, wl * rpw + rpw);
    for (int gpos = wl * rpw; gpos < gend;) {  // one unit segment per pass
        const int u = fdiv(gpos, div_rpu);
        const int r0 = gpos - u * rpu;
        const int r1 = min(rpu, r0 + (gend - gpos));
        const int slot = wl - fdiv(u * rpu, div_rpw);  // < n_slots
        const bool first = gpos == wl * rpw;
        gpos += r1 - r0;
        const int b = fdiv(u, div_stiles), stile = u - b * stiles;
        // this wave's first tile; the last super tile may reach past the tree
        const int tile0 = (stile * TW + w / G) * QT;

        if (!first) __syncthreads();  // the previous segment's waves are past their page-id reads
        const int pg0 = r0 * (TA_SUB / 16), npg = (r1 - r0) * (TA_SUB / 16);  // npg <= TA_MAX_PAGES (rpw <= 64)
        for (int j = tid; j < npg; j += NT) spg[j] = pg0 + j < max_pages ? pt[(size_t)b * max_pages + pg0 + j] : -1;
        int ctx = ctx_len[b];
        if (ctx > max_ctx || ctx < 0) ctx = ctx < 0 ? 0 : max_ctx;  // flagged by tree_prep
        const int t0 = r0 * TA_SUB;
        const int t1 = min(ctx, r1 * TA_SUB);

        u32x4 pf[PPT];
        uint32_t okmask = 0;
        auto prefetch = [&](int ts) {
            okmask = 0;
#pragma unroll
            for (int e = 0; e < NPG; ++e) {
                const int tp = ts + 16 * e;
                const int page = tp < t1 ? spg[(tp - t0) >> 4] : -1;
                const bool ok = page >= 0 && page < n_pages;
                const size_t ofs = ((size_t)(ok ? page : 0) * nkv + kvh) * page_elems;
                okmask |= (ok ? 1u : 0u) << e;
#pragma unroll
                for (int u = 0; u < PPP; ++u) {
                    const int qq = tid + u * NT;
                    pf[e * PPP + u] = ld16((qq < 256 ? kpool : vpool) + ofs + (qq & 255) * 8);
                }
            }
        };
        // piece qq of page slot e into LDS: K row-major, V^T (piece q2 = slots 8 h .. 8 h + 7 of row d, groups 2 h
        // and 2 h + 1) into the interleaved value rows
        auto put = [&](int e, int qq, u32x4 v) {
            if (qq < 256) {
                *(u32x4*)(sk + (e * 16 + (qq >> 4)) * TA_KLD + (qq & 15) * 8) = v;
            } else {
                const int q2 = qq - 256, half = q2 & 1;
                bf16_t* row = sv + ((e >> 1) * D + (q2 >> 1)) * TA_SVLD + (e & 1) * 4;
                *(u32x2*)(row + (2 * half) * 8) = u32x2{v[0], v[1]};
                *(u32x2*)(row + (2 * half + 1) * 8) = u32x2{v[2], v[3]};
            }
        };
        auto stash = [&](int ts) {
            okmask = __builtin_amdgcn_readfirstlane(okmask);
            if (okmask == (1u << NPG) - 1 && ts + TA_SUB <= t1) {  // every page mapped and full (scalar branch)
#pragma unroll
                for (int e = 0; e < NPG; ++e)
#pragma unroll
                    for (int u = 0; u < PPP; ++u) put(e, tid + u * NT, pf[e * PPP + u]);
                return;
            }
#pragma unroll
            for (int e = 0; e < NPG; ++e) {
                const bool ok = (okmask >> e) & 1u;
                const int nvalid = t1 - (ts + 16 * e);
#pragma unroll
                for (int u = 0; u < PPP; ++u) {
                    const int qq = tid + u * NT;
                    u32x4 v = pf[e * PPP + u];
                    if (!ok) v = u32x4{0u, 0u, 0u, 0u};
                    if (qq >= 256 && nvalid < 16) {  // values of slots past the last key may hold anything: zero them
                        const int half = (qq - 256) & 1;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int s0 = half * 8 + 2 * j;
                            const uint32_t m = (s0 < nvalid ? 0x0000FFFFu : 0u) | (s0 + 1 < nvalid ? 0xFFFF0000u : 0u);
                            v[j] &= m;
                        }
                    }
                    put(e, qq, v);
                }
            }
        };

        // Q^T operands: lane supplies query row r of each tile (token tile * 16 + r), 8 d-values per k-step
        u32x4 qf[QT][4];
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
            const bool ok = tile0 + qi < tiles;
            const bf16_t* qp = qr + (((size_t)b * Tpad + (ok ? tile0 + qi : 0) * 16 + r) * nq + h) * D + g * 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) qf[qi][s] = ok ? ld16(qp + s * 32) : u32x4{0u, 0u, 0u, 0u};
        }
        // o[qi][0..7]: O^T for the eight 16-row d-tiles; o[qi][8]: the same product against an all-ones V^T,
        // i.e. the row sums l of the bfloat16 P that weighted O (every lane ends with its token's sum).
        f32x4 o[QT][9];
        float m_run[QT];
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
#pragma unroll
            for (int dt = 0; dt < 9; ++dt) o[qi][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run[qi] = -INFINITY;
        }
        const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bfloat16 1.0 x 8

        __syncthreads();  // page ids in LDS
        for (int j = tid; j < npg && t0 + 16 * j < t1; j += NT) {
            if ((t0 >> 4) + j >= max_pages) set_err(err, DFLASH_DEVERR_POS);
            else if (spg[j] < 0 || spg[j] >= n_pages) set_err(err, DFLASH_DEVERR_PAGE);
        }
        // One 64-key round starting at ts.  TAIL: the round runs past the chunk's last key (masked scores, slices
        // past the end skipped); the full rounds carry no masking code.
        //
        // Softmax in the log2 domain against a running reference m: p = 2^(s * scale - m).  The reference is raised
        // (and O, l rescaled by 2^(m_old - m_new)) only when some row's maximum exceeds it by more than
        // TA_RESCALE; otherwise p may reach 2^TA_RESCALE, which float32 sums and the bfloat16 P hold at the same
        // relative precision.  The (m, l, O) partials are exact for any reference, so the merge is unchanged.
        auto round = [&](int ts, auto tail_tag) {
            constexpr bool TAIL = decltype(tail_tag)::value;
            __syncthreads();
            stash(ts);
            __syncthreads();
            if (ts + TA_SUB < t1) prefetch(ts + TA_SUB);
            f32x4 sa[QT][NPG];
#pragma unroll
            for (int qi = 0; qi < QT; ++qi)
#pragma unroll
                for (int e = 0; e < NPG; ++e) sa[qi][e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < NPG; ++e) {
                    const u32x4 kf = ld16(sk + (e * 16 + r) * TA_KLD + g * 8 + s * 32);
#pragma unroll
                    for (int qi = 0; qi < QT; ++qi) sa[qi][e] = mfma16(kf, qf[qi][s], sa[qi][e]);
                }
            u32x4 pb[QT][NPG / 2];
#pragma unroll
            for (int qi = 0; qi < QT; ++qi) {
                if (TAIL) {
                    const int nk = t1 - ts;
#pragma unroll
                    for (int e = 0; e < NPG; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sa[qi][e][i] = 16 * e + 4 * g + i < nk ? sa[qi][e][i] : -INFINITY;
                }
                // row maximum of the raw scores (scale_log2 > 0 keeps the order)
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < NPG; ++e)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sa[qi][e][i]);
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mxs = mx * scale_log2;
                if (__any(mxs > m_run[qi] + TA_RESCALE)) {
                    const float m_new = fmaxf(m_run[qi], mxs);
                    const float alpha = __builtin_amdgcn_exp2f(m_run[qi] - (m_new == -INFINITY ? 0.f : m_new));
                    m_run[qi] = m_new;
#pragma unroll
                    for (int dt = 0; dt < 9; ++dt) {
                        o[qi][dt][0] *= alpha; o[qi][dt][1] *= alpha; o[qi][dt][2] *= alpha; o[qi][dt][3] *= alpha;
                    }
                }
                const float neg_m = m_run[qi] == -INFINITY ? 0.f : -m_run[qi];
                float p[NPG][4];
#pragma unroll
                for (int e = 0; e < NPG; ++e)
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[e][i] = __builtin_amdgcn_exp2f(fmaf(sa[qi][e][i], scale_log2, neg_m));
#pragma unroll
                for (int hk = 0; hk < NPG / 2; ++hk)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pb[qi][hk][j] = f2bf2(p[2 * hk + (j >> 1)][2 * (j & 1)], p[2 * hk + (j >> 1)][2 * (j & 1) + 1]);
            }
            // O^T += V^T P^T over 32-key slices, P as bfloat16; each V^T fragment feeds every tile, and the
            // all-ones operand accumulates the row sums from the same P
#pragma unroll
            for (int hk = 0; hk < NPG / 2; ++hk) {
                if (TAIL && ts + 32 * hk >= t1) break;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const u32x4 vf = ld16(sv + (hk * D + dt * 16 + r) * TA_SVLD + g * 8);
#pragma unroll
                    for (int qi = 0; qi < QT; ++qi) o[qi][dt] = mfma16(vf, pb[qi][hk], o[qi][dt]);
                }
#pragma unroll
                for (int qi = 0; qi < QT; ++qi) o[qi][8] = mfma16(ones, pb[qi][hk], o[qi][8]);
            }
        };
        if (t0 < t1) prefetch(t0);
        int ts = t0;
        for (; ts + TA_SUB <= t1; ts += TA_SUB) round(ts, std::false_type{});
        if (ts < t1) round(ts, std::true_type{});
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) {
            const int tile = tile0 + qi;
            if (tile >= tiles) continue;
            const size_t base = ((((size_t)b * tiles + tile) * nq + h) * n_slots + slot) * 16 + r;
            float* op = opart + base * D;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *(float4*)(op + dt * 16 + 4 * g) = make_float4(o[qi][dt][0], o[qi][dt][1], o[qi][dt][2], o[qi][dt][3]);
            if (g == 0) {
                mlpart[base * 2 + 0] = m_run[qi];
                mlpart[base * 2 + 1] = o[qi][8][0];
            }
        }
    }  // segment
}

// ------------------------------------------------------------------------------------------------------
// tree_merge: ancestors + context partials -> output
// ------------------------------------------------------------------------------------------------------
// Wave layout: lane = 16 * hs + dl: query head hs of the current group of four, eight d-values at 8 dl.
__global__ __launch_bounds__(256) void tree_merge(int T, int Tpad, int tiles, int nq, int nkv,
                                                  const int32_t* __restrict__ n_tokens,
                                                  const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr,
                                                  const bf16_t* __restrict__ v, const int32_t* __restrict__ anc,
                                                  const float* __restrict__ opart, const float* __restrict__ mlpart,
                                                  int rpu, FastDiv div_rpw, int tw_log2, int n_slots,
                                                  bf16_t* __restrict__ out) {
    const int b = blockIdx.y;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, KV head)
    const int lane = threadIdx.x & 63;
    const int i = item / nkv, kvh = item % nkv;
    if (i >= T || i >= n_tokens[b]) return;
    const int G = nq / nkv;
    const int hs = lane >> 4, dl = lane & 15;
    const int32_t* a = anc + ((size_t)b * Tpad + i) * TREE_MAX_ANC;
    // the depth and the ancestor list in one round trip (lane e: the e-th entry, read whatever the depth)
    const int depth = a[0];
    const int anc_e = a[1 + min(lane, TREE_MAX_ANC - 2)];
    if (depth < 0) return;
    const int my_anc = lane <= depth ? anc_e : 0;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)TA_D);
    const int tile = i >> 4, row = i & 15;
    // the context partials of this token's unit: one per workgroup its rounds met (none without a context)
    // (tiles per context workgroup: 2^tw_log2; u0 < 2^31, bounded by the API)
    const int u0 = (b * ((tiles + (1 << tw_log2) - 1) >> tw_log2) + (tile >> tw_log2)) * rpu;
    const int n_chunks =
        __builtin_amdgcn_readfirstlane(n_slots > 0 ? fdiv(u0 + rpu - 1, div_rpw) - fdiv(u0, div_rpw) + 1 : 0);
    for (int hg = 0; hg < G; hg += 4) {
        const int hq = hg + hs;
        const bool live = hq < G;
        const int h = kvh * G + (live ? hq : 0);
        // query
        float qv[8];
        {
            const u32x4 u = ld16(qr + (((size_t)b * Tpad + i) * nq + h) * TA_D + 8 * dl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qv[2 * j] = __uint_as_float(u[j] << 16);
                qv[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
            }
        }
        // context partials (chunk order), in the log2 domain
        float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.f;
        const size_t cbase = (((size_t)b * tiles + tile) * nq + h) * n_slots;
        for (int c0 = 0; c0 < n_chunks; c0 += TM_BATCH) {  // TM_BATCH chunks' loads in flight at a time
            float2 mlc[TM_BATCH];
            float4 oc0[TM_BATCH], oc1[TM_BATCH];
#pragma unroll
            for (int u = 0; u < TM_BATCH; ++u) {
                const size_t base = (cbase + min(c0 + u, n_chunks - 1)) * 16 + row;
                mlc[u] = *(const float2*)(mlpart + base * 2);
                oc0[u] = *(const float4*)(opart + base * TA_D + 8 * dl);
                oc1[u] = *(const float4*)(opart + base * TA_D + 8 * dl + 4);
            }
#pragma unroll
            for (int u = 0; u < TM_BATCH; ++u) {
                const float mc = mlc[u].x, lc = mlc[u].y;
                if (c0 + u >= n_chunks || mc == -INFINITY) continue;
                const float mn = fmaxf(m, mc);
                const float sa = __builtin_amdgcn_exp2f(m - mn), sb = __builtin_amdgcn_exp2f(mc - mn);
                l = l * sa + lc * sb;
                const float oc[8] = {oc0[u].x, oc0[u].y, oc0[u].z, oc0[u].w, oc1[u].x, oc1[u].y, oc1[u].z, oc1[u].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = acc[j] * sa + oc[j] * sb;
                m = mn;
            }
        }
        // the token's ancestors and itself, root first: lane e holds the e-th, TM_BATCH keys in flight at a time
        for (int e0 = 0; e0 <= depth; e0 += TM_BATCH) {
            u32x4 ku[TM_BATCH], vu[TM_BATCH];
#pragma unroll
            for (int u = 0; u < TM_BATCH; ++u) {
                const int tok = __shfl(my_anc, min(e0 + u, depth), 64);
                ku[u] = ld16(kr + (((size_t)b * Tpad + tok) * nkv + kvh) * TA_D + 8 * dl);
                vu[u] = ld16(v + (((size_t)b * T + tok) * nkv + kvh) * TA_D + 8 * dl);
            }
#pragma unroll
            for (int u = 0; u < TM_BATCH; ++u) {
                if (e0 + u > depth) break;  // uniform
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s += qv[2 * j] * __uint_as_float(ku[u][j] << 16);
                    s += qv[2 * j + 1] * __uint_as_float(ku[u][j] & 0xFFFF0000u);
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);  // within the head's 16 lanes
                s *= scale_log2;
                const float mn = fmaxf(m, s);
                const float sa = __builtin_amdgcn_exp2f(m - mn), sb = __builtin_amdgcn_exp2f(s - mn);
                l = l * sa + sb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] = acc[2 * j] * sa + sb * __uint_as_float(vu[u][j] << 16);
                    acc[2 * j + 1] = acc[2 * j + 1] * sa + sb * __uint_as_float(vu[u][j] & 0xFFFF0000u);
                }
                m = mn;
            }
        }
        if (live) {
            const float inv = 1.f / l;
            u32x4 ov;
#pragma unroll
            for (int j = 0; j < 4; ++j) ov[j] = f2bf2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
            *(u32x4*)(out + (((size_t)b * T + i) * nq + h) * TA_D + 8 * dl) = ov;
        }
    }
}

hipError_t launch_tree_attention(const TreePlan& p, int batch, int T, const int32_t* n_tokens, const int32_t* parent,
                                 int nq, int nkv, const void* q, const void* k, const void* v, const void* kpool,
                                 const void* vpool, int n_pages, const int32_t* pt, int max_pages,
                                 const int32_t* ctx_len, int max_ctx, const RopeFreq& rf, void* out, void* ws,
                                 hipStream_t st) {
    char* W = (char*)ws;
    uint32_t* err = (uint32_t*)W;
    bf16_t* qr = (bf16_t*)(W + p.q_off);
    bf16_t* kr = (bf16_t*)(W + p.k_off);
    int32_t* anc = (int32_t*)(W + p.anc_off);
    float* opart = (float*)(W + p.o_off);
    float* ml = (float*)(W + p.ml_off);
    const int Tpad = p.tiles * 16;
    hipError_t e = launch_clear_err(err, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tree_prep, dim3(p.tiles, batch, (nq + nkv + TP_HEADS - 1) / TP_HEADS), dim3(256), 0, st, T,
                       n_tokens, parent, nq, nkv,
                       (const bf16_t*)q, (const bf16_t*)k, ctx_len, max_ctx, rf, qr, kr, anc, Tpad, err);
    if (p.slots > 0) {
        const dim3 grid(nkv * p.wgs);
        const int G = nq / nkv;
#define TA_LAUNCH(GG)                                                                                          \
    hipLaunchKernelGGL((tree_ctx_bf16<GG>), grid, dim3(64 * TA_WAVES), 0, st, qr, Tpad, p.tiles, nq, nkv,        \
                       (const bf16_t*)kpool, (const bf16_t*)vpool, n_pages, pt, max_pages, ctx_len, max_ctx,    \
                       batch * p.stiles, p.rpu, p.rpw, fast_div(p.rpu), fast_div(p.rpw), fast_div(p.stiles),    \
                       p.slots, opart, ml, err)
        if (G == 1) TA_LAUNCH(1);
        else if (G == 2) TA_LAUNCH(2);
        else if (G == 4) TA_LAUNCH(4);
        else TA_LAUNCH(8);
#undef TA_LAUNCH
    }
    hipLaunchKernelGGL(tree_merge, dim3((T * nkv + 3) / 4, batch), dim3(256), 0, st, T, Tpad, p.tiles, nq, nkv,
                       n_tokens, qr, kr, (const bf16_t*)v, anc, opart, ml, p.rpu,
                       fast_div(p.slots > 0 ? p.rpw : 1), __builtin_ctz((unsigned)(TA_WAVES / (nq / nkv) * TA_QT)),
                       p.slots, (bf16_t*)out);
    return hipGetLastError();
}

}  // namespace df
