// Block attention over [injected context ; block] (non-causal), grouped-query, paged context.
//
// Work split: one workgroup per (request, KV head, chunk of the request's cached context); chunk 0 also
// takes the block's own 16 keys, straight from registers while its first context round is in flight.  Wave
// w of the workgroup serves query head kv_head * G + w (G = query heads per KV head), whose L block rows form
// one 16-row MFMA tile.  Per pair of 16-key pages the wave computes S^T = K Q^T (keys in rows, so a lane's
// four scores belong to one query row), updates an online softmax in the log2 domain, and accumulates
// O^T = V^T P^T.  Values are cached transposed inside each page ([d][slot]) and staged so that a lane's V^T
// operand is one 16-byte LDS read; the probabilities enter the MFMA as P = P_hi + P_lo (two bfloat16 terms),
// which keeps them float32-exact.  Each chunk writes (m, l, O) partials; attn_merge combines the chunks in a
// fixed order.
#include "common.h"
#include "kernels.h"

namespace df {

#define AT_MAX_PAGES 256  // pages of one context chunk (their ids are staged in LDS up front)

// Keys staged per LDS round (four pages).  Measured on MI355X at the Qwen3-8B decode shape: 64-key rounds
// with 128-key chunks beat 128-key rounds (fewer registers, two rounds to overlap load and compute).
static int attn_sub(int) { return 64; }

AttnPlan plan_attention(int batch, int n_q, int n_kv, int max_ctx, int n_layers) {
    const int sub = attn_sub(n_q / n_kv);
    AttnPlan p{0, sub, 0};
    if (max_ctx <= 0) return p;
    // The weights are streamed with non-temporal loads, so a pass's cached K/V that fit in the 256 MB Infinity
    // Cache stay there from one pass to the next and are read with ordinary loads; larger caches are streamed
    // non-temporally like the weights (measured on MI355X: LLaMA-3.1-8B shape at 32768 tokens, 671 MB of K/V
    // per pass, -8.5 us per pass; Qwen3-8B shape at 4096 tokens, 84 MB, +6.6 us if streamed).
    const double kv_bytes = (double)n_layers * batch * max_ctx * n_kv * 128 * 2 * 2;
    p.stream_kv = kv_bytes > 128.0 * (1 << 20) ? 1 : 0;
    // one workgroup per CU over (request, KV head, chunk): a CU that had to take a second workgroup would
    // finish last (measured: 264 workgroups for 256 CUs ended ~3 us after the median); chunks of whole
    // staging rounds and at most AT_MAX_PAGES pages
    const int units = batch * n_kv;
    int want = 256 / units;
    // Long contexts: two workgroups per CU, twice the loads in flight, each chunk still eight or more
    // rounds long (measured on MI355X at 32768 tokens, 8 KV heads: 64 chunks instead of 32, -30 us per
    // pass; at 4096 tokens one-round chunks are slower than two-round ones).
    if (want > 0 && (long)max_ctx >= (long)want * sub * 8) want = 512 / units;
    const int max_chunks = (max_ctx + sub - 1) / sub;
    if (want > max_chunks) want = max_chunks;
    if (want < 1) want = 1;
    int ct = (max_ctx + want - 1) / want;
    ct = (ct + sub - 1) / sub * sub;
    if (ct > 16 * AT_MAX_PAGES) ct = 16 * AT_MAX_PAGES;
    p.chunk_tokens = ct;
    p.n_chunks = (max_ctx + ct - 1) / ct;
    return p;
}


// ------------------------------------------------------------------------------------------------------
// bfloat16 MFMA kernel (head_dim 128)
// ------------------------------------------------------------------------------------------------------
// Sub-chunks of SUB keys (SUB / 16 pages) are staged in LDS by the whole
// workgroup, so the G query heads of a KV group read each K/V byte from HBM once.  The chunk's page ids and
// the context length are fetched together up front (neither load waits on the other), and while the waves
// compute on one sub-chunk the next one is already in flight into registers.  Slots past the chunk's last
// key and pages the table does not map are staged as zeros, so uninitialised cache memory can never reach
// the MFMAs.
// q and the block's own k / v are activation pairs (hi + lo bfloat16 planes); the cached K/V are plain
// bfloat16.  The block's keys are attended first (every pair of hi / lo terms), from operands each lane
// loads itself at the start, so they add no staging round: chunk 0 then takes as many rounds as the
// other chunks, and its block step overlaps the wait for its first context round.
#define AT_KPAD 8  // padding of an LDS key row (elements), so that 16 consecutive keys spread over the banks
// Values in LDS: one row per (32-key slice hk, d) holding the slice's two pages interleaved by groups of four
// slots, [g][page 2 hk + pp][4 slots] (g = slot / 4), so that the 16 bytes a lane needs for the V^T operand
// (slots 4g..4g+3 of both pages) are one aligned LDS read; rows padded to 80 bytes spread a wave's reads over
// the banks.
#define AT_SVLD (32 + 8)

template <int G, int SUB, bool NTKV, int D>
__global__ __launch_bounds__(64 * G, 2) void attn_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kb,
                                                    const bf16_t* __restrict__ vbt, const bf16_t* __restrict__ kpool,
                                                    const bf16_t* __restrict__ vpool, int layer, int n_pages,
                                                    const int32_t* __restrict__ pt, int max_pages,
                                                    const int32_t* __restrict__ ctx_len, int max_ctx,
                                                    int chunk_tokens, int L, int nq, int nkv,
                                                    float* __restrict__ opart, float* __restrict__ mlpart,
                                                    uint32_t* err) {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int NT = 64 * G;
    constexpr int NPG = SUB / 16;        // pages per sub-chunk
    constexpr int KS = D / 32;           // 32-wide k-steps of q . k
    constexpr int DT = D / 16;           // 16-row d-tiles of the output
    constexpr int KLD = D + AT_KPAD;     // LDS key row (elements)
    constexpr int PG_PIECES = 4 * D;     // 16-byte pieces per page: 2 D of K, then 2 D of V^T
    // pieces per page per thread; with more threads than pieces (eight heads per KV head at d = 64) the first
    // PG_PIECES threads move every page and the rest stage nothing
    constexpr int PPP = PG_PIECES >= NT ? PG_PIECES / NT : 1;
    constexpr int PPT = NPG * PPP;
    __shared__ __attribute__((aligned(16))) bf16_t sk[SUB * KLD];
    __shared__ __attribute__((aligned(16))) bf16_t sv[(NPG / 2) * D * AT_SVLD];
    __shared__ int spg[AT_MAX_PAGES];
    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int h = kvh * G + w;
    const int C1 = gridDim.x;  // partial slots per (request, head): one per workgroup of the head
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const size_t page_elems = (size_t)16 * D;

    const size_t qplane = (size_t)gridDim.z * L * nq * D;         // hi -> lo plane of q
    const size_t bplane = (size_t)gridDim.z * nkv * page_elems;  // hi -> lo plane of the block's k / v
    // The chunk's page ids are requested first and only they are waited for before the first K/V round is
    // issued; q and, in chunk 0, the block's own k / v (requested once the ids are in LDS) arrive meanwhile.
    constexpr int PGT = (AT_MAX_PAGES + NT - 1) / NT;  // page ids per thread
    const int npg = chunk_tokens / 16, pg0 = c * npg;
    int pgv[PGT];
#pragma unroll
    for (int u = 0; u < PGT; ++u) {
        const int j = tid + u * NT;
        // every load is issued (from a clamped index; without a page table, from ctx_len) so that the waits
        // below count exactly these loads
        pgv[u] = *(max_pages > 0 ? pt + (size_t)b * max_pages + min(pg0 + j, max_pages - 1) : ctx_len);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the page-id loads ahead of the q loads
    // Q^T operand: lane supplies query row r (zero beyond L), eight d-values per 32-wide k-step
    u32x4 qf[KS], ql[KS];
    {
        const bool ok = r < L;
        const bf16_t* qp = q + ((size_t)(b * L + (ok ? r : 0)) * nq + h) * D + g * 8;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = ld16(qp + s * 32);  // unconditional loads (row 0 for rows past L), zeroed below
            ql[s] = ld16(qp + qplane + s * 32);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                qf[s][w4] = ok ? qf[s][w4] : 0u;
                ql[s][w4] = ok ? ql[s][w4] : 0u;
            }
    }
#pragma unroll
    for (int u = 0; u < PGT; ++u) {
        const int j = tid + u * NT;
        // (stored for every j < AT_MAX_PAGES, -1 past the chunk: an unconditional use keeps the load where it is)
        if (NT * PGT <= AT_MAX_PAGES || j < AT_MAX_PAGES) spg[j] = j < npg && pg0 + j < max_pages ? pgv[u] : -1;
    }
    // chunk 0: the block's K operand (lane: key slot r, d = 32 s + 8 g ..) and V^T operand (lane: d = 16 dt + r,
    // slots 4 g .. 4 g + 3), hi and lo planes
    u32x4 bk[2][KS];
    u32x2 bv[2][DT];
    if (c == 0) {
        const bf16_t* kr = kb + (((size_t)b * nkv + kvh) * 16 + r) * D + g * 8;
        const bf16_t* vr = vbt + ((size_t)b * nkv + kvh) * page_elems + (size_t)r * 16 + 4 * g;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
#pragma unroll
            for (int s = 0; s < KS; ++s) bk[pl][s] = ld16(kr + pl * bplane + s * 32);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) bv[pl][dt] = *(const u32x2*)(vr + pl * bplane + (size_t)dt * 16 * 16);
        }
    }

    // context keys [t0, t1) of chunk c
    int t0 = 0, t1 = 0;
    {
        int ctx = ctx_len[b];
        if (ctx > max_ctx || ctx < 0) {
            if (c == 0 && tid == 0) set_err(err, DFLASH_DEVERR_POS);
            ctx = ctx < 0 ? 0 : max_ctx;
        }
        t0 = c * chunk_tokens;
        t1 = min(ctx, t0 + chunk_tokens);
    }
    const int R = t0 < t1 ? (t1 - t0 + SUB - 1) / SUB : 0;  // context rounds of this workgroup
    auto ts_of = [&](int rr) { return t0 + rr * SUB; };

    // Staging: a page is 4 D 16-byte pieces (2 D of K, then 2 D of V^T), and piece j of either half sits at
    // element 8 j of its page, so thread tid moves pieces tid, tid + NT, ... of every page of the sub-chunk:
    // the per-thread offsets are compile-time constants and only the page bases change per sub-chunk.
    u32x4 pf[PPT];
    uint32_t okm = 0u;
    // Page slot e of the sub-chunk starting at key ts: its K and V^T bases always name readable memory (an
    // unmapped or out-of-range slot, or a round past the chunk, reads the block's own k / v page, which every
    // call has) and bit e of okmask says whether the slot holds data.  Loads are issued unconditionally and
    // the unmapped slots zeroed at stash time, so no load has to wait for another.
    auto prefetch = [&](int rr) {
        const int ts = ts_of(rr);
        uint32_t okmask = 0;
#pragma unroll
        for (int e = 0; e < NPG; ++e) {
            const int tp = ts + 16 * e;
            const int page = tp < t1 ? spg[(tp - t0) >> 4] : -1;
            const bool ok = page >= 0 && page < n_pages;
            const size_t ofs = (((size_t)layer * n_pages + (ok ? page : 0)) * nkv + kvh) * page_elems;
            okmask |= (ok ? 1u : 0u) << e;
            const bf16_t* kbase = ok ? kpool + ofs : kb;
            const bf16_t* vbase = ok ? vpool + ofs : vbt;
#pragma unroll
            for (int u = 0; u < PPP; ++u) {
                const int qq = tid + u * NT;
                if (PG_PIECES < NT && qq >= PG_PIECES) continue;  // (eight heads at d = 64: an idle thread)
                const bf16_t* src = (qq < 2 * D ? kbase : vbase) + (qq & (2 * D - 1)) * 8;
                pf[e * PPP + u] = NTKV ? ld16_nt(src) : ld16(src);
            }
        }
        okm = okmask;
    };
    auto stash = [&](int rr) {
        const int ts = ts_of(rr);
        const uint32_t okmask = __builtin_amdgcn_readfirstlane(okm);  // the same in every lane: scalar branches
#pragma unroll
        for (int e = 0; e < NPG; ++e) {
            const bool ok = (okmask >> e) & 1u;
            const int nvalid = t1 - (ts + 16 * e);
#pragma unroll
            for (int u = 0; u < PPP; ++u) {
                const int qq = tid + u * NT;
                if (PG_PIECES < NT && qq >= PG_PIECES) continue;
                u32x4 v = pf[e * PPP + u];
                if (!ok) v = u32x4{0u, 0u, 0u, 0u};
                if (qq < 2 * D) {  // key row qq / (D / 8), pieces of 8 elements
                    *(u32x4*)(sk + (e * 16 + qq / (D / 8)) * KLD + (qq % (D / 8)) * 8) = v;
                } else {
                    const int q2 = qq - 2 * D;
                    if (nvalid < 16) {
                        // zero the values of slots past the last key (they may hold anything)
                        const int half = q2 & 1;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int s0 = half * 8 + 2 * j;
                            const uint32_t m = (s0 < nvalid ? 0x0000FFFFu : 0u) | (s0 + 1 < nvalid ? 0xFFFF0000u : 0u);
                            v[j] &= m;
                        }
                    }
                    // piece q2 = slots 8 h .. 8 h + 7 of row d: groups g = 2 h and 2 h + 1
                    const int half = q2 & 1;
                    bf16_t* row = sv + ((e >> 1) * D + (q2 >> 1)) * AT_SVLD + (e & 1) * 4;
                    *(u32x2*)(row + (2 * half) * 8) = u32x2{v[0], v[1]};
                    *(u32x2*)(row + (2 * half + 1) * 8) = u32x2{v[2], v[3]};
                }
            }
        }
    };


    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    __syncthreads();  // page ids in LDS
    // flag pages the chunk needs that lie beyond the table or outside the pool (their slots read as zero)
    for (int j = tid; j < chunk_tokens / 16 && t0 + 16 * j < t1; j += NT) {
        if ((t0 >> 4) + j >= max_pages) set_err(err, DFLASH_DEVERR_POS);
        else if (spg[j] < 0 || spg[j] >= n_pages) set_err(err, DFLASH_DEVERR_PAGE);
    }
    // always issued (a chunk without keys reads the block page and never stashes it), so that the block step
    // below waits only for its own loads
    prefetch(0);
    if (c == 0) {
        // the block's keys (L of the 16 slots): S = (K_hi + K_lo)(Q_hi + Q_lo)^T in one accumulator chain, then
        // the first online-softmax step, then O^T = (V_hi + V_lo)^T P^T with P = P_hi + P_lo; values of slots
        // past L are zeroed (they may hold anything)
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sa = mfma16(bk[pl][s], qf[s], sa);
                sa = mfma16(bk[pl][s], ql[s], sa);
            }
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = 4 * g + i < L ? sa[i] * scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // L >= 1, so every row has a finite maximum
        m_run = mx;
        float p4[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p4[i] = __builtin_amdgcn_exp2f(x[i] - mx);
            psum += p4[i];
        }
        l_run = psum;
        u32x4 phi = u32x4{0u, 0u, 0u, 0u}, plo = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float v0 = p4[2 * j], v1 = p4[2 * j + 1];
            const uint32_t h2 = f2bf2(v0, v1);
            phi[j] = h2;
            plo[j] = f2bf2(v0 - __uint_as_float(h2 << 16), v1 - __uint_as_float(h2 & 0xFFFF0000u));
        }
        uint32_t vm[2];
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
            const int s0 = 4 * g + 2 * wd;
            vm[wd] = (s0 < L ? 0x0000FFFFu : 0u) | (s0 + 1 < L ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x2 v = bv[t >> 1][dt];
                o[dt] = mfma16(u32x4{v[0] & vm[0], v[1] & vm[1], 0u, 0u}, (t & 1) ? plo : phi, o[dt]);
            }
    }
    // round rr: the sub-chunk of context keys starting at ts; the next round's loads are issued before the
    // MFMAs of this one
    for (int rr = 0; rr < R; ++rr) {
        const int ts = ts_of(rr);
        __syncthreads();
        stash(rr);
        __syncthreads();
        if (rr + 1 < R) prefetch(rr + 1);
        // scores S^T[key][query]: lane holds keys 4g+i of each page for query r
        float x[NPG][4];
        // every page's tile first (independent MFMA chains; hi and lo query terms in separate
        // accumulators), then scale, and mask only in a sub-chunk that runs past the chunk's end
        f32x4 sh[NPG], sl[NPG];
#pragma unroll
        for (int e = 0; e < NPG; ++e) {
            sh[e] = f32x4{0.f, 0.f, 0.f, 0.f};
            sl[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < NPG; ++e) {
                const u32x4 kf = ld16(sk + (e * 16 + r) * KLD + g * 8 + s * 32);
                sh[e] = mfma16(kf, qf[s], sh[e]);
                sl[e] = mfma16(kf, ql[s], sl[e]);
            }
#pragma unroll
        for (int e = 0; e < NPG; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[e][i] = (sh[e][i] + sl[e][i]) * scale_log2;
        if (ts + SUB > t1) {
            const int nk = t1 - ts;
#pragma unroll
            for (int e = 0; e < NPG; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[e][i] = 16 * e + 4 * g + i < nk ? x[e][i] : -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < NPG; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[e][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        // while every key so far is masked use 0 as reference: alpha and p become 0, not exp2(-inf + inf)
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
        m_run = m_new;
        float p[NPG][4];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < NPG; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[e][i] = __builtin_amdgcn_exp2f(x[e][i] - m_ref);
                psum += p[e][i];
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
        }
        // O^T += V^T P^T over the sub-chunk's 32-key slices; P enters as two bfloat16 terms (hi + lo)
#pragma unroll
        for (int hk = 0; hk < NPG / 2; ++hk) {
            if (ts + 32 * hk >= t1) break;  // uniform: the rest of the round is masked
            u32x4 phi, plo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v0 = p[2 * hk + (j >> 1)][2 * (j & 1)], v1 = p[2 * hk + (j >> 1)][2 * (j & 1) + 1];
                const uint32_t h2 = f2bf2(v0, v1);
                phi[j] = h2;
                plo[j] = f2bf2(v0 - __uint_as_float(h2 << 16), v1 - __uint_as_float(h2 & 0xFFFF0000u));
            }
            // four d-tiles' operands at a time, then their MFMAs term by term (independent accumulators back to
            // back; each tile still adds its terms in the same order)
#pragma unroll
            for (int d0 = 0; d0 < DT; d0 += 4) {
                u32x4 vf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) vf[u] = ld16(sv + (hk * D + (d0 + u) * 16 + r) * AT_SVLD + g * 8);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[d0 + u] = mfma16(vf[u], phi, o[d0 + u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[d0 + u] = mfma16(vf[u], plo, o[d0 + u]);
            }
        }
    }

    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const size_t base = (((size_t)b * nq + h) * C1 + c) * 16 + r;
    float* op = opart + base * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(float4*)(op + dt * 16 + 4 * g) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
        mlpart[base * 2 + 0] = m_run;
        mlpart[base * 2 + 1] = l_tot;
    }
}

// ------------------------------------------------------------------------------------------------------
// merge of the chunk partials -> o (rounded), and the float32 attention kernel
// ------------------------------------------------------------------------------------------------------
// One wave per (request, query head, block row): lanes first combine the chunks' (m, l) in the log2 domain,
// then each lane accumulates two of the 128 output columns over the chunks in a fixed order.
// TWO: two output columns per lane (d = 128: lane and lane + 64), else one (d = 64).
template <typename T, bool TWO>
__global__ __launch_bounds__(256) void attn_merge(const float* __restrict__ opart, const float* __restrict__ mlpart,
                                                  int B, int L, int nq, int d, int C1, T* __restrict__ o) {
    __shared__ float wsh[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int item = blockIdx.x * 4 + w;  // (b, row, h)
    if (item >= B * L * nq) return;
    const int h = item % nq;
    const int row = (item / nq) % L;
    const int b = item / (nq * L);
    const size_t base = ((size_t)b * nq + h) * C1;
    const size_t base_o = ((size_t)(b * L + row) * nq + h) * d, plane = (size_t)B * L * nq * d;
    float M = -INFINITY;
    for (int c = lane; c < C1; c += 64) M = fmaxf(M, mlpart[((base + c) * 16 + row) * 2]);
    M = wave_max(M);
    float lsum = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int c0 = 0; c0 < C1; c0 += 64) {
        const int c = c0 + lane;
        float wgt = 0.f;
        if (c < C1) {
            const float mc = mlpart[((base + c) * 16 + row) * 2];
            wgt = mc == -INFINITY ? 0.f : exp2f(mc - M);
            lsum += wgt * mlpart[((base + c) * 16 + row) * 2 + 1];
        }
        wsh[w][lane] = wgt;
        __builtin_amdgcn_wave_barrier();
        const int cn = min(64, C1 - c0);
        const float* op = opart + ((base + c0) * 16 + row) * d;
#pragma unroll 16  // sixteen chunks' loads in flight per batch (the additions keep their order)
        for (int i = 0; i < cn; ++i) {
            const float wi = wsh[w][i];
            acc0 += wi * op[(size_t)i * 16 * d + lane];
            if (TWO) acc1 += wi * op[(size_t)i * 16 * d + lane + 64];
        }
        __builtin_amdgcn_wave_barrier();
    }
    lsum = wave_sum(lsum);
    put_act(o, plane, base_o + lane, acc0 / lsum);
    if (TWO) put_act(o, plane, base_o + lane + 64, acc1 / lsum);
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
        const dim3 grid(attn_slots(p), nkv, B);
        if (p.chunk_tokens % attn_sub(G) || p.chunk_tokens > 16 * AT_MAX_PAGES || (d != 64 && d != 128))
            return hipErrorInvalidValue;
#define DF_ATTN_NT(GG, NT, DD)                                                                                     \
    DF_LAUNCH((attn_bf16<GG, 64, NT, DD>), grid, dim3(64 * GG), 0, st, (const bf16_t*)q, (const bf16_t*)kb,    \
              (const bf16_t*)vbt, (const bf16_t*)kpool, (const bf16_t*)vpool, layer, n_pages, page_table,       \
              max_pages, ctx_len, max_ctx, p.chunk_tokens, L, nq, nkv, opart, mlpart, err)
#define DF_ATTN(GG)                                       \
    if (d == 64) {                                        \
        if (p.stream_kv) DF_ATTN_NT(GG, true, 64);        \
        else DF_ATTN_NT(GG, false, 64);                   \
    } else {                                              \
        if (p.stream_kv) DF_ATTN_NT(GG, true, 128);       \
        else DF_ATTN_NT(GG, false, 128);                  \
    }
        switch (G) {
            case 1: DF_ATTN(1); break;
            case 2: DF_ATTN(2); break;
            case 4: DF_ATTN(4); break;
            case 8: DF_ATTN(8); break;
            default: return hipErrorInvalidValue;
        }
#undef DF_ATTN
#undef DF_ATTN_NT
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
    const long n = (long)B * L * nq;  // one wave each (d = 64 or 128)
    const dim3 grid((unsigned)((n + 3) / 4));
    if (d != 64 && d != 128) return hipErrorInvalidValue;
    if (bf16) {
        if (d == 128)
            hipLaunchKernelGGL((attn_merge<bf16_t, true>), grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d,
                               attn_slots(p), (bf16_t*)o);
        else
            hipLaunchKernelGGL((attn_merge<bf16_t, false>), grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d,
                               attn_slots(p), (bf16_t*)o);
    } else {
        if (d == 128)
            hipLaunchKernelGGL((attn_merge<float, true>), grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d,
                               attn_slots(p), (float*)o);
        else
            hipLaunchKernelGGL((attn_merge<float, false>), grid, dim3(256), 0, st, opart, mlpart, B, L, nq, d,
                               attn_slots(p), (float*)o);
    }
    return hipGetLastError();
}

}  // namespace df
