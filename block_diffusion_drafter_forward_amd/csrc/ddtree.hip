// DDTree on the drafter's marginals ("Accelerating Speculative Decoding with Block Diffusion Draft Trees",
// §3.4.4 and §3.4.5): the per-position top-K log-probabilities (K up to 1024), the best-first construction
// of the top-B prefix tree over rank tuples, and the greedy verifier walk over the target's choices.
#include "common.h"
#include "kernels.h"

namespace df {

// ------------------------------------------------------------------------------------------------------
// wide top-K of one logits row: radix select of the K-th largest key, gather, bitonic sort
// ------------------------------------------------------------------------------------------------------
// One workgroup of 1024 threads per row.  Floats map to unsigned keys that order like the floats
// (negative: all bits flipped; non-negative: sign bit set; -0 taken as +0).  Three radix passes (11, 11 and 10 bits, the
// first one over the row also accumulating an online max / sum of exponentials) find the key T of the K-th
// largest value and how many entries equal to T belong to the top K; a gather takes every key above T and
// the entries equal to T (all of them in the common case where they all fit, else the ones with the
// smallest ids, found by a radix select on the ids of the tied entries).  When the keys at or above the
// first pass's bin number at most TK_CAND (a few thousand for continuous logits), they are gathered into
// LDS once and every later step runs there, so the row is read twice; otherwise every step re-reads the
// row.  Rows are read with 16-byte loads, eight in flight per thread.  The K winners are sorted by (value descending, id ascending) with a bitonic
// network in LDS; log-probabilities are value - logsumexp(row).
#define TK_THREADS 1024
#define TK_MAX 1024
#define TK_BINS 2048
#define TK_UNROLL 8

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;  // -0 and +0 are one value: equal logits tie by id
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Calls f(id, key) for every element of the row; 16-byte loads, TK_UNROLL of them in flight per thread.
// Rows whose start is not 16-byte aligned or whose length is not a multiple of 4 take a scalar tail.
template <typename F>
__device__ __forceinline__ void tk_for_row(const float* __restrict__ x, int V, F&& f) {
    const int t = threadIdx.x;
    const bool vec = (((uintptr_t)x) & 15) == 0;
    const int nv = vec ? V / 4 : 0;
    const float4* x4 = (const float4*)x;
    for (int i0 = 0; i0 < nv; i0 += TK_THREADS * TK_UNROLL) {
        float4 v[TK_UNROLL];
#pragma unroll
        for (int u = 0; u < TK_UNROLL; ++u) {
            const int i = i0 + u * TK_THREADS + t;
            v[u] = i < nv ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < TK_UNROLL; ++u) {
            const int i = i0 + u * TK_THREADS + t;
            if (i < nv) {
                f(4 * i + 0, order_key(v[u].x));
                f(4 * i + 1, order_key(v[u].y));
                f(4 * i + 2, order_key(v[u].z));
                f(4 * i + 3, order_key(v[u].w));
            }
        }
    }
    for (int j = 4 * nv + t; j < V; j += TK_THREADS) f(j, order_key(x[j]));
}

__device__ __forceinline__ float tk_block_max(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < TK_THREADS / 64; ++i) t = fmaxf(t, red[i]);
    return t;
}

// Radix step over the histogram: the bin (from the top) that holds the krem-th largest, and the rank left
// inside it.  Every thread takes two adjacent bins from the top (nbins <= 2 * TK_THREADS), so neighbouring
// lanes read neighbouring words; a block-wide prefix sum over the pairs finds the bin.  All threads call it.
__device__ __forceinline__ void tk_pick_bin(const uint32_t* hist, int nbins, int krem, int* s_bin, int* s_krem) {
    __shared__ int wsum[TK_THREADS / 64];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int b0 = nbins - 1 - 2 * t;
    const int h0 = b0 >= 0 ? (int)hist[b0] : 0, h1 = b0 >= 1 ? (int)hist[b0 - 1] : 0;
    const int pair = h0 + h1;
    int incl = pair;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int i = 0; i < TK_THREADS / 64; ++i) base += i < w ? wsum[i] : 0;
    const int excl = base + incl - pair;
    if (excl < krem && excl + h0 >= krem) {
        *s_bin = b0;
        *s_krem = krem - excl;
    } else if (excl + h0 < krem && excl + pair >= krem) {
        *s_bin = b0 - 1;
        *s_krem = krem - excl - h0;
    }
    __syncthreads();  // wsum is free again
}

// The selection after the first radix pass: radix passes 2 and 3 (11 and 10 bits) among the keys with
// the chosen top bits, the gather of every key above the K-th key T, and the entries equal to T (all, or
// the smallest ids by a radix select on ids).  `each(f)` calls f(id, key) for every element of the source:
// the row itself, or the candidates already gathered into LDS.  Leaves the K winners in skey / sid.
template <typename Each>
__device__ void tk_select(Each&& each, uint32_t prefix, uint32_t mask, int krem, int K, uint32_t* hist,
                          float* red, uint32_t* skey, int* sid, int* s_bin, int* s_krem, int* s_slot) {
    const int t = threadIdx.x;
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const int nb = pass == 0 ? 2048 : 1024;
        for (int i = t; i < TK_BINS; i += TK_THREADS) hist[i] = 0u;
        __syncthreads();
        each([&](int, uint32_t k) {
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
        });
        __syncthreads();
        tk_pick_bin(hist, nb, krem, s_bin, s_krem);
        __syncthreads();
        prefix |= (uint32_t)*s_bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        krem = *s_krem;
        __syncthreads();
    }
    const uint32_t T = prefix;  // key of the K-th largest entry; krem entries equal to T are in the top K
    if (t == 0) *s_slot = 0;
    __syncthreads();
    int n_eq = 0;
    each([&](int j, uint32_t k) {
        if (k > T) {
            const int slot = atomicAdd(s_slot, 1);
            skey[slot] = k;
            sid[slot] = j;
        }
        n_eq += k == T ? 1 : 0;
    });
    n_eq = (int)block_sum((float)n_eq, red);  // exact: counts stay far below 2^24
    int id_cut = 0x7FFFFFFF;
    if (n_eq > krem) {
        uint32_t ipre = 0u, imask = 0u;
        int irem = krem;
        for (int shift = 22; shift >= 0; shift -= 11) {  // ids < 2^31: 9 + 11 + 11 bits, smallest first
            const int nb = shift == 22 ? 512 : 2048;
            for (int i = t; i < TK_BINS; i += TK_THREADS) hist[i] = 0u;
            __syncthreads();
            each([&](int j, uint32_t k) {
                if (k == T && ((uint32_t)j & imask) == ipre)
                    atomicAdd(&hist[nb - 1 - (((uint32_t)j >> shift) & (nb - 1))], 1u);
            });
            __syncthreads();
            tk_pick_bin(hist, nb, irem, s_bin, s_krem);  // bins reversed: "largest" = smallest id digit
            __syncthreads();
            ipre |= (uint32_t)(nb - 1 - *s_bin) << shift;
            imask |= (uint32_t)(nb - 1) << shift;
            irem = *s_krem;
            __syncthreads();
        }
        id_cut = (int)ipre;  // the krem-th smallest id among the tied entries
    }
    each([&](int j, uint32_t k) {
        if (k == T && j <= id_cut) {
            const int slot = atomicAdd(s_slot, 1);
            skey[slot] = k;
            sid[slot] = j;
        }
    });
    __syncthreads();
}

#define TK_CAND 6144  // candidates kept in LDS after the first radix pass

// Sort entries are packed as key << 32 | ~id: a larger packed value is a larger key, then a smaller id.
__device__ __forceinline__ uint64_t tk_pack(uint32_t key, int id) {
    return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)id);
}
__device__ __forceinline__ uint32_t tk_pkey(uint64_t p) { return (uint32_t)(p >> 32); }
__device__ __forceinline__ int tk_pid(uint64_t p) { return (int)~(uint32_t)p; }
// The value of lane (lane ^ lx), lx in {1, 2, 4, 8, 16, 32}, with VALU lane moves only: DPP quad
// permutations (1, 2), row shifts (4), a row rotation (8), and the row-swap permutes (16, 32).
__device__ __forceinline__ uint32_t tk_xor_lane(uint32_t v, int lx) {
    const int x = (int)v;
    const int lane = threadIdx.x & 63;
    switch (lx) {
        case 1:
            return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        case 2:
            return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        case 4: {
            const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0xF, false);  // row_shl:4, lane + 4
            const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false);  // row_shr:4, lane - 4
            return (uint32_t)((lane & 4) ? dn : up);
        }
        case 8:
            return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);  // row_ror:8
        case 16: {
            const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            return (lane & 16) ? p[0] : p[1];
        }
        default: {
            const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            return (lane & 32) ? p[0] : p[1];
        }
    }
}
__device__ __forceinline__ uint64_t tk_shfl_xor64(uint64_t v, int lx) {
    const uint32_t lo = tk_xor_lane((uint32_t)v, lx);
    const uint32_t hi = tk_xor_lane((uint32_t)(v >> 32), lx);
    return ((uint64_t)hi << 32) | lo;
}

// One bitonic stage between a lane's own elements s and s ^ J (J < E), in runs of size kk.
template <int E, int J>
__device__ __forceinline__ void tk_lane_stage(uint64_t (&v)[E], int base, int kk) {
#pragma unroll
    for (int s = 0; s < E; ++s) {
        if ((s & J) == 0 && (s ^ J) < E) {
            const int q = s ^ J;
            const bool desc = ((base + s) & kk) == 0;  // this run is sorted largest first
            const uint64_t a = v[s], b = v[q];
            const bool sw = desc ? b > a : a > b;
            v[s] = sw ? b : a;
            v[q] = sw ? a : b;
        }
    }
}

// Bitonic sort, largest first, of the 64E packed entries a wave holds (lane l: run positions E l + s), in
// registers: swaps inside a lane, shuffles across lanes.  No barrier.
template <int E>
__device__ __forceinline__ void tk_wave_sort(uint64_t (&v)[E]) {
    const int lane = threadIdx.x & 63, base = E * lane;
#pragma unroll
    for (int kk = 2; kk <= 64 * E; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            if (j < E) {
                if (j == 1)
                    tk_lane_stage<E, 1>(v, base, kk);
                else
                    tk_lane_stage<E, 2>(v, base, kk);
            } else {
                const int lx = j / E;
                const bool lower = (lane & lx) == 0;
#pragma unroll
                for (int s = 0; s < E; ++s) {
                    const uint64_t o = tk_shfl_xor64(v[s], lx);
                    const bool desc = ((base + s) & kk) == 0;
                    const bool take_max = lower == desc;
                    v[s] = take_max ? (o > v[s] ? o : v[s]) : (o < v[s] ? o : v[s]);
                }
            }
        }
    }
}

// Number of entries of the descending run a[0, len) larger than x, len <= RUN (a power of two): a
// fixed-length binary search, so that several of them interleave.
template <int RUN>
__device__ __forceinline__ int tk_count_larger(const uint64_t* a, int len, uint64_t x) {
    int pos = 0;
#pragma unroll
    for (int step = RUN; step > 0; step >>= 1)
        if (pos + step <= len && a[pos + step - 1] > x) pos += step;
    return pos;
}

// One four-way merge round over the first n entries: runs of RUN entries in groups of four, the last run
// holding fewer than RUN real entries being cut at n.  An entry's place in its merged group is its index
// in its own run plus the number of larger entries in each of the three other runs (three independent
// searches); entries are distinct, so the places are a permutation of [0, n).
template <int E, int RUN>
__device__ __forceinline__ void tk_merge4(const uint64_t* src, uint64_t* dst, int n) {
    const int t = threadIdx.x;
#pragma unroll
    for (int s = 0; s < E; ++s) {
        const int i = t + TK_THREADS * s;
        if (i < n) {
            const uint64_t x = src[i];
            const int g0 = i & ~(4 * RUN - 1), a = (i - g0) / RUN;
            int pos = g0 + (i & (RUN - 1));
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int len = min(RUN, n - (g0 + b * RUN));
                if (b != a && len > 0) pos += tk_count_larger<RUN>(src + g0 + b * RUN, len, x);
            }
            dst[pos] = x;
        }
    }
}

// Sorts the packed entries [0, n) of buf, largest first, n <= 1024 E; buf holds 2048 E entries (the second
// half is the merge target).  Each wave sorts a run of 64E in registers (a run past n is skipped, one cut
// by n is padded with entries smaller than every real one); two four-way merge rounds over the real
// entries then join the runs, one barrier each.  All threads call it; the result is in buf[0, n).
template <int E>
__device__ __forceinline__ void tk_sort_lds(int n, uint64_t* buf) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    constexpr int R = 64 * E, P = TK_THREADS * E;
    const bool live = w * R < n;
    uint64_t v[E];
    if (live) {
#pragma unroll
        for (int s = 0; s < E; ++s) {
            const int i = w * R + E * lane + s;
            v[s] = i < n ? buf[i] : tk_pack(0u, 0x7FFFFFFF - (i - n));
        }
        tk_wave_sort<E>(v);
    }
    __syncthreads();  // every entry read before the runs are written back
    if (live) {
#pragma unroll
        for (int s = 0; s < E; ++s) {
            const int i = w * R + E * lane + s;
            if (i < n) buf[i] = v[s];  // the padding sorts last
        }
    }
    __syncthreads();
    tk_merge4<E, R>(buf, buf + P, n);
    __syncthreads();
    tk_merge4<E, 4 * R>(buf + P, buf, n);
    __syncthreads();
}

// n <= 2 * TK_THREADS
__device__ __forceinline__ void tk_sort_any(int n, uint64_t* buf) {
    if (n <= TK_THREADS)
        tk_sort_lds<1>(n, buf);
    else
        tk_sort_lds<2>(n, buf);
}

// The whole selection for one row in one workgroup: ids / lp of the row's K best (value descending, id
// ascending) and log-probabilities value - logsumexp.
__device__ __forceinline__ void tk_row(const float* __restrict__ x, int V, int K, int32_t* __restrict__ ids,
                       float* __restrict__ lp) {
    __shared__ uint32_t hist[TK_BINS];
    __shared__ float red[TK_THREADS / 64];
    __shared__ float red2[TK_THREADS / 64];
    __shared__ uint32_t skey[TK_MAX];
    __shared__ int sid[TK_MAX];
    __shared__ uint64_t sbuf[2 * TK_MAX];
    __shared__ uint32_t ckey[TK_CAND];
    __shared__ int cid[TK_CAND];
    __shared__ int s_bin, s_krem, s_slot, s_cnt;
    const int t = threadIdx.x;

    // pass 1: online max / sum of exponentials, and the histogram of the top 11 key bits
    for (int i = t; i < TK_BINS; i += TK_THREADS) hist[i] = 0u;
    if (t == 0) s_cnt = 0;
    __syncthreads();
    float m = -INFINITY, se = 0.f;
    tk_for_row(x, V, [&](int, uint32_t k) {
        const float v = key_value(k);
        if (v > m) {
            se = se * expf(m - v) + 1.f;
            m = v;
        } else {
            se += expf(v - m);
        }
        atomicAdd(&hist[k >> 21], 1u);
    });
    const float mx = tk_block_max(m, red);
    se = m == -INFINITY ? 0.f : se * expf(m - mx);
    se = block_sum(se, red2);
    const float lse = mx + logf(se);
    tk_pick_bin(hist, TK_BINS, K, &s_bin, &s_krem);
    const uint32_t b1 = (uint32_t)s_bin;
    const int krem = s_krem;
    const int n_cand = (K - krem) + (int)hist[b1];  // keys in bin b1 or above
    __syncthreads();
    if (n_cand <= TK_CAND) {
        // gather the candidates once; the rest of the selection runs on LDS
        tk_for_row(x, V, [&](int j, uint32_t k) {
            if ((k >> 21) >= b1) {
                const int slot = atomicAdd(&s_cnt, 1);
                ckey[slot] = k;
                cid[slot] = j;
            }
        });
        __syncthreads();
        auto each = [&](auto&& f) {
            for (int i = t; i < n_cand; i += TK_THREADS) f(cid[i], ckey[i]);
        };
        tk_select(each, b1 << 21, 0xFFE00000u, krem, K, hist, red, skey, sid, &s_bin, &s_krem, &s_slot);
    } else {
        auto each = [&](auto&& f) { tk_for_row(x, V, f); };
        tk_select(each, b1 << 21, 0xFFE00000u, krem, K, hist, red, skey, sid, &s_bin, &s_krem, &s_slot);
    }
    for (int i = t; i < K; i += TK_THREADS) sbuf[i] = tk_pack(skey[i], sid[i]);
    __syncthreads();
    tk_sort_lds<1>(K, sbuf);
    for (int i = t; i < K; i += TK_THREADS) {
        ids[i] = tk_pid(sbuf[i]);
        lp[i] = key_value(tk_pkey(sbuf[i])) - lse;
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows(const float* __restrict__ logits, int64_t stride, int V,
                                                         int K, int32_t* __restrict__ ids, float* __restrict__ lp) {
    tk_row(logits + (size_t)blockIdx.x * stride, V, K, ids + (size_t)blockIdx.x * K, lp + (size_t)blockIdx.x * K);
}

// ------------------------------------------------------------------------------------------------------
// the same top-K with each row split over C workgroups
// ------------------------------------------------------------------------------------------------------
// With few rows, one workgroup per row leaves most of the chip idle.  topk_chunk takes one chunk of CL
// entries of a row into registers, computes its max and sum of exponentials, and finds a threshold key t_c
// at or below its kt-th largest key (kt about 1.5 K / C: the chunk's expected share of the row's top K, with
// room to spare) by histograms over the chunk's key range, refined once inside the bin that holds it.  It
// writes every entry with key >= t_c (at most capc; more marks the chunk as overflowed) and its partial
// (max, sum, t_c, count).  topk_merge sorts the union of the candidates (a few thousand) and takes the first
// K.  That is the row's top K whenever the K-th key T is >= every t_c: an entry left out scores below its
// chunk's t_c <= T and so has K entries ahead of it.  Chunks with t_c > T are read again for their entries
// in [T, t_c), and the union is sorted once more; an overflow falls back to the one-workgroup selection.
#define TK_PER 12            // chunk entries per thread, held in registers
#define TK_SORT_MAX 2048     // candidates a merge sorts

__global__ __launch_bounds__(TK_THREADS) void topk_chunk(const float* __restrict__ logits, int64_t stride, int V,
                                                          int C, int CL, int kt, int capc, uint2* __restrict__ cand,
                                                          float4* __restrict__ part) {
    __shared__ uint32_t hist[TK_BINS];
    __shared__ float fred[TK_THREADS / 64];
    __shared__ uint32_t ured[2 * (TK_THREADS / 64)];
    __shared__ int s_bin, s_krem;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, row = blockIdx.x / C, c = blockIdx.x % C;
    const int j0 = c * CL, n = min(V - j0, CL);
    const float* x = logits + (size_t)row * stride + j0;
    for (int i = t; i < TK_BINS; i += TK_THREADS) hist[i] = 0u;
    float v[TK_PER];
#pragma unroll
    for (int q = 0; q < TK_PER; ++q) {
        const int e = q * TK_THREADS + t;
        v[q] = e < n ? x[e] : -INFINITY;
    }
    uint32_t k[TK_PER];
    float m = -INFINITY;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int q = 0; q < TK_PER; ++q) {
        k[q] = order_key(v[q]);
        if (q * TK_THREADS + t < n) {
            m = fmaxf(m, v[q]);
            lo = min(lo, k[q]);
            hi = max(hi, k[q]);
        }
    }
    // one block reduction: the chunk's max value and its smallest and largest keys
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        m = fmaxf(m, __shfl_xor(m, o, 64));
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    }
    if (lane == 0) {
        fred[w] = m;
        ured[w] = lo;
        ured[TK_THREADS / 64 + w] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TK_THREADS / 64; ++i) {
        m = fmaxf(m, fred[i]);
        lo = min(lo, ured[i]);
        hi = max(hi, ured[TK_THREADS / 64 + i]);
    }
    float se = 0.f;  // sum of exp(v - max) over the chunk, finished with the count below
    if (m != -INFINITY) {
#pragma unroll
        for (int q = 0; q < TK_PER; ++q) se += __expf(v[q] - m);  // exp(-inf) = 0 for the padding
    }
    uint32_t tc = 0u;  // every entry is a candidate
    if (n > kt) {
        tc = lo;
        int need = kt;
        uint32_t L = lo, H = hi;
        for (int round = 0; round < 2 && H > L; ++round) {
            const uint32_t span = H - L;
            const int sh = max(0, 32 - __clz((int)span) - 11);  // (key - L) >> sh < TK_BINS
            if (round > 0) {
                for (int i = t; i < TK_BINS; i += TK_THREADS) hist[i] = 0u;
                __syncthreads();
            }
#pragma unroll
            for (int q = 0; q < TK_PER; ++q)
                if (q * TK_THREADS + t < n && k[q] >= L && k[q] <= H) atomicAdd(&hist[(k[q] - L) >> sh], 1u);
            __syncthreads();
            tk_pick_bin(hist, TK_BINS, need, &s_bin, &s_krem);
            const int b = s_bin, rem = s_krem;
            const int inbin = (int)hist[b];
            __syncthreads();
            tc = L + ((uint32_t)b << sh);
            if (sh == 0 || (need - rem) + inbin <= need + 32) break;
            need = rem;  // refine inside the bin
            L = tc;
            H = min(H, tc + ((1u << sh) - 1u));
        }
    }
    uint32_t cnt = 0u;
#pragma unroll
    for (int q = 0; q < TK_PER; ++q) cnt += (q * TK_THREADS + t < n && k[q] >= tc) ? 1u : 0u;
    // block prefix sum of the counts, with the block sum of se alongside
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += y;
        se += __shfl_xor(se, o, 64);
    }
    __syncthreads();  // fred / ured are reused
    if (lane == 63) ured[w] = incl;
    if (lane == 0) fred[w] = se;
    __syncthreads();
    uint32_t off = 0u, total = 0u;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < TK_THREADS / 64; ++i) {
        const uint32_t q = ured[i];
        off += i < w ? q : 0u;
        total += q;
        sum += fred[i];
    }
    off += incl - cnt;
    const bool ovf = total > (uint32_t)capc;
    if (!ovf) {
        uint2* out = cand + (size_t)blockIdx.x * capc;
#pragma unroll
        for (int q = 0; q < TK_PER; ++q) {
            const int e = q * TK_THREADS + t;
            if (e < n && k[q] >= tc) out[off++] = make_uint2(k[q], (uint32_t)(j0 + e));
        }
    }
    if (t == 0) part[blockIdx.x] = make_float4(m, sum, __uint_as_float(tc), __int_as_float(ovf ? -1 : (int)total));
}

#define TK_SLOTS_PT 8  // candidate slots each merge thread loads at once
#define TK_BIN_MAX 64  // fullest bin the merge's counting sort takes (more: heavy ties, left to the sort)

// Bin of key kk (>= tmax) in the merge's counting sort: descending keys, width 2^sh, bin 0 from kmax down.
__device__ __forceinline__ int tk_cbin(uint32_t kk, uint32_t kmax, int sh, int nb) {
    return kk >= kmax ? 0 : min(nb - 1, (int)((kmax - kk) >> sh));
}

__global__ __launch_bounds__(TK_THREADS) void topk_merge(const float* __restrict__ logits, int64_t stride, int V,
                                                          int K, int C, int CL, int capc,
                                                          const uint2* __restrict__ cand,
                                                          const float4* __restrict__ part, int32_t* __restrict__ ids,
                                                          float* __restrict__ lp) {
    __shared__ uint64_t cb[2 * TK_SORT_MAX];
    __shared__ uint32_t ptc[64];
    __shared__ int pcnt[64], poff[65];
    __shared__ int s_n, s_ovf;
    __shared__ float s_lse;
    __shared__ uint32_t bcnt[TK_BINS], bcur[TK_BINS], wsum[TK_THREADS / 64], wocc[TK_THREADS / 64];
    __shared__ uint32_t s_tmax, s_kmax;
    const int t = threadIdx.x, row = blockIdx.x;
    const float* x = logits + (size_t)row * stride;
    const uint2* cr = cand + (size_t)row * C * capc;
    const int slots = C * capc;
    // the partials and the first candidate slots in one round trip (slots past a chunk's count are ignored)
    float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < C) q4 = part[(size_t)row * C + t];
    uint2 e[TK_SLOTS_PT];
#pragma unroll
    for (int u = 0; u < TK_SLOTS_PT; ++u) {
        const int i = u * TK_THREADS + t;
        e[u] = i < slots ? cr[i] : make_uint2(0u, 0u);
    }
    if (t < 64) {  // wave 0, lane c = chunk c: offsets, overflow and logsumexp by lane reductions
        const bool on = t < C;
        const int cnt = on ? __float_as_int(q4.w) : 0;
        const bool bad = on && cnt < 0;
        int incl = bad ? 0 : cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (t >= o) incl += y;
        }
        const int total = __shfl(incl, 63, 64);
        float M = on ? q4.x : -INFINITY;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        float S = (on && q4.x != -INFINITY) ? q4.y * __expf(q4.x - M) : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) S += __shfl_xor(S, o, 64);
        const bool any_bad = __ballot(bad) != 0ull;
        uint32_t tm = on ? __float_as_uint(q4.z) : 0u;  // the largest chunk threshold
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) tm = max(tm, (uint32_t)__shfl_xor((int)tm, o, 64));
        if (on) {
            pcnt[t] = cnt;
            ptc[t] = __float_as_uint(q4.z);
            poff[t] = incl - (bad ? 0 : cnt);
        }
        if (t == 0) {
            poff[C] = total;
            s_n = (any_bad || total > TK_SORT_MAX || total < K) ? -1 : total;
            s_ovf = 0;
            s_lse = M + __logf(S);
            s_tmax = tm;
            s_kmax = max(order_key(M), tm);
        }
    }
    __syncthreads();
    const float lse = s_lse;
    int n = s_n;
    bool fallback = n < 0;  // a chunk overflowed, or too many candidates: the one-workgroup selection
    if (!fallback) {
    for (int i0 = 0; i0 < slots; i0 += TK_SLOTS_PT * TK_THREADS) {
#pragma unroll
        for (int u = 0; u < TK_SLOTS_PT; ++u) {
            const int i = i0 + u * TK_THREADS + t;
            if (i0 > 0) e[u] = i < slots ? cr[i] : make_uint2(0u, 0u);
            if (i < slots) {
                const int c = i / capc, r = i - c * capc;
                if (r < pcnt[c]) cb[poff[c] + r] = tk_pack(e[u].x, (int)e[u].y);
            }
        }
    }
    __syncthreads();
    {
        // Counting sort of the candidates at or above tmax = the largest t_c, taken when at least K of them
        // are: the K-th key T is then >= every t_c, so no chunk is read again, and every candidate below tmax
        // ranks K or later.  Keys bin by (kmax - key) >> sh, so that bins run in descending key order; an
        // entry's place is its bin's start plus the number of larger (key, ~id) pairs in its bin.  A bin of
        // more than TK_BIN_MAX entries (heavy ties) or fewer than K such candidates leave the row to the sort.
        const uint32_t tmax = s_tmax, kmax = s_kmax, span = kmax - tmax;
        const int sh = span >> 11 ? 32 - __clz((int)(span >> 11)) : 0;  // span >> sh < TK_BINS
        const int nb = (int)(span >> sh) + 1;
        for (int b = t; b < nb; b += TK_THREADS) bcnt[b] = 0u;
        __syncthreads();
        for (int i = t; i < n; i += TK_THREADS) {
            const uint32_t kk = tk_pkey(cb[i]);
            if (kk >= tmax) atomicAdd(&bcnt[tk_cbin(kk, kmax, sh, nb)], 1u);
        }
        __syncthreads();
        // exclusive scan of the bin counts (two bins per thread) with the fullest bin alongside
        const int lane = t & 63, w = t >> 6, b0 = 2 * t;
        const uint32_t c0 = b0 < nb ? bcnt[b0] : 0u, c1 = b0 + 1 < nb ? bcnt[b0 + 1] : 0u;
        uint32_t incl = c0 + c1, occ = max(c0, c1);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
            if (lane >= o) incl += y;
            occ = max(occ, (uint32_t)__shfl_xor((int)occ, o, 64));
        }
        if (lane == 63) wsum[w] = incl;
        if (lane == 0) wocc[w] = occ;
        __syncthreads();
        uint32_t before = 0u, total = 0u;
#pragma unroll
        for (int i = 0; i < TK_THREADS / 64; ++i) {
            before += i < w ? wsum[i] : 0u;
            total += wsum[i];
            occ = max(occ, wocc[i]);
        }
        if ((int)total >= K && occ <= TK_BIN_MAX) {  // the same decision in every thread
            const uint32_t st0 = before + incl - c0 - c1;
            if (b0 < nb) bcur[b0] = st0;
            if (b0 + 1 < nb) bcur[b0 + 1] = st0 + c0;
            __syncthreads();
            uint64_t* binned = cb + TK_SORT_MAX;
            for (int i = t; i < n; i += TK_THREADS) {
                const uint64_t e = cb[i];
                const uint32_t kk = tk_pkey(e);
                if (kk >= tmax) binned[atomicAdd(&bcur[tk_cbin(kk, kmax, sh, nb)], 1u)] = e;
            }
            __syncthreads();
            // bcur[b] is now the end of bin b
            for (int i = t; i < (int)total; i += TK_THREADS) {
                const uint64_t e = binned[i];
                const int b = tk_cbin(tk_pkey(e), kmax, sh, nb);
                const int end = (int)bcur[b], beg = end - (int)bcnt[b];
                if (beg >= K) continue;
                int r = beg;
                for (int j = beg; j < end; ++j) r += binned[j] > e ? 1 : 0;
                if (r < K) {
                    ids[(size_t)row * K + r] = tk_pid(e);
                    lp[(size_t)row * K + r] = key_value(tk_pkey(e)) - lse;
                }
            }
            return;
        }
    }
    for (int pass = 0; pass < 2; ++pass) {
        tk_sort_any(n, cb);
        const uint32_t T = tk_pkey(cb[K - 1]);
        bool again = false;
        for (int c = 0; c < C; ++c) again |= ptc[c] > T;
        if (!again) break;
        // chunks cut above T: their entries in [T, t_c) join the candidates, and the union is sorted again
        // (once: the K-th key can only rise, and every chunk then holds all of its entries >= T)
        if (t == 0) s_n = n;
        __syncthreads();
        for (int c = 0; c < C; ++c) {
            if (ptc[c] <= T) continue;
            const int j0 = c * CL, nc = min(V - j0, CL);
            for (int j = t; j < nc; j += TK_THREADS) {
                const uint32_t kk = order_key(x[j0 + j]);
                if (kk >= T && kk < ptc[c]) {
                    const int sl = atomicAdd(&s_n, 1);
                    if (sl < TK_SORT_MAX)
                        cb[sl] = tk_pack(kk, j0 + j);
                    else
                        s_ovf = 1;
                }
            }
        }
        __syncthreads();
        if (s_ovf) {
            fallback = true;
            break;
        }
        n = s_n;
    }
    }
    if (fallback) {
        tk_row(x, V, K, ids + (size_t)row * K, lp + (size_t)row * K);
        return;
    }
    for (int i = t; i < K; i += TK_THREADS) {
        const uint64_t p = cb[i];
        ids[(size_t)row * K + i] = tk_pid(p);
        lp[(size_t)row * K + i] = key_value(tk_pkey(p)) - lse;
    }
}

// Split of each row: C chunks of CL entries (a multiple of 4), kt the share each chunk keeps, capc the
// candidate slots per chunk.  C = 1: one workgroup per row.
struct TkSplit {
    int C, CL, kt, capc;
};
static TkSplit topk_split(int rows, int V, int K) {
    TkSplit sp{1, V, K, 0};
    int C = (256 + rows - 1) / rows;  // about one workgroup per compute unit
    if (C < 2) return sp;              // enough rows to fill the chip one workgroup each
    C = std::max(C, (V + TK_PER * TK_THREADS - 1) / (TK_PER * TK_THREADS));  // chunks fit in registers
    C = std::min(C, 32);
    const int CL = (((V + C - 1) / C) + 3) & ~3;
    if (CL > TK_PER * TK_THREADS) return sp;
    C = (V + CL - 1) / CL;  // no empty chunk
    if (C < 2) return sp;
    const int kt = std::min(CL, (3 * K + 2 * C - 1) / (2 * C) + 8);
    sp.C = C;
    sp.CL = CL;
    sp.kt = kt;
    sp.capc = std::min(CL, 2 * kt + 32);
    return sp;
}

size_t topk_workspace_bytes(int rows, int V, int K) {
    const TkSplit sp = topk_split(rows, V, K);
    if (sp.C < 2) return 0;
    return (size_t)rows * sp.C * (sizeof(float4) + (size_t)sp.capc * sizeof(uint2));
}

hipError_t launch_topk_rows(int rows, const float* logits, int64_t stride, int V, int K, int32_t* ids, float* lp,
                            void* ws, hipStream_t st) {
    const TkSplit sp = topk_split(rows, V, K);
    if (sp.C < 2) {
        hipLaunchKernelGGL(topk_rows, dim3(rows), dim3(TK_THREADS), 0, st, logits, stride, V, K, ids, lp);
        return hipGetLastError();
    }
    float4* part = (float4*)ws;
    uint2* cand = (uint2*)(part + (size_t)rows * sp.C);
    hipLaunchKernelGGL(topk_chunk, dim3(rows * sp.C), dim3(TK_THREADS), 0, st, logits, stride, V, sp.C, sp.CL, sp.kt,
                       sp.capc, cand, part);
    hipLaunchKernelGGL(topk_merge, dim3(rows), dim3(TK_THREADS), 0, st, logits, stride, V, K, sp.C, sp.CL, sp.capc,
                       cand, part, ids, lp);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// best-first tree construction (Algorithm 1), one wave per request
// ------------------------------------------------------------------------------------------------------
// The heap is a pool of candidate slots in LDS; slot i belongs to lane i % 64, and each lane caches the best
// of its own live slots as one 64-bit key (order key of the score, then the inverted slot index, so that
// equal scores pop in creation order).  A pop is a wave-wide max over the cached keys; the popped slot's
// owner gets its new best from a wave-wide max over its remaining slots (one slot per lane).  The popped rank
// tuple becomes node n; its next sibling (same parent, next rank; score = parent score + that rank's
// log-probability) and its first child (rank 1 at the next depth; score = its own + that log-probability) are
// appended as new slots.  The per-depth log-probabilities sit in LDS.
#define DT_POOL 4096
#define DT_MAXD 16

__device__ __forceinline__ uint64_t dt_key(float s, int slot) {
    return ((uint64_t)order_key(s) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)slot);
}
// Wave-wide max of a 64-bit key with DPP row operations (quad swaps, half-row and row mirrors, then the
// row broadcasts of lanes 15 and 31), which leave the maximum in lane 63; it is then read into every lane.
// All 64 lanes must be active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dt_dpp_max(uint64_t k) {
    const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
    const uint32_t ylo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xF, false);
    const uint32_t yhi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xF, false);
    const uint64_t y = ((uint64_t)yhi << 32) | ylo;
    return y > k ? y : k;
}
__device__ __forceinline__ uint64_t dt_wave_max(uint64_t k) {
    k = dt_dpp_max<0xB1, 0xF>(k);   // quad_perm [1, 0, 3, 2]
    k = dt_dpp_max<0x4E, 0xF>(k);   // quad_perm [2, 3, 0, 1]
    k = dt_dpp_max<0x141, 0xF>(k);  // row_half_mirror
    k = dt_dpp_max<0x140, 0xF>(k);  // row_mirror
    k = dt_dpp_max<0x142, 0xA>(k);  // row_bcast:15 into rows 1 and 3
    k = dt_dpp_max<0x143, 0xC>(k);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 63), hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Slot record in LDS (16 bytes, one read per pop): the 64-bit key, the packed (parent + 1, depth, rank)
// and the parent's score.
struct DtSlot {
    uint32_t key_lo, key_hi, meta, psig;
};
__device__ __forceinline__ uint32_t dt_meta(int parent, int depth, int rank) {
    return ((uint32_t)(parent + 1) << 16) | ((uint32_t)depth << 11) | (uint32_t)rank;
}

// With `only_undecided`, a request whose n_nodes entry is not -1 was already built by ddtree_select and is
// left alone.
__global__ __launch_bounds__(64) void ddtree_build(int D, int K, const float* __restrict__ lp,
                                                   const int32_t* __restrict__ ids, int64_t req_stride, int budget,
                                                   int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
                                                   int32_t* __restrict__ node_depth, float* __restrict__ node_logq,
                                                   int32_t* __restrict__ n_nodes, int only_undecided) {
    __shared__ DtSlot slot[DT_POOL];                 // key 0: popped (or never written)
    __shared__ uint2 nrec[DT_POOL / 2];              // popped nodes: (meta, score bits)
    __shared__ float slq[DT_MAXD * TK_MAX];
    const int r = blockIdx.x, lane = threadIdx.x;
    if (only_undecided && n_nodes[r] != -1) return;
    const float* l = lp + (size_t)r * req_stride;
    const int32_t* idr = ids + (size_t)r * req_stride;
    // the log-probabilities into LDS, sixteen independent loads in flight per lane
    for (int i0 = 0; i0 < D * K; i0 += 64 * 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = i0 + u * 64 + lane;
            v[u] = i < D * K ? l[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = i0 + u * 64 + lane;
            if (i < D * K) slq[(i / K) * TK_MAX + i % K] = v[u];
        }
    }
    const float lqf = lane < D ? l[(size_t)lane * K] : 0.f;  // lane d: best log-prob at depth d + 1
    if (lane == 0) {
        const uint64_t k0 = dt_key(l[0], 0);
        slot[0] = DtSlot{(uint32_t)k0, (uint32_t)(k0 >> 32), dt_meta(-1, 1, 0), __float_as_uint(0.f)};
    }
    __syncthreads();
    uint64_t best = lane == 0 ? dt_key(slq[0], 0) : 0ull;  // 0: no live slot
    int next = 1;
    int n = 0;
    for (; n < budget; ++n) {
        const uint64_t top = dt_wave_max(best);
        if (top == 0ull) break;  // every prefix of the rank space is already in the tree
        const int sl = (int)(0xFFFFFFFFu - (uint32_t)top);
        const DtSlot rec = slot[sl];
        const float s = key_value((uint32_t)(top >> 32));
        const int p = (int)(rec.meta >> 16) - 1, d = (rec.meta >> 11) & 31, k = rec.meta & 2047;
        const float ps = __uint_as_float(rec.psig);
        // independent LDS reads: the owner's other slots (one per lane) and the next sibling's log-prob
        const int owner = sl & 63;
        const int q = owner + 64 * lane;
        const DtSlot c = q < next ? slot[q] : DtSlot{0u, 0u, 0u, 0u};
        const float lq_sib = k + 1 < K ? slq[(d - 1) * TK_MAX + k + 1] : 0.f;
        const float lq_child = __shfl(lqf, d < D ? d : 0, 64);
        if (lane == 0) nrec[n] = make_uint2(rec.meta, __float_as_uint(s));
        uint64_t cand = (q != sl) ? (((uint64_t)c.key_hi << 32) | c.key_lo) : 0ull;
        cand = dt_wave_max(cand);
        if (lane == owner) best = cand;
        if (lane == 0) {
            slot[sl].key_lo = 0u;
            slot[sl].key_hi = 0u;
        }
        if (k + 1 < K) {  // next sibling: same parent, next rank
            const float ss = ps + lq_sib;
            if (lane == (next & 63)) {
                const uint64_t kk = dt_key(ss, next);
                slot[next] = DtSlot{(uint32_t)kk, (uint32_t)(kk >> 32), dt_meta(p, d, k + 1), rec.psig};
                best = kk > best ? kk : best;
            }
            ++next;
        }
        if (d < D) {  // first child: best token at the next depth
            const float cs = s + lq_child;
            if (lane == (next & 63)) {
                const uint64_t kk = dt_key(cs, next);
                slot[next] = DtSlot{(uint32_t)kk, (uint32_t)(kk >> 32), dt_meta(n, d + 1, 0), __float_as_uint(s)};
                best = kk > best ? kk : best;
            }
            ++next;
        }
        __syncthreads();  // this pop's LDS writes before the next pop reads them
    }
    int32_t* out_tok = node_token + (size_t)r * budget;
    int32_t* out_par = node_parent + (size_t)r * budget;
    int32_t* out_dep = node_depth + (size_t)r * budget;
    float* out_lq = node_logq + (size_t)r * budget;
    for (int i = lane; i < n; i += 64) {
        const uint2 e = nrec[i];
        const int di = (e.x >> 11) & 31, ki = e.x & 2047;
        out_tok[i] = idr[(size_t)(di - 1) * K + ki];
        out_par[i] = (int)(e.x >> 16) - 1;
        out_dep[i] = di;
        out_lq[i] = __uint_as_float(e.y);
    }
    if (lane == 0) n_nodes[r] = n;
}

// ------------------------------------------------------------------------------------------------------
// the same tree by parallel selection, one 1024-thread workgroup per request
// ------------------------------------------------------------------------------------------------------
// Scores are float32 path sums (parent score + own log-probability), so along every edge of Algorithm 1's
// generation order (a tuple -> its next sibling, a tuple -> its first child) the score never rises when the
// log-probabilities are <= 0 and each depth's row is non-increasing.  The pops therefore come out in
// non-increasing score order, equal scores in creation order, and the first B pops are the B best tuples
// under that order (Proposition 2 of §3.4.3).  The kernel finds them without the heap:
//   1. a pool in LDS holds every tuple whose score key is >= a threshold tau, which only rises and always
//      stays at or below the B-th best score, level by level: the children of depth d's pool entries with
//      scores >= tau are a rank prefix of each parent (a binary search over the sorted row), appended in
//      parent order;
//   2. when the pool would overflow, tau is raised to the lower edge of the histogram bin that holds the B-th
//      best key in the pool (refined inside that bin up to three times) and everything below is dropped;
//      a child never scores above its parent, so the pool stays prefix-closed;
//   3. the pool is sorted by score (bitonic, in LDS), runs of equal scores are put in creation order by
//      comparing their generators (the previous sibling, or the parent for a first child; one generator's
//      sibling is created before its child), and the first B entries are the tree.
// A request it cannot decide -- rows that are not sorted log-probabilities, runs of more than DS_RUN_MAX
// equal scores, a tie chain longer than DS_WALK_MAX, a pool that no threshold can thin -- gets
// n_nodes = -1; ddtree_build then runs the heap on it.
#define DS_THREADS 1024
#define DS_CAP 4096
#define DS_NB 2048
#define DS_RUN_MAX 32
#define DS_WALK_MAX 256
#define DS_MAX_RAISES 64

struct DsLds {
    float lq[DT_MAXD * TK_MAX];  // row d at d * K
    uint32_t key[DS_CAP];        // order key of the score
    uint32_t meta[DS_CAP];       // (parent + 1) << 15 | depth << 10 | rank; parent = pool index, -1 at depth 1
    union {
        struct {
            uint32_t rc[DS_CAP];   // per parent of the level being built: next rank << 16 | end rank
            uint32_t off[DS_CAP];  // exclusive prefix of the ranks still to append
        } lv;
        uint64_t sk[DS_CAP];  // sort keys: score key << 32 | 0xFFFF - pool index
    } u;
    uint16_t idx[DS_CAP];  // compaction targets, then output positions
    uint32_t hist[DS_NB];
    uint32_t red[2 * (DS_THREADS / 64)];
    int flag, bstar;
    uint32_t above, inbin;
};

__device__ __forceinline__ uint32_t ds_meta(int p, int d, int r) {
    return ((uint32_t)(p + 1) << 15) | ((uint32_t)d << 10) | (uint32_t)r;
}
__device__ __forceinline__ int ds_par(uint32_t m) { return (int)(m >> 15) - 1; }
__device__ __forceinline__ int ds_dep(uint32_t m) { return (int)((m >> 10) & 31u); }
__device__ __forceinline__ int ds_rank(uint32_t m) { return (int)(m & 1023u); }
__device__ __forceinline__ int ds_slot(uint64_t k) { return 0xFFFF - (int)(k & 0xFFFFu); }

// Score key of the tuple (pool parent p, depth d, rank r): the parent's score + the log-probability.
__device__ __forceinline__ uint32_t ds_score(const DsLds& s, int K, int p, int d, int r) {
    const float sp = p < 0 ? 0.f : key_value(s.key[p]);
    return order_key(sp + s.lq[(d - 1) * K + r]);
}

// Block-wide exclusive prefix sum (all threads call it); `total` gets the sum over the block.
__device__ __forceinline__ uint32_t ds_scan(uint32_t v, uint32_t* red, uint32_t& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[w] = x;
    __syncthreads();
    uint32_t base = 0u, tot = 0u;
#pragma unroll
    for (int i = 0; i < DS_THREADS / 64; ++i) {
        const uint32_t q = red[i];
        base += i < w ? q : 0u;
        tot += q;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

__device__ __forceinline__ void ds_minmax(uint32_t& mn, uint32_t& mx, uint32_t* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    }
    if (lane == 0) {
        red[w] = mn;
        red[DS_THREADS / 64 + w] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DS_THREADS / 64; ++i) {
        mn = min(mn, red[i]);
        mx = max(mx, red[DS_THREADS / 64 + i]);
    }
    __syncthreads();
}

// First rank in [lo, hi) of depth-(d + 1) row whose score under a parent of score sp falls below tau (the
// scores fall with the rank); hi when none does.
__device__ __forceinline__ int ds_count(const DsLds& s, int K, float sp, int d, int lo, int hi, uint32_t tau) {
    const float* row = s.lq + d * K;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (order_key(sp + row[mid]) >= tau)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// A threshold >= tau that keeps at least `budget` of the N > budget pool entries: the lower edge of the
// histogram bin holding the budget-th best key, the bin refined by further histograms while it holds many.
__device__ uint32_t ds_raise(DsLds& s, int N, int budget, uint32_t tau) {
    const int t = threadIdx.x;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int e = t; e < N; e += DS_THREADS) {
        const uint32_t k = s.key[e];
        lo = min(lo, k);
        hi = max(hi, k);
    }
    ds_minmax(lo, hi, s.red);
    uint32_t need = (uint32_t)budget, v = lo;  // `need` of the keys in [lo, hi] are still to be kept
    for (int round = 0; round < 3 && hi > lo; ++round) {
        const uint32_t span = hi - lo;
        const int sh = max(0, 32 - __clz((int)span) - 11);  // (k - lo) >> sh < DS_NB
        for (int b = t; b < DS_NB; b += DS_THREADS) s.hist[b] = 0u;
        __syncthreads();
        for (int e = t; e < N; e += DS_THREADS) {
            const uint32_t k = s.key[e];
            if (k >= lo && k <= hi) atomicAdd(&s.hist[(k - lo) >> sh], 1u);
        }
        __syncthreads();
        const int b0 = DS_NB - 1 - 2 * t;  // two bins per thread, from the top
        const uint32_t h0 = s.hist[b0], h1 = s.hist[b0 - 1];
        uint32_t tot;
        const uint32_t above = ds_scan(h0 + h1, s.red, tot);
        if (above < need && above + h0 >= need) {
            s.bstar = b0;
            s.above = above;
            s.inbin = h0;
        } else if (above + h0 < need && above + h0 + h1 >= need) {
            s.bstar = b0 - 1;
            s.above = above + h0;
            s.inbin = h1;
        }
        __syncthreads();
        const uint32_t bs = (uint32_t)s.bstar, ab = s.above, ib = s.inbin;
        __syncthreads();
        v = lo + (bs << sh);
        if (sh == 0 || ab + ib <= need + DS_CAP / 32) break;
        need -= ab;  // refine inside the bin
        lo = v;
        hi = min(hi, v + ((1u << sh) - 1u));
    }
    return v > tau ? v : tau;
}

// Drops the pool entries below tau, keeping the order; the parents [ps, pe) of the level being built carry
// their rank state along when `parents`.
__device__ void ds_compact(DsLds& s, int& N, uint32_t tau, int& ps, int& pe, bool parents) {
    const int t = threadIdx.x, e0 = 4 * t;
    uint32_t k4[4], m4[4], rc4[4];
    bool keep[4];
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = e0 + u;
        k4[u] = e < N ? s.key[e] : 0u;
        keep[u] = e < N && k4[u] >= tau;
        m4[u] = keep[u] ? s.meta[e] : 0u;
        rc4[u] = (parents && keep[u] && e >= ps && e < pe) ? s.u.lv.rc[e - ps] : 0u;
        cnt += keep[u] ? 1u : 0u;
    }
    uint32_t nn;
    uint32_t o = ds_scan(cnt, s.red, nn);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (e0 + u < N) s.idx[e0 + u] = (uint16_t)o;
        o += keep[u] ? 1u : 0u;
    }
    __syncthreads();
    const int nps = ps < N ? (int)s.idx[ps] : (int)nn, npe = pe < N ? (int)s.idx[pe] : (int)nn;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (!keep[u]) continue;
        const int e = e0 + u, dst = s.idx[e], p = ds_par(m4[u]);
        s.key[dst] = k4[u];
        s.meta[dst] = p < 0 ? m4[u] : ds_meta(s.idx[p], ds_dep(m4[u]), ds_rank(m4[u]));
        if (parents && e >= ps && e < pe) s.u.lv.rc[dst - nps] = rc4[u];
    }
    __syncthreads();
    N = (int)nn;
    ps = nps;
    pe = npe;
}

// Whether the pool entry x was created before the pool entry y, both of equal score: a tuple is created
// when its generator pops (the previous sibling, or the parent for a first child), so the order is that of
// the generators -- by score, then recursively -- and one generator's sibling comes before its child.  The
// first depth-1 tuple is created before everything.
__device__ bool ds_before(const DsLds& s, int K, int xi, int yi, int* flag) {
    const uint32_t mx = s.meta[xi], my = s.meta[yi];
    int xp = ds_par(mx), xd = ds_dep(mx), xr = ds_rank(mx);
    int yp = ds_par(my), yd = ds_dep(my), yr = ds_rank(my);
    for (int step = 0; step < DS_WALK_MAX; ++step) {
        if (xd == 1 && xr == 0) return true;
        if (yd == 1 && yr == 0) return false;
        int gxp, gxd = xd, gxr, gyp, gyd = yd, gyr;
        const int tx = xr > 0 ? 0 : 1, ty = yr > 0 ? 0 : 1;  // 0: sibling, 1: first child
        if (tx == 0) {
            gxp = xp;
            gxr = xr - 1;
        } else {
            const uint32_t m = s.meta[xp];
            gxp = ds_par(m);
            gxd = xd - 1;
            gxr = ds_rank(m);
        }
        if (ty == 0) {
            gyp = yp;
            gyr = yr - 1;
        } else {
            const uint32_t m = s.meta[yp];
            gyp = ds_par(m);
            gyd = yd - 1;
            gyr = ds_rank(m);
        }
        if (gxp == gyp && gxd == gyd && gxr == gyr) return tx < ty;
        const uint32_t sx = ds_score(s, K, gxp, gxd, gxr), sy = ds_score(s, K, gyp, gyd, gyr);
        if (sx != sy) return sx > sy;
        xp = gxp, xd = gxd, xr = gxr;
        yp = gyp, yd = gyd, yr = gyr;
    }
    *flag = 1;
    return false;
}

__global__ __launch_bounds__(DS_THREADS) void ddtree_select(int D, int K, const float* __restrict__ lp,
                                                             const int32_t* __restrict__ ids, int64_t req_stride,
                                                             int budget, int32_t* __restrict__ node_token,
                                                             int32_t* __restrict__ node_parent,
                                                             int32_t* __restrict__ node_depth,
                                                             float* __restrict__ node_logq,
                                                             int32_t* __restrict__ n_nodes) {
    __shared__ DsLds s;
    const int r = blockIdx.x, t = threadIdx.x;
    const float* l = lp + (size_t)r * req_stride;
    const int DK = D * K;
    for (int i0 = 0; i0 < DK; i0 += DS_THREADS * 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = i0 + u * DS_THREADS + t;
            v[u] = i < DK ? l[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = i0 + u * DS_THREADS + t;
            if (i < DK) s.lq[i] = v[u];
        }
    }
    if (t == 0) s.flag = 0;
    __syncthreads();
    // the method's input: every row sorted, non-increasing log-probabilities (no NaN, nothing above 0)
    for (int i = t; i < DK; i += DS_THREADS) {
        const float x = s.lq[i];
        if (!(x <= 0.f) || ((i % K) + 1 < K && !(s.lq[i + 1] <= x))) s.flag = 1;
    }
    __syncthreads();
    bool fail = s.flag != 0;
    int N = 0, ps = 0, pe = 0, raises = 0;
    uint32_t tau = 0u;  // no threshold yet: every key is >= 0
    for (int d = 0; d < D && !fail; ++d) {
        // build depth d + 1 from the pool entries [ps, pe) of depth d (the root when d = 0)
        const int lim = min(K, budget - d);  // a rank-r child has r elder siblings and d ancestors before it
        if (lim <= 0) break;
        if (d > 0 && N > budget + DS_CAP / 8) {
            tau = ds_raise(s, N, budget, tau);
            ds_compact(s, N, tau, ps, pe, false);
        }
        int P = d == 0 ? 1 : pe - ps;
        if (P == 0) break;
        for (int i = t; i < P; i += DS_THREADS) {
            const float sp = d == 0 ? 0.f : key_value(s.key[ps + i]);
            s.u.lv.rc[i] = (uint32_t)ds_count(s, K, sp, d, 0, lim, tau);
        }
        __syncthreads();
        while (true) {
            uint32_t n4[4], loc = 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = 4 * t + u;
                const uint32_t rc = i < P ? s.u.lv.rc[i] : 0u;
                n4[u] = (rc & 0xFFFFu) - (rc >> 16);
                loc += n4[u];
            }
            uint32_t T;
            uint32_t o = ds_scan(loc, s.red, T);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (4 * t + u < P) s.u.lv.off[4 * t + u] = o;
                o += n4[u];
            }
            const int room = DS_CAP - N;
            const int E = min((int)T, room);
            __syncthreads();
            for (int j = t; j < E; j += DS_THREADS) {
                int lo = 0, hi = P;  // the last parent whose offset is <= j
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int)s.u.lv.off[mid] <= j)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                const int i = lo - 1;
                const int rank = (int)(s.u.lv.rc[i] >> 16) + (j - (int)s.u.lv.off[i]);
                const int p = d == 0 ? -1 : ps + i;
                s.key[N + j] = ds_score(s, K, p, d + 1, rank);
                s.meta[N + j] = ds_meta(p, d + 1, rank);
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = 4 * t + u;
                if (i < P && n4[u] > 0u) {
                    const uint32_t rc = s.u.lv.rc[i];
                    const int took = min((int)n4[u], max(0, E - (int)s.u.lv.off[i]));
                    s.u.lv.rc[i] = rc + ((uint32_t)took << 16);
                }
            }
            N += E;
            __syncthreads();
            if ((int)T <= room) break;
            // the pool is full: raise the threshold, drop what falls below, recount what is left to append
            if (++raises > DS_MAX_RAISES) {
                fail = true;
                break;
            }
            tau = ds_raise(s, N, budget, tau);
            ds_compact(s, N, tau, ps, pe, d > 0);
            if (DS_CAP - N < DS_CAP / 16) {
                fail = true;
                break;
            }
            P = d == 0 ? 1 : pe - ps;
            for (int i = t; i < P; i += DS_THREADS) {
                const uint32_t rc = s.u.lv.rc[i];
                const float sp = d == 0 ? 0.f : key_value(s.key[ps + i]);
                const int c = ds_count(s, K, sp, d, (int)(rc >> 16), (int)(rc & 0xFFFFu), tau);
                s.u.lv.rc[i] = (rc & 0xFFFF0000u) | (uint32_t)c;
            }
            __syncthreads();
        }
        ps = pe;
        pe = N;
    }
    if (!fail && N > budget) {
        tau = ds_raise(s, N, budget, tau);
        ds_compact(s, N, tau, ps, pe, false);
    }
    const int nout = min(N, budget);
    if (!fail) {
        // sort by score, best first; the low half only makes the keys distinct
        int S = 64;
        while (S < N) S <<= 1;
        for (int i = t; i < S; i += DS_THREADS)
            s.u.sk[i] = i < N ? (((uint64_t)s.key[i] << 32) | (uint64_t)(0xFFFFu - (uint32_t)i)) : 0ull;
        __syncthreads();
        for (int k = 2; k <= S; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = t; i < S / 2; i += DS_THREADS) {
                    const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1)), b = a + j;
                    const uint64_t ka = s.u.sk[a], kb = s.u.sk[b];
                    if (((a & k) == 0) ? ka < kb : ka > kb) {
                        s.u.sk[a] = kb;
                        s.u.sk[b] = ka;
                    }
                }
                __syncthreads();
            }
        }
        // runs of equal scores that reach into the first `budget` positions: creation order
        for (int j = t; j < nout; j += DS_THREADS) {
            const uint32_t h = (uint32_t)(s.u.sk[j] >> 32);
            if (j + 1 >= N || (uint32_t)(s.u.sk[j + 1] >> 32) != h) continue;
            if (j > 0 && (uint32_t)(s.u.sk[j - 1] >> 32) == h) continue;
            int e = j + 1;
            while (e < N && e - j <= DS_RUN_MAX && (uint32_t)(s.u.sk[e] >> 32) == h) ++e;
            if (e - j > DS_RUN_MAX) {
                s.flag = 1;
                continue;
            }
            for (int a = j + 1; a < e; ++a) {
                const uint64_t x = s.u.sk[a];
                int b = a;
                while (b > j && ds_before(s, K, ds_slot(x), ds_slot(s.u.sk[b - 1]), &s.flag)) {
                    s.u.sk[b] = s.u.sk[b - 1];
                    --b;
                }
                s.u.sk[b] = x;
            }
        }
        for (int i = t; i < N; i += DS_THREADS) s.idx[i] = 0xFFFFu;
        __syncthreads();
        for (int j = t; j < nout; j += DS_THREADS) s.idx[ds_slot(s.u.sk[j])] = (uint16_t)j;
        __syncthreads();
        int32_t* out_tok = node_token + (size_t)r * budget;
        int32_t* out_par = node_parent + (size_t)r * budget;
        int32_t* out_dep = node_depth + (size_t)r * budget;
        float* out_lq = node_logq + (size_t)r * budget;
        const int32_t* idr = ids + (size_t)r * req_stride;
        for (int j = t; j < nout; j += DS_THREADS) {
            const uint64_t k = s.u.sk[j];
            const uint32_t m = s.meta[ds_slot(k)];
            const int p = ds_par(m), dd = ds_dep(m), rk = ds_rank(m);
            int pj = -1;
            if (p >= 0) {
                pj = (int)s.idx[p];
                if (pj >= j) s.flag = 1;  // never: a parent scores and is created before its children
            }
            out_tok[j] = idr[(size_t)(dd - 1) * K + rk];
            out_par[j] = pj;
            out_dep[j] = dd;
            out_lq[j] = key_value((uint32_t)(k >> 32));
        }
        __syncthreads();
        fail = s.flag != 0;
    }
    if (t == 0) n_nodes[r] = fail ? -1 : nout;
}

// Below this budget the heap's few pops take less time than the selection's fixed cost of one
// synchronised round per depth (measured: 12.8 vs 22.5 us at 16 nodes, 42.5 vs 20.6 us at 64).
#define DS_MIN_BUDGET 28

hipError_t launch_ddtree_build(int batch, int D, int K, const float* lp, const int32_t* ids, int64_t req_stride,
                               int budget, int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                               float* node_logq, int32_t* n_nodes, bool select_only, hipStream_t st) {
    if (!select_only && budget < DS_MIN_BUDGET) {
        hipLaunchKernelGGL(ddtree_build, dim3(batch), dim3(64), 0, st, D, K, lp, ids, req_stride, budget, node_token,
                           node_parent, node_depth, node_logq, n_nodes, 0);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(ddtree_select, dim3(batch), dim3(DS_THREADS), 0, st, D, K, lp, ids, req_stride, budget,
                       node_token, node_parent, node_depth, node_logq, n_nodes);
    if (select_only) return hipGetLastError();
    hipLaunchKernelGGL(ddtree_build, dim3(batch), dim3(64), 0, st, D, K, lp, ids, req_stride, budget, node_token,
                       node_parent, node_depth, node_logq, n_nodes, 1);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------------
// greedy verifier walk, one wave per request
// ------------------------------------------------------------------------------------------------------
// From the root: the target's choice after the current prefix (target_next[0] after the root, [i + 1]
// after node i) is looked up among the current node's children (a wave-wide scan of the parent links); the
// walk moves there or stops, and the stopping choice is the next bonus token.
__global__ __launch_bounds__(64) void ddtree_walk(int budget, int max_accept, const int32_t* __restrict__ node_token,
                                                  const int32_t* __restrict__ node_parent,
                                                  const int32_t* __restrict__ n_nodes,
                                                  const int32_t* __restrict__ target_next,
                                                  int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
                                                  int32_t* __restrict__ bonus) {
    const int r = blockIdx.x, lane = threadIdx.x;
    const int n = min(n_nodes[r], budget);
    const int32_t* tok = node_token + (size_t)r * budget;
    const int32_t* par = node_parent + (size_t)r * budget;
    const int32_t* tgt = target_next + (size_t)r * (budget + 1);
    int cur = -1, len = 0, y = 0;
    while (true) {
        y = tgt[cur + 1];
        int found = 0x7FFFFFFF;
        for (int i = lane; i < n; i += 64)
            if (par[i] == cur && tok[i] == y) found = min(found, i);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) found = min(found, __shfl_xor(found, o, 64));
        if (found == 0x7FFFFFFF || len >= max_accept) break;
        if (lane == 0) accept_nodes[(size_t)r * max_accept + len] = found;
        ++len;
        cur = found;
    }
    if (lane == 0) {
        accept_len[r] = len;
        bonus[r] = y;
    }
}

hipError_t launch_ddtree_walk(int batch, int budget, int max_accept, const int32_t* node_token,
                              const int32_t* node_parent, const int32_t* n_nodes, const int32_t* target_next,
                              int32_t* accept_len, int32_t* accept_nodes, int32_t* bonus, hipStream_t st) {
    hipLaunchKernelGGL(ddtree_walk, dim3(batch), dim3(64), 0, st, budget, max_accept, node_token, node_parent,
                       n_nodes, target_next, accept_len, accept_nodes, bonus);
    return hipGetLastError();
}

}  // namespace df
