// Output stages of the stacked projections: q/k/v with rotary embedding and the block's K / V^T layouts,
// and the SwiGLU gate.
#pragma once

#include "common.h"

// ---- rotary embedding and the q / block K / block V^T stores ----------------------------------------------
__device__ __forceinline__ void rope_pair_inv(float& a, float& b, int pos, float inv) {
    const float ang = (float)pos * inv;
    float sn, cs;
    sincosf(ang, &sn, &cs);
    const float x1 = a, x2 = b;
    a = x1 * cs - x2 * sn;
    b = x2 * cs + x1 * sn;
}
__device__ __forceinline__ void rope_pair(float& a, float& b, int pos, int i, const RopeFreq& rf) {
    if (rf.on) rope_pair_inv(a, b, pos, rf.inv[i]);
}

// Rotary pair i (head columns i and i + d/2) of stacked head hd (q heads, then k, then v) for block row m:
// rotation at position pos (= ctx_len[b] + row) with inverse frequency inv (rope: rotation on) for q and k; q
// stored row-major [m][nq][d], the block's keys as a 16-slot page [b][kv head][slot][d] and its values
// transposed [b][kv head][d][slot].
template <typename T>
__device__ __forceinline__ void qkv_store(float a, float c, int m, int hd, int i, int B, int L, int nq, int nkv,
                                          int d, int pos, bool rope, float inv, T* q, T* kb, T* vbt) {
    const int half = d >> 1;
    const int b = m / L, row = m % L;
    const size_t qplane = (size_t)B * L * nq * d, bplane = (size_t)B * nkv * 16 * d;
    if (hd < nq) {
        if (rope) rope_pair_inv(a, c, pos, inv);
        const size_t o = (size_t)m * nq * d + hd * d + i;
        put_act(q, qplane, o, a);
        put_act(q, qplane, o + half, c);
    } else if (hd < nq + nkv) {
        const int kh = hd - nq;
        if (rope) rope_pair_inv(a, c, pos, inv);
        const size_t o = (((size_t)b * nkv + kh) * 16 + row) * d + i;
        put_act(kb, bplane, o, a);
        put_act(kb, bplane, o + half, c);
    } else {
        const int kh = hd - nq - nkv;
        const size_t o = ((size_t)b * nkv + kh) * d * 16 + row;
        put_act(vbt, bplane, o + (size_t)i * 16, a);
        put_act(vbt, bplane, o + (size_t)(i + half) * 16, c);
    }
}

__device__ __forceinline__ float swiglu_value(float g, float up) { return g / (1.0f + expf(-g)) * up; }
