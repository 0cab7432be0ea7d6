// Shared device helpers for the gfx950 kernels: bfloat16 conversion, MFMA operand types, wave reductions,
// and the launch-parameter structs the host layer fills.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dflash.h"

#define DF_WAVE 64

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- number formats --------------------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (NaN stays NaN): one v_cvt_pk_bf16_f32 on gfx950,
// which gives the same bits as the integer formula (u + 0x7FFF + ((u >> 16) & 1)) >> 16 for every non-NaN
// input (all 2^32 patterns compared on MI355X).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two conversions in one instruction: low half = bf16(lo), high half = bf16(hi).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Storage type of weights and cached values: bfloat16 bits or float32.
template <typename T> struct Act;
template <> struct Act<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
    static __device__ __forceinline__ bf16_t from(float f) { return f2bf(f); }
};
template <> struct Act<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ float from(float f) { return f; }
};

// Transient activations of a bfloat16 drafter are kept at float32 precision as two bfloat16 planes,
// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi) (relative error <= 2^-17), so that they can enter the
// bfloat16 MFMAs exactly enough: a product with hi + lo costs two MFMAs.  `plane` is the element distance
// from the hi plane to the lo plane.  Float32 drafters store the value itself (plane unused).
__device__ __forceinline__ void put_act(bf16_t* p, size_t plane, size_t i, float v) {
    const bf16_t h = f2bf(v);
    p[i] = h;
    p[i + plane] = f2bf(v - bf2f(h));
}
__device__ __forceinline__ void put_act(float* p, size_t, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ float get_act(const bf16_t* p, size_t plane, size_t i) {
    return bf2f(p[i]) + bf2f(p[i + plane]);
}
__device__ __forceinline__ float get_act(const float* p, size_t, size_t i) { return p[i]; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes = eight bfloat16 MFMA operands
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte loads: plain (cached) and non-temporal (weights streamed once; kept out of the caches' LRU).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }

// D += A * B on one 16x16x32 bfloat16 MFMA.  Lane l supplies A row (l % 16) and B column (l % 16), eight
// k-values each; D lane l holds rows 4*(l/16) + i, column l % 16 (i = 0..3).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---- reductions ------------------------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, DF_WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, DF_WAVE));
    return v;
}

// Block-wide sum in a fixed order (deterministic).  `red` needs blockDim.x / 64 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t flag) {
    if (err) atomicOr(err, flag);
}

// ---- GEMM operand description ----------------------------------------------------------------------------

// The output columns of one GEMM may come from up to DF_MAX_SEG weight matrices stacked along N (e.g. wq,
// wk, wv).  Segment s covers columns [start[s], start[s+1]) and reads rows of ptr[s].  Every boundary is a
// multiple of 16.
#define DF_MAX_SEG 12
struct Segs {
    const void* ptr[DF_MAX_SEG];
    int start[DF_MAX_SEG + 1];
    int n;
};

__device__ __forceinline__ const void* seg_row(const Segs& s, int n, int K, int elt_bytes) {
    int i = 0;
#pragma unroll 1
    while (i + 1 < s.n && n >= s.start[i + 1]) ++i;
    return (const char*)s.ptr[i] + (size_t)(n - s.start[i]) * (size_t)K * elt_bytes;
}

// Rotary frequencies theta^(-2i/d) rounded to float32, computed on the host and passed by value.
struct RopeFreq {
    float inv[64];
    int on;
};

// ---- top-k state for the fused LM head -------------------------------------------------------------------

#define DF_TOPK 8

// (v, id) ranks above (w, jd): larger logit first, then smaller id.
__device__ __forceinline__ bool df_better(float v, int id, float w, int jd) {
    return v > w || (v == w && id < jd);
}

