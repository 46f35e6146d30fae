// Device-side helpers shared by the gfx950 kernels of libcad (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cad_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- bf16 storage (raw uint16 bit patterns) ----------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even (inputs are finite on this path)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Storage element abstraction: uint16_t = bf16 bits, float = fp32.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
    static __device__ __forceinline__ float rnd(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};
template <> struct Elt<float> {
    static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
    static __device__ __forceinline__ float rnd(float v) { return v; }
};

// four consecutive values -> four consecutive stored elements (8 bytes of bf16 / 16 of fp32)
__device__ __forceinline__ void st4(uint16_t* p, f32x4_t v) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *(uint2*)p = w;
}

// ---- wavefront reductions (64 lanes) ------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// (value, index) max with ties to the lowest index
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Per-sequence state captured by the first kernel of a forward: the cache length every
// later kernel of the same forward uses, and whether the sequence fits.
__device__ __forceinline__ bool seq_ok(const int32_t* len_snap, int b, int Nq, int cap) {
    return len_snap[b] >= 0 && len_snap[b] + Nq <= cap;
}
