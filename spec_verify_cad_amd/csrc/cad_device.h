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

// runner-up of two (max, second) pairs: the larger of both seconds and of the smaller maximum
// (equal maxima make the runner-up equal to the maximum, a gap of zero)
__device__ __forceinline__ float second_merge(float b1, float s1, float b2, float s2) {
    return fmaxf(fmaxf(s1, s2), fminf(b1, b2));
}

// Per-sequence state captured by the first kernel of a forward: the cache length every
// later kernel of the same forward uses, and whether the sequence fits.
__device__ __forceinline__ bool seq_ok(const int32_t* len_snap, int b, int Nq, int cap) {
    return len_snap[b] >= 0 && len_snap[b] + Nq <= cap;
}

// ---- stochastic verification -------------------------------------------------------------
// Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies and word mixing, the key
// bumped by two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// (0, 1) uniform from 32 random bits: the top 23 bits k give (2k + 1) / 2^24 (exact in fp32)
__device__ __forceinline__ float uniform_from_bits(uint32_t w) {
    return (float)(2u * (w >> 9) + 1u) * (1.0f / 16777216.0f);
}

// Gumbel noise -log(-log(u)) with the accurate logarithm (u close to 1 needs it)
__device__ __forceinline__ float gumbel(uint32_t w) { return -logf(-logf(uniform_from_bits(w))); }

// Per-row state of a sampled LM head over a set of vocabulary ids: the Gumbel-perturbed
// maximum over all ids (y) and over the ids other than the row's draft (z), both with ties to
// the lowest id; the running log-sum-exp (m, s) of the tempered logits; the draft's tempered
// logit (-inf until seen).
struct SampleState {
    float yv, zv, m, s, dl;
    int yi, zi;
};

__device__ __forceinline__ void sample_init(SampleState& st) {
    st.yv = st.zv = st.m = st.dl = -INFINITY;
    st.s = 0.f;
    st.yi = st.zi = 0x7fffffff;
}

// one logit v of id n (tempered value sv = v * inv_temp, Gumbel noise g).  A state takes its
// ids in increasing order, so a strict comparison keeps the lowest id among equal values.  No
// branches: the log-sum-exp update uses the one weight exp(-|sv - m|), which is exp(m - sv) when
// sv raises the maximum (s = s * w + 1) and exp(sv - m) otherwise (s = s + w).
__device__ __forceinline__ void sample_add(SampleState& st, float sv, float g, int n, int draft) {
    const float pv = sv + g;
    const bool ty = pv > st.yv;
    st.yv = ty ? pv : st.yv;
    st.yi = ty ? n : st.yi;
    const bool nd = n != draft;
    const bool tz = nd && pv > st.zv;
    st.zv = tz ? pv : st.zv;
    st.zi = tz ? n : st.zi;
    st.dl = nd ? st.dl : sv;
    const float d = sv - st.m;
    const float w = __expf(-fabsf(d));
    const bool up = d > 0.f;
    st.s = up ? fmaf(st.s, w, 1.f) : st.s + w;
    st.m = up ? sv : st.m;
}

__device__ __forceinline__ void sample_merge(SampleState& a, const SampleState& b) {
    argmax_merge(a.yv, a.yi, b.yv, b.yi);
    argmax_merge(a.zv, a.zi, b.zv, b.zi);
    a.dl = fmaxf(a.dl, b.dl);
    if (b.m > a.m) {
        a.s = a.s * __expf(a.m - b.m) + b.s;
        a.m = b.m;
    } else if (b.m > -INFINITY) {
        a.s += b.s * __expf(b.m - a.m);
    }
}

__device__ __forceinline__ SampleState sample_shfl_xor(const SampleState& st, int o) {
    SampleState r;
    r.yv = __shfl_xor(st.yv, o, 64);
    r.zv = __shfl_xor(st.zv, o, 64);
    r.m = __shfl_xor(st.m, o, 64);
    r.s = __shfl_xor(st.s, o, 64);
    r.dl = __shfl_xor(st.dl, o, 64);
    r.yi = __shfl_xor(st.yi, o, 64);
    r.zi = __shfl_xor(st.zi, o, 64);
    return r;
}

// slot layout of a sampled LM head: two float4 per (row, slot)
__device__ __forceinline__ void sample_store(float4* slot, const SampleState& st) {
    slot[0] = make_float4(st.yv, __int_as_float(st.yi), st.zv, __int_as_float(st.zi));
    slot[1] = make_float4(st.m, st.s, st.dl, 0.f);
}
__device__ __forceinline__ SampleState sample_load(const float4* slot) {
    const float4 a = slot[0], b = slot[1];
    SampleState st;
    st.yv = a.x; st.yi = __float_as_int(a.y); st.zv = a.z; st.zi = __float_as_int(a.w);
    st.m = b.x; st.s = b.y; st.dl = b.z;
    return st;
}

// The row's draft token and its Philox key words for a sampled LM head: row tok of sequence
// b = tok / Nq at position len_snap[b] + it holds a draft when it < draft_len[b] (clamped to
// Nq - 1): the next row's input token.
// In copy-commit mode (row_pos_last) row tok is sequence tok's last row and holds no draft.
struct SampleRow { int b, pos, draft; };
__device__ __forceinline__ SampleRow sample_row(const EpiParams& p, int tok) {
    SampleRow r;
    const int it = p.row_pos_last ? p.Nq - 1 : tok % p.Nq;
    r.b = p.row_pos_last ? tok : tok / p.Nq;
    r.pos = p.len_snap[r.b] + it;
    r.draft = -1;
    if (p.draft_len && !p.row_pos_last) {
        int dl = p.draft_len[r.b];
        dl = dl < p.Nq - 1 ? dl : p.Nq - 1;
        if (it < dl) r.draft = p.tokens[(size_t)r.b * p.Nq + it + 1];
    }
    return r;
}

// the Gumbel noise of ids n0 .. n0 + 3 (n0 a multiple of 4) of a row
__device__ __forceinline__ uint4 sample_bits(const EpiParams& p, const SampleRow& r, int n0) {
    return philox4x32_10(make_uint4((uint32_t)(n0 >> 2), (uint32_t)r.pos, (uint32_t)r.b, 0u), p.seed_lo, p.seed_hi);
}
