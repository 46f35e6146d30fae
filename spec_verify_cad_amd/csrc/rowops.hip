// Row-wise kernels of the span forward.
//
// k_embed_norm  first kernel of every forward: captures the per-sequence cache length the
//               rest of the forward uses (flagging sequences that would overflow or hold a token
//               id outside the vocabulary), gathers the
//               embedding rows, applies RMSNorm and tabulates the (cos, sin) of each row's
//               rotary angles p * base^(-2i/d) (Copy-as-Decode, Appendix K: the rows take the
//               absolute positions N sequential decode steps would have).  The angle is formed
//               and reduced modulo 2*pi in double, so positions in the tens of thousands keep
//               full fp32 accuracy in cos and sin.
// k_resid_norm  residual add of the K-slice partial sums of a projection (in slice order,
//               so the result does not depend on scheduling), optional rounded copy, and the
//               RMSNorm that feeds the next projection.
// k_argmax_final reduces the LM head's (max, index) slots of each row (ties to the lowest
//               index) and, for a committing forward, advances the cache length: the last
//               kernel of a full forward.
// k_commit      len += Nq for a K/V-only forward.
#include "cad_device.h"

namespace {

constexpr int NT = 256;
constexpr int FB = 8;            // slot loads in flight per lane in the final reductions

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
}

// Four consecutive values to four consecutive stored elements.
__device__ __forceinline__ void st4v(uint16_t* p, float4 v) { st4(p, f32x4_t{v.x, v.y, v.z, v.w}); }
__device__ __forceinline__ void st4v(float* p, float4 v) { *(float4*)p = v; }
// Four consecutive stored elements (8 bytes of bf16 / 16 of fp32) as fp32.
__device__ __forceinline__ float4 ld4(const uint16_t* p) {
    const uint2 w = *(const uint2*)p;
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
}
__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }

template <typename T>
__global__ __launch_bounds__(NT) void k_embed_norm(const int32_t* __restrict__ tokens, const T* __restrict__ embed,
                                                   int h, int vocab, int Nq, int cap, float eps, int mode, int Dblk,
                                                   int half, RopeFreqs freqs, const int32_t* __restrict__ kv_len,
                                                   int32_t* __restrict__ err, int32_t* __restrict__ len_snap,
                                                   float2* __restrict__ rope_cs,
                                                   float* __restrict__ x, T* __restrict__ u) {
    __shared__ float red[4];
    const int r = blockIdx.x, b = r / Nq, it = r % Nq;
    const int len = kv_len[b];
    const bool ok = len >= 0 && len + Nq <= cap;
    const int t = tokens[r];
    if (it == 0) {
        // the sequence's first row also checks every token id of the sequence: one outside
        // [0, vocab) flags the sequence and makes its whole forward a no-op
        int bad = 0;
        for (int j = threadIdx.x; j < Nq; j += NT) {
            const int tj = tokens[(size_t)b * Nq + j];
            bad |= tj < 0 || tj >= vocab;
        }
        const int bad_tok = __syncthreads_or(bad);
        if (threadIdx.x == 0) {
            len_snap[b] = ok && !bad_tok ? len : -1;
            if (err && !ok) err[b] = CAD_ECAPACITY;
            else if (err && bad_tok) err[b] = CAD_EINVAL;
        }
    }
    if (!ok || t < 0 || t >= vocab) return;
    if (rope_cs) {
        const int pos = len + (mode == CAD_MASK_BLOCK_TRI ? it % Dblk : it);
        for (int i = threadIdx.x; i < half; i += NT) {
            const double ang = (double)pos * freqs.inv[i];
            const double k = rint(ang * 0.15915494309189535);            // 1 / (2 pi)
            double red = fma(-k, 6.283185307179586, ang);                 // 2 pi, high part
            red = fma(-k, 2.4492935982947064e-16, red);                   // 2 pi, low part
            float sn, cn;
            sincosf((float)red, &sn, &cn);
            rope_cs[(size_t)r * half + i] = make_float2(cn, sn);
        }
    }
    const T* e = embed + (size_t)t * h;
    // the row is read once, four elements per thread per pass, and kept in registers
    constexpr int QMAX = 8;                        // h <= 4 * NT * QMAX
    float4 v[QMAX];
    float ss = 0.f;
#pragma unroll
    for (int qq = 0; qq < QMAX; ++qq) {
        const int j = 4 * (threadIdx.x + qq * NT);
        if (j < h) {
            v[qq] = ld4(e + j);
            ss += (v[qq].x * v[qq].x + v[qq].y * v[qq].y) + (v[qq].z * v[qq].z + v[qq].w * v[qq].w);
        }
    }
    ss = block_sum(ss, red);
    const float scale = 1.0f / sqrtf(ss / (float)h + eps);
#pragma unroll
    for (int qq = 0; qq < QMAX; ++qq) {
        const int j = 4 * (threadIdx.x + qq * NT);
        if (j < h) {
            if (x) *(float4*)(x + (size_t)r * h + j) = v[qq];
            st4v(u + (size_t)r * h + j, make_float4(v[qq].x * scale, v[qq].y * scale, v[qq].z * scale, v[qq].w * scale));
        }
    }
}


constexpr int RN_NT = 512;

// out = base + sum_s part[s] (fp32); out_t = rnd(out) if given; normed = rnd(RMSNorm(out)).
// One workgroup per row, four columns per thread.  The partial sums of a column are loaded SB
// slices at a time, all of a batch in flight together (clamped addresses, unused ones added as
// zero), and added in slice order, so the result does not depend on scheduling.
template <typename T, int SB>
__global__ __launch_bounds__(RN_NT) void k_resid_norm(const float* __restrict__ base, const float* __restrict__ part,
                                                      int slices, int M, int h, int Nq, int cap, float eps,
                                                      int last_only, const int32_t* __restrict__ len_snap,
                                                      float* __restrict__ out, T* __restrict__ out_t,
                                                      T* __restrict__ normed) {
    __shared__ float red[RN_NT / 64];
    extern __shared__ float4 rowbuf4[];          // [h / 4]
    const int r = blockIdx.x;
    if (!seq_ok(len_snap, r / Nq, Nq, cap)) return;
    const int h4 = h >> 2;
    const size_t sstride = (size_t)M * h;
    float ss = 0.f;
    for (int j4 = threadIdx.x; j4 < h4; j4 += RN_NT) {
        const size_t off = (size_t)r * h + 4 * (size_t)j4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < slices; s0 += SB) {
            float4 v[SB];
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const int sl = min(s0 + i, slices - 1);
                v[i] = *(const float4*)(part + sl * sstride + off);
            }
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const bool use = s0 + i < slices;
                acc.x += use ? v[i].x : 0.f;
                acc.y += use ? v[i].y : 0.f;
                acc.z += use ? v[i].z : 0.f;
                acc.w += use ? v[i].w : 0.f;
            }
        }
        const float4 b = *(const float4*)(base + off);
        const float4 o = make_float4(b.x + acc.x, b.y + acc.y, b.z + acc.z, b.w + acc.w);
        rowbuf4[j4] = o;
        *(float4*)(out + off) = o;
        if (out_t) st4v(out_t + off, o);
        ss += (o.x * o.x + o.y * o.y) + (o.z * o.z + o.w * o.w);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < RN_NT / 64; ++w) t += red[w];
    const float scale = 1.0f / sqrtf(t / (float)h + eps);
    if (last_only && r % Nq != Nq - 1) return;
    const size_t nrow = last_only ? (size_t)(r / Nq) : (size_t)r;   // compact: one row per sequence
    for (int j4 = threadIdx.x; j4 < h4; j4 += RN_NT) {
        const float4 o = rowbuf4[j4];
        st4v(normed + nrow * h + 4 * (size_t)j4, make_float4(o.x * scale, o.y * scale, o.z * scale, o.w * scale));
    }
}

// The split form of the QKV epilogue: one workgroup per row r (token it of sequence b).  Each
// thread takes four consecutive rotation pairs (i, i + d/2) of one produced head, adds the K-slice
// partials in slice order, rotates q and k with the row's (cos, sin) and stores q to the
// workspace, k to cache slot len + it and v (unrotated) to the dim-major cache.
__global__ __launch_bounds__(256) void k_qkv_finish(const float* __restrict__ part, int slices, int M, int N,
                                                    int head_off, int Hq, int Hkv, int d, int Nq, int cap,
                                                    const int32_t* __restrict__ len_snap,
                                                    const float2* __restrict__ rope_cs, uint16_t* __restrict__ q_out,
                                                    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
    const int r = blockIdx.x, b = r / Nq, it = r % Nq;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const size_t slot = (size_t)len_snap[b] + it;
    const int half = d / 2, groups = N / 8;               // 4 pairs per group, N/2 pairs per row
    const size_t sstride = (size_t)M * N;
    for (int gi = threadIdx.x; gi < groups; gi += 256) {
        const int hl = gi / (half / 4), i0 = (gi % (half / 4)) * 4;
        const size_t c1 = (size_t)r * N + (size_t)hl * d + i0;
        float4 x1 = make_float4(0.f, 0.f, 0.f, 0.f), x2 = x1;
        for (int sl = 0; sl < slices; ++sl) {             // slice order
            const float4 a = *(const float4*)(part + sl * sstride + c1);
            const float4 c = *(const float4*)(part + sl * sstride + c1 + half);
            x1.x += a.x; x1.y += a.y; x1.z += a.z; x1.w += a.w;
            x2.x += c.x; x2.y += c.y; x2.z += c.z; x2.w += c.w;
        }
        const int head = hl + head_off;
        const float v1[4] = {x1.x, x1.y, x1.z, x1.w}, v2[4] = {x2.x, x2.y, x2.z, x2.w};
        if (head >= Hq + Hkv) {                           // V: dim-major cache, stored unrotated
            uint16_t* vp = vc + (((size_t)b * Hkv + (head - Hq - Hkv)) * d + i0) * cap + slot;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vp[(size_t)i * cap] = f32_to_bf16(v1[i]);
                vp[(size_t)(i + half) * cap] = f32_to_bf16(v2[i]);
            }
            continue;
        }
        const float2* cs = rope_cs + (size_t)r * half + i0;
        f32x4_t y1, y2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2 t = cs[i];
            y1[i] = v1[i] * t.x - v2[i] * t.y;
            y2[i] = v2[i] * t.x + v1[i] * t.y;
        }
        uint16_t* dst = head < Hq ? q_out + ((size_t)r * Hq + head) * d
                                  : kc + (((size_t)b * Hkv + (head - Hq)) * cap + slot) * d;
        st4(dst + i0, y1);
        st4(dst + i0 + half, y2);
    }
}

// Grammar-masked argmax: one workgroup of AMAX waves per row of u3 (rps rows per sequence: Nq,
// or 1 when only each sequence's last row was normed).  Wave a computes the logit of allowed
// slot a, the dot product of the final normed row with that LM-head row (16-byte vector loads,
// fp32 sums); then thread 0 takes the largest logit (ties to the lowest id), writes the slot
// logits and, for the sequence's first row, advances the cache length by Nq.
constexpr int AMAX = 16;
__device__ __forceinline__ float dot_vec(uint4 x, uint4 w) {
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ws[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc += __uint_as_float(xs[i] << 16) * __uint_as_float(ws[i] << 16);
        acc += __uint_as_float(xs[i] & 0xFFFF0000u) * __uint_as_float(ws[i] & 0xFFFF0000u);
    }
    return acc;
}
__device__ __forceinline__ float dot_vec(float4 x, float4 w) { return x.x * w.x + x.y * w.y + x.z * w.z + x.w * w.w; }
template <typename T> struct VecOf;
template <> struct VecOf<uint16_t> { using type = uint4; static constexpr int n = 8; };
template <> struct VecOf<float> { using type = float4; static constexpr int n = 4; };

template <typename T>
__global__ __launch_bounds__(AMAX * 64) void k_allowed_argmax(const T* __restrict__ u3, const T* __restrict__ wlm,
                                                              int h, int V, const int32_t* __restrict__ allowed,
                                                              int A, int rps, int Nq, int cap,
                                                              const int32_t* __restrict__ len_snap,
                                                              int32_t* __restrict__ out, float* __restrict__ logits,
                                                              int32_t* __restrict__ kv_len) {
    using VT = typename VecOf<T>::type;
    __shared__ float val[AMAX];
    __shared__ int idv[AMAX];
    const int r = blockIdx.x, b = r / rps;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const int lane = threadIdx.x & 63, a = threadIdx.x >> 6;
    if (a < A) {
        const int raw = allowed[(size_t)r * A + a];
        const int id = (raw >= 0 && raw < V) ? raw : -1;
        float acc = 0.f;
        if (id >= 0) {
            const VT* x = (const VT*)(u3 + (size_t)r * h);
            const VT* w = (const VT*)(wlm + (size_t)id * h);
            const int nv = h / VecOf<T>::n;
#pragma unroll 4
            for (int v = lane; v < nv; v += 64) acc += dot_vec(x[v], w[v]);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            val[a] = acc;
            idv[a] = id;
        }
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    float best = -INFINITY;
    int bi = -1;
    for (int k = 0; k < A; ++k) {
        const int id = idv[k];
        const float v = id >= 0 ? val[k] : -INFINITY;
        if (id >= 0 && (bi < 0 || v > best || (v == best && id < bi))) { best = v; bi = id; }
        if (logits) logits[(size_t)r * A + k] = v;
    }
    out[r] = bi;
    if (kv_len && r % rps == 0) kv_len[b] = len_snap[b] + Nq;
}

// Sampled forward, one wave per row: merges the row's LM-head slots (Gumbel-perturbed maxima y
// over all ids and z over the ids other than the draft, and the log-sum-exp of the tempered
// logits), then the prediction: a row holding a draft d keeps it when the row's acceptance
// uniform is below p(d) = exp(logit_d / T - lse) and otherwise takes z; a row without a draft
// takes y.  The first row of each sequence advances the cache length.
__global__ __launch_bounds__(64) void k_sample_final(const float4* __restrict__ part, int slots, int rps, int Nq,
                                                     int cap, const int32_t* __restrict__ len_snap,
                                                     const int32_t* __restrict__ tokens,
                                                     const int32_t* __restrict__ draft_len, uint32_t seed_lo,
                                                     uint32_t seed_hi, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ kv_len) {
    const int r = blockIdx.x, b = r / rps;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    SampleState st;
    sample_init(st);
    // a lane merges slots lane, lane + 64, ... in that order; the loads of FB of them are issued
    // before the first is used (clamped addresses, surplus ones not merged)
    for (int t0 = 0; t0 < slots; t0 += 64 * FB) {
        SampleState v[FB];
#pragma unroll
        for (int u = 0; u < FB; ++u)
            v[u] = sample_load(part + ((size_t)r * slots + min(t0 + (int)threadIdx.x + 64 * u, slots - 1)) * 2);
#pragma unroll
        for (int u = 0; u < FB; ++u)
            if (t0 + (int)threadIdx.x + 64 * u < slots) sample_merge(st, v[u]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sample_merge(st, sample_shfl_xor(st, o));
    if (threadIdx.x != 0) return;
    const int it = rps == 1 ? Nq - 1 : r % Nq;
    int d = -1;
    if (draft_len && rps != 1) {
        int dl = draft_len[b];
        dl = dl < Nq - 1 ? dl : Nq - 1;
        if (it < dl) d = tokens[(size_t)b * Nq + it + 1];
    }
    int pred = st.yi;
    if (d >= 0) {
        const float lse = st.m + logf(st.s);
        const float pd = expf(st.dl - lse);
        const uint4 w = philox4x32_10(make_uint4(0u, (uint32_t)(len_snap[b] + it), (uint32_t)b, 1u), seed_lo, seed_hi);
        pred = uniform_from_bits(w.x) < pd ? d : st.zi;
    }
    out[r] = pred;
    if (kv_len && r % rps == 0) kv_len[b] = len_snap[b] + Nq;
}

// One wave per row.  The LM head ran on rps rows per sequence (Nq, or 1 for the last row only):
// row r belongs to sequence b = r / rps, and the wave of the sequence's first row commits.
// With top2_gap, the runner-up slots (sec) are merged too and the row's largest minus
// second-largest logit is written.
template <bool GAP>
__global__ __launch_bounds__(64) void k_argmax_final(const float2* __restrict__ part, const float* __restrict__ sec,
                                                     int slots, int rps, int Nq, int cap,
                                                     const int32_t* __restrict__ len_snap, int32_t* __restrict__ out,
                                                     float* __restrict__ gap, int32_t* __restrict__ kv_len) {
    const int r = blockIdx.x, b = r / rps;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    float best = -INFINITY, second = -INFINITY;
    int bi = 0x7fffffff;
    // slots lane, lane + 64, ... with the loads of FB of them in flight at once (clamped
    // addresses, surplus ones not merged)
    for (int t0 = 0; t0 < slots; t0 += 64 * FB) {
        float2 pv[FB];
        float sv[FB];
#pragma unroll
        for (int u = 0; u < FB; ++u) {
            const size_t i = (size_t)r * slots + min(t0 + (int)threadIdx.x + 64 * u, slots - 1);
            pv[u] = part[i];
            if constexpr (GAP) sv[u] = sec[i];
        }
#pragma unroll
        for (int u = 0; u < FB; ++u)
            if (t0 + (int)threadIdx.x + 64 * u < slots) {
                if constexpr (GAP) second = second_merge(best, second, pv[u].x, sv[u]);
                argmax_merge(best, bi, pv[u].x, __float_as_int(pv[u].y));
            }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(best, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        if constexpr (GAP) second = second_merge(best, second, v2, __shfl_xor(second, o, 64));
        argmax_merge(best, bi, v2, i2);
    }
    if (threadIdx.x == 0) {
        out[r] = bi;
        if constexpr (GAP) gap[r] = best - second;
        if (kv_len && r % rps == 0) kv_len[b] = len_snap[b] + Nq;
    }
}

__global__ void k_commit(const int32_t* __restrict__ len_snap, int B, int Nq, int cap, int32_t* __restrict__ kv_len) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B && seq_ok(len_snap, b, Nq, cap)) kv_len[b] = len_snap[b] + Nq;
}

}  // namespace

hipError_t launch_embed_norm(const FwdDims& fd, const int32_t* tokens, const void* embed, float eps,
                             const RopeFreqs& freqs, const int32_t* kv_len, int32_t* err, const FwdBufs& wb,
                             hipStream_t s) {
    const int half = fd.d / 2;
    if (fd.dtype == CAD_DTYPE_F32)
        hipLaunchKernelGGL(k_embed_norm<float>, dim3(fd.M), dim3(NT), 0, s, tokens, (const float*)embed, fd.h, fd.V,
                           fd.Nq, fd.cap, eps, fd.mode, fd.Dblk, half, freqs, kv_len, err, wb.len_snap,
                           wb.rope_cs, wb.x, (float*)wb.u);
    else
        hipLaunchKernelGGL(k_embed_norm<uint16_t>, dim3(fd.M), dim3(NT), 0, s, tokens, (const uint16_t*)embed, fd.h,
                           fd.V, fd.Nq, fd.cap, eps, fd.mode, fd.Dblk, half, freqs, kv_len, err, wb.len_snap,
                           wb.rope_cs, wb.x, (uint16_t*)wb.u);
    return hipGetLastError();
}

template <typename T, int SB>
static void resid_norm_go(const FwdDims& fd, const float* base, const float* part, int slices, float* out_f32,
                          void* out_t, void* normed, int last, float eps, const int32_t* len_snap, hipStream_t s) {
    const size_t smem = (size_t)fd.h * sizeof(float);
    hipLaunchKernelGGL((k_resid_norm<T, SB>), dim3(fd.M), dim3(RN_NT), smem, s, base, part, slices, fd.M, fd.h,
                       fd.Nq, fd.cap, eps, last, len_snap, out_f32, (T*)out_t, (T*)normed);
}

template <typename T>
static void resid_norm_t(const FwdDims& fd, const float* base, const float* part, int slices, float* out_f32,
                         void* out_t, void* normed, int last, float eps, const int32_t* len_snap, hipStream_t s) {
    if (slices <= 4) resid_norm_go<T, 4>(fd, base, part, slices, out_f32, out_t, normed, last, eps, len_snap, s);
    else if (slices <= 8) resid_norm_go<T, 8>(fd, base, part, slices, out_f32, out_t, normed, last, eps, len_snap, s);
    else resid_norm_go<T, 16>(fd, base, part, slices, out_f32, out_t, normed, last, eps, len_snap, s);
}

hipError_t launch_resid_norm(const FwdDims& fd, const float* base, const float* part, int slices, float* out_f32,
                             void* out_t, void* normed, bool last_only, float eps, const int32_t* len_snap,
                             hipStream_t s) {
    const int last = last_only ? 1 : 0;
    if (fd.dtype == CAD_DTYPE_F32)
        resid_norm_t<float>(fd, base, part, slices, out_f32, out_t, normed, last, eps, len_snap, s);
    else resid_norm_t<uint16_t>(fd, base, part, slices, out_f32, out_t, normed, last, eps, len_snap, s);
    return hipGetLastError();
}

hipError_t launch_argmax_final(const FwdDims& fd, const FwdBufs& wb, bool last_only, int32_t* argmax_out,
                               float* top2_gap, int32_t* kv_len, hipStream_t s) {
    const int rps = last_only ? 1 : fd.Nq;
    const int slots = last_only ? wb.amax_slots_last : wb.amax_slots;
    if (top2_gap)
        hipLaunchKernelGGL(k_argmax_final<true>, dim3(fd.B * rps), dim3(64), 0, s, wb.amax_part, wb.amax_sec, slots,
                           rps, fd.Nq, fd.cap, wb.len_snap, argmax_out, top2_gap, kv_len);
    else
        hipLaunchKernelGGL(k_argmax_final<false>, dim3(fd.B * rps), dim3(64), 0, s, wb.amax_part, nullptr, slots,
                           rps, fd.Nq, fd.cap, wb.len_snap, argmax_out, nullptr, kv_len);
    return hipGetLastError();
}

hipError_t launch_commit(const FwdDims& fd, const FwdBufs& wb, int32_t* kv_len, hipStream_t s) {
    hipLaunchKernelGGL(k_commit, dim3((fd.B + 255) / 256), dim3(256), 0, s, wb.len_snap, fd.B, fd.Nq, fd.cap, kv_len);
    return hipGetLastError();
}

hipError_t launch_qkv_finish(const FwdDims& fd, const float* part, int slices, int N, int head_off,
                             const FwdBufs& wb, void* kc, void* vc, hipStream_t s) {
    hipLaunchKernelGGL(k_qkv_finish, dim3(fd.M), dim3(256), 0, s, part, slices, fd.M, N, head_off, fd.Hq, fd.Hkv,
                       fd.d, fd.Nq, fd.cap, wb.len_snap, wb.rope_cs, (uint16_t*)wb.q, (uint16_t*)kc, (uint16_t*)vc);
    return hipGetLastError();
}

hipError_t launch_allowed_argmax(const FwdDims& fd, const FwdBufs& wb, const void* w_lm, const int32_t* allowed, int A,
                                 bool last_only, int32_t* argmax_out, float* logits_out, int32_t* kv_len,
                                 hipStream_t s) {
    if (A < 1 || A > AMAX) return hipErrorInvalidValue;
    const int rps = last_only ? 1 : fd.Nq;
    const int rows = fd.B * rps;
    if (fd.dtype == CAD_DTYPE_F32)
        hipLaunchKernelGGL(k_allowed_argmax<float>, dim3(rows), dim3(AMAX * 64), 0, s, (const float*)wb.u3,
                           (const float*)w_lm, fd.h, fd.V, allowed, A, rps, fd.Nq, fd.cap, wb.len_snap, argmax_out,
                           logits_out, kv_len);
    else
        hipLaunchKernelGGL(k_allowed_argmax<uint16_t>, dim3(rows), dim3(AMAX * 64), 0, s, (const uint16_t*)wb.u3,
                           (const uint16_t*)w_lm, fd.h, fd.V, allowed, A, rps, fd.Nq, fd.cap, wb.len_snap, argmax_out,
                           logits_out, kv_len);
    return hipGetLastError();
}

hipError_t launch_sample_final(const FwdDims& fd, const FwdBufs& wb, bool last_only, const int32_t* tokens,
                               const SampleArgs& sa, int32_t* pred_out, int32_t* kv_len, hipStream_t s) {
    const int rps = last_only ? 1 : fd.Nq;
    const int slots = last_only ? wb.samp_slots_last : wb.samp_slots;
    hipLaunchKernelGGL(k_sample_final, dim3(fd.B * rps), dim3(64), 0, s, wb.samp_part, slots, rps, fd.Nq, fd.cap,
                       wb.len_snap, tokens, sa.draft_len, (uint32_t)(sa.seed & 0xFFFFFFFFu), (uint32_t)(sa.seed >> 32),
                       pred_out, kv_len);
    return hipGetLastError();
}
