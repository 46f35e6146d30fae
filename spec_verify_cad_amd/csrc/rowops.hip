// Row-wise kernels of the span forward: embedding gather + RMSNorm (which also captures the
// per-sequence cache length the rest of the forward uses), RMSNorm of the residual stream,
// the LM-head argmax finalisation over column-tile partials, and the length commit.
#include "cad_device.h"

namespace {

constexpr int NT = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
}

template <typename T>
__global__ __launch_bounds__(NT) void k_embed_norm(const int32_t* __restrict__ tokens, const T* __restrict__ embed,
                                                   int h, int vocab, int Nq, int cap, float eps,
                                                   const int32_t* __restrict__ kv_len, int32_t* __restrict__ err,
                                                   int32_t* __restrict__ len_snap, float* __restrict__ x,
                                                   T* __restrict__ u) {
    __shared__ float red[4];
    const int r = blockIdx.x, b = r / Nq, it = r % Nq;
    const int len = kv_len[b];
    const bool ok = len >= 0 && len + Nq <= cap;
    if (it == 0 && threadIdx.x == 0) {
        len_snap[b] = ok ? len : -1;
        if (!ok && err) err[b] = CAD_ECAPACITY;
    }
    if (!ok) return;
    int t = tokens[r];
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    const T* e = embed + (size_t)t * h;
    float ss = 0.f;
    for (int j = threadIdx.x; j < h; j += NT) {
        const float v = Elt<T>::ld(e, j);
        ss += v * v;
    }
    ss = block_sum(ss, red);
    const float scale = 1.0f / sqrtf(ss / (float)h + eps);
    for (int j = threadIdx.x; j < h; j += NT) {
        const float v = Elt<T>::ld(e, j);
        if (x) x[(size_t)r * h + j] = v;
        Elt<T>::st(u, (size_t)r * h + j, v * scale);
    }
}

template <typename T>
__global__ __launch_bounds__(NT) void k_rmsnorm(const float* __restrict__ in, T* __restrict__ out, int h, int Nq,
                                                int cap, float eps, const int32_t* __restrict__ len_snap) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    if (!seq_ok(len_snap, r / Nq, Nq, cap)) return;
    const float* p = in + (size_t)r * h;
    float ss = 0.f;
    for (int j = threadIdx.x; j < h; j += NT) ss += p[j] * p[j];
    ss = block_sum(ss, red);
    const float scale = 1.0f / sqrtf(ss / (float)h + eps);
    for (int j = threadIdx.x; j < h; j += NT) Elt<T>::st(out, (size_t)r * h + j, p[j] * scale);
}

// One wave per row: reduce the (max, index) partials of all column tiles.
__global__ __launch_bounds__(64) void k_argmax_final(const float2* __restrict__ part, int ntiles, int Nq, int cap,
                                                     const int32_t* __restrict__ len_snap, int32_t* __restrict__ out) {
    const int r = blockIdx.x;
    if (!seq_ok(len_snap, r / Nq, Nq, cap)) return;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = threadIdx.x; t < ntiles; t += 64) {
        const float2 pv = part[(size_t)r * ntiles + t];
        argmax_merge(best, bi, pv.x, __float_as_int(pv.y));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(best, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        argmax_merge(best, bi, v2, i2);
    }
    if (threadIdx.x == 0) out[r] = bi;
}

__global__ void k_commit(const int32_t* __restrict__ len_snap, int B, int Nq, int cap, int32_t* __restrict__ kv_len) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B && seq_ok(len_snap, b, Nq, cap)) kv_len[b] = len_snap[b] + Nq;
}

}  // namespace

hipError_t launch_embed_norm(const FwdDims& fd, const int32_t* tokens, const void* embed, float eps,
                             const int32_t* kv_len, int32_t* err, const FwdBufs& wb, hipStream_t s) {
    if (fd.dtype == CAD_DTYPE_F32)
        hipLaunchKernelGGL(k_embed_norm<float>, dim3(fd.M), dim3(NT), 0, s, tokens, (const float*)embed, fd.h, fd.V,
                           fd.Nq, fd.cap, eps, kv_len, err, wb.len_snap, wb.x, (float*)wb.u);
    else
        hipLaunchKernelGGL(k_embed_norm<uint16_t>, dim3(fd.M), dim3(NT), 0, s, tokens, (const uint16_t*)embed, fd.h,
                           fd.V, fd.Nq, fd.cap, eps, kv_len, err, wb.len_snap, wb.x, (uint16_t*)wb.u);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const FwdDims& fd, const float* in, void* out, float eps, const int32_t* len_snap,
                          hipStream_t s) {
    if (fd.dtype == CAD_DTYPE_F32)
        hipLaunchKernelGGL(k_rmsnorm<float>, dim3(fd.M), dim3(NT), 0, s, in, (float*)out, fd.h, fd.Nq, fd.cap, eps,
                           len_snap);
    else
        hipLaunchKernelGGL(k_rmsnorm<uint16_t>, dim3(fd.M), dim3(NT), 0, s, in, (uint16_t*)out, fd.h, fd.Nq, fd.cap,
                           eps, len_snap);
    return hipGetLastError();
}

hipError_t launch_argmax_final(const FwdDims& fd, const FwdBufs& wb, int32_t* argmax_out, hipStream_t s) {
    hipLaunchKernelGGL(k_argmax_final, dim3(fd.M), dim3(64), 0, s, wb.amax_part, fd.lm_tiles, fd.Nq, fd.cap,
                       wb.len_snap, argmax_out);
    return hipGetLastError();
}

hipError_t launch_commit(const FwdDims& fd, const FwdBufs& wb, int32_t* kv_len, hipStream_t s) {
    hipLaunchKernelGGL(k_commit, dim3((fd.B + 255) / 256), dim3(256), 0, s, wb.len_snap, fd.B, fd.Nq, fd.cap, kv_len);
    return hipGetLastError();
}
