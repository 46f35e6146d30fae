// Projection GEMMs of the span forward: Y[M, N] = A[M, K] . W[N, K]^T, where A holds the
// M = B*Nq token rows of the forward (activations) and W is a row-major [out, in] weight.
// bf16 layers run on gfx950 MFMA: few-row launches on the weight-streaming kernel
// (gemm_skinny.hip), the others on the LDS-tiled kernel (gemm_big.hip).  This file holds the
// dispatch and the plain-FMA kernel of an fp32 layer, which stages its fp32 tile in LDS and
// finishes with one of the fused epilogues (EpiKind):
//   EPI_QKV     RoPE at the row's absolute position, q -> workspace, k/v appended to the cache
//               (Copy-as-Decode, Appendix K: positions advance exactly as in decode steps);
//   EPI_SWIGLU  silu(gate) * up, the tile holding matching gate and up columns;
//   EPI_ARGMAX  per-(row, column-tile) max with the lowest index among ties (LM head), so the
//               logits never reach memory unless a debug buffer is given;
//   EPI_PARTIAL fp32 partial sums of one K slice (O and down projections; the residual add
//               and the following RMSNorm happen in the next row kernel).
#include "cad_device.h"

hipError_t launch_skinny(int kind, const void* A, const void* W, int M, int N, int K, const EpiParams& p,
                         hipStream_t s);
bool skinny_supports(int kind, int M, int K);
int skinny_partial_slices(int K);
int skinny_argmax_slots(int kind, int M, int N, int K);
hipError_t launch_big(int kind, const void* A, const void* W, int M, int N, int K, int slices, const EpiParams& p,
                      hipStream_t s);
int big_slots(int kind, int M, int N, int K);
int big_partial_slices(int M, int N, int K, int cus);

namespace {

// ---------------------------------------------------------------------------------------
// epilogues on the fp32 tile C[BM][ldc] in LDS (token-major), run by all 256 threads
// ---------------------------------------------------------------------------------------
template <typename T, int KIND>
__device__ void tile_epilogue(const float* C, int ldc, int m0, int n0, int BM, int BN, int ks, const EpiParams& p) {
    if constexpr (KIND == EPI_QKV) {
        const int half = p.d / 2, npair = BN / 2;
        for (int idx = threadIdx.x; idx < BM * npair; idx += blockDim.x) {
            const int r = idx / npair, q = idx % npair;
            const int f1 = (q / half) * p.d + q % half, i = q % half;
            const int row = m0 + r, F1 = n0 + f1;
            if (row >= p.M || F1 >= p.N) continue;
            const int b = row / p.Nq, it = row % p.Nq;
            if (!seq_ok(p.len_snap, b, p.Nq, p.cap)) continue;
            const int head = F1 / p.d + p.head_off;
            const size_t slot = (size_t)p.len_snap[b] + it;
            const float x1 = C[r * ldc + f1], x2 = C[r * ldc + f1 + half];
            if (head >= p.Hq + p.Hkv) {                  // V cache is dim-major [d][cap]
                T* v = (T*)p.vc + ((size_t)b * p.Hkv + (head - p.Hq - p.Hkv)) * p.d * p.cap + slot;
                Elt<T>::st(v, (size_t)i * p.cap, x1);
                Elt<T>::st(v, (size_t)(i + half) * p.cap, x2);
                continue;
            }
            const float2 cs = p.rope_cs[(size_t)row * half + i];
            const float y1 = x1 * cs.x - x2 * cs.y, y2 = x2 * cs.x + x1 * cs.y;
            T* dst = head < p.Hq ? (T*)p.q_out + ((size_t)row * p.Hq + head) * p.d
                                 : (T*)p.kc + (((size_t)b * p.Hkv + (head - p.Hq)) * p.cap + slot) * p.d;
            Elt<T>::st(dst, i, y1);
            Elt<T>::st(dst, i + half, y2);
        }
    } else if constexpr (KIND == EPI_SWIGLU) {
        const int hb = BN / 2, f0 = n0 / 2;      // the tile holds gate cols [0,hb) and up cols [hb,BN)
        for (int idx = threadIdx.x; idx < BM * hb; idx += blockDim.x) {
            const int r = idx / hb, j = idx % hb;
            const int row = m0 + r, F = f0 + j;
            if (row >= p.M || F >= p.ffn) continue;
            if (!seq_ok(p.len_snap, row / p.Nq, p.Nq, p.cap)) continue;
            const float g = C[r * ldc + j], u = C[r * ldc + hb + j];
            Elt<T>::st((T*)p.act, (size_t)row * p.ffn + F, g / (1.0f + __expf(-g)) * u);
        }
    } else if constexpr (KIND == EPI_PARTIAL) {
        for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
            const int r = idx / BN, f = idx % BN;
            const int row = m0 + r, F = n0 + f;
            if (row >= p.M || F >= p.N) continue;
            p.part[((size_t)ks * p.M + row) * p.N + F] = C[r * ldc + f];
        }
    } else {                                     // EPI_ARGMAX
        const int tpr = blockDim.x / BM;         // threads per row (power of two, <= 64)
        const int r = threadIdx.x / tpr, sub = threadIdx.x % tpr;
        const int row = m0 + r;
        float best = -INFINITY, second = -INFINITY;
        int bi = 0x7fffffff;
        const bool live = row < p.M && seq_ok(p.len_snap, row / p.Nq, p.Nq, p.cap);
        if (live) {
            for (int f = sub; f < BN; f += tpr) {
                const int F = n0 + f;
                if (F >= p.N) break;
                const float v = C[r * ldc + f];
                second = fmaxf(second, fminf(best, v));
                if (v > best) { best = v; bi = F; }                      // increasing F: first max kept
                if (p.logits) p.logits[(size_t)row * p.N + F] = v;
            }
        }
        for (int o = tpr / 2; o > 0; o >>= 1) {
            const float v2 = __shfl_xor(best, o, 64);
            const int i2 = __shfl_xor(bi, o, 64);
            second = second_merge(best, second, v2, __shfl_xor(second, o, 64));
            argmax_merge(best, bi, v2, i2);
        }
        if (live && sub == 0) {
            p.amax_part[(size_t)row * p.amax_slots + n0 / BN] = make_float2(best, __int_as_float(bi));
            if (p.amax_sec) p.amax_sec[(size_t)row * p.amax_slots + n0 / BN] = second;
        }
    }
}

// W row read by tile row `tr` of column tile `nt`.  For SwiGLU the first half of the tile
// takes gate rows and the second half the matching up rows.
__device__ __forceinline__ int w_row(int tr, int nt, int BN, int N, int ffn, bool& valid) {
    if (ffn == 0) {
        const int r = nt * BN + tr;
        valid = r < N;
        return r;
    }
    const int hb = BN / 2, F = nt * hb + (tr % hb);
    valid = F < ffn;
    return tr < hb ? F : ffn + F;
}

// ---------------------------------------------------------------------------------------
// fp32 kernel (fp32 layers): tile 16 tokens x 128 features, plain FMA.
// ---------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                  int M, int N, int K, int nmt, int nnt, int S, int ffn,
                                                  EpiParams p) {
    constexpr int BM = 16, BN = 128, BKF = 32;
    __shared__ float As[BM][BKF + 1];
    __shared__ float Ws[BN][BKF + 1];
    __shared__ float C[BM * (BN + 4)];
    const int unit = blockIdx.x;
    if (unit < nmt * nnt * S) {
        const int ks = unit % S, tile = unit / S;
        const int mt = tile % nmt, nt = tile / nmt, m0 = mt * BM;
        const int kbeg = ks * p.k_slice, kend = min(K, kbeg + p.k_slice);
        const int tid = threadIdx.x;
        const int r = tid / 16, fc = tid % 16;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k0 = kbeg; k0 < kend; k0 += BKF) {
            for (int e = tid; e < BM * BKF; e += 256) {
                const int rr = e / BKF, kk = e % BKF;
                As[rr][kk] = (m0 + rr < M && k0 + kk < kend) ? A[(size_t)(m0 + rr) * K + k0 + kk] : 0.f;
            }
            for (int e = tid; e < BN * BKF; e += 256) {
                const int tr = e / BKF, kk = e % BKF;
                bool v;
                const int wr = w_row(tr, nt, BN, N, ffn, v);
                Ws[tr][kk] = (v && k0 + kk < kend) ? W[(size_t)wr * K + k0 + kk] : 0.f;
            }
            __syncthreads();
            for (int kk = 0; kk < BKF; ++kk) {
                const float a = As[r][kk];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] += a * Ws[fc + 16 * j][kk];
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) C[r * (BN + 4) + fc + 16 * j] = acc[j];
        __syncthreads();
        tile_epilogue<float, KIND>(C, BN + 4, m0, nt * BN, BM, BN, ks, p);
    }
}

struct TilePlan { int BM, BN, nmt, nnt, S, k_slice, grid; };

TilePlan tile_plan(int kind, int M, int N, int K, int slices) {
    TilePlan t;
    t.BN = 128;
    t.BM = 16;
    t.nmt = (M + t.BM - 1) / t.BM;
    // SwiGLU tiles cover BN/2 gate columns and the matching BN/2 up columns (N = 2*ffn)
    t.nnt = kind == EPI_SWIGLU ? (N / 2 + t.BN / 2 - 1) / (t.BN / 2) : (N + t.BN - 1) / t.BN;
    t.S = kind == EPI_PARTIAL ? slices : 1;
    t.k_slice = ((K + t.S - 1) / t.S + 31) / 32 * 32;
    t.grid = t.nmt * t.nnt * t.S;
    return t;
}

template <int KIND>
hipError_t dispatch_f32(const void* A, const void* W, int M, int N, int K, int slices, EpiParams p, hipStream_t s) {
    const int ffn = KIND == EPI_SWIGLU ? p.ffn : 0;
    const TilePlan t = tile_plan(KIND, M, N, K, slices);
    p.k_slice = t.k_slice;
    hipLaunchKernelGGL((k_gemm_f32<KIND>), dim3(t.grid), dim3(256), 0, s, (const float*)A, (const float*)W, M, N, K,
                       t.nmt, t.nnt, t.S, ffn, p);
    return hipGetLastError();
}

}  // namespace

// K slices of an EPI_PARTIAL launch (the O and down projections); the workspace holds
// slices x M x N fp32 partials.
int gemm_argmax_slots(int dtype, int M, int N, int K, int kind) {
    if (dtype == CAD_DTYPE_F32) return tile_plan(EPI_ARGMAX, M, N, K, 1).nnt;
    if (skinny_supports(kind, M, K)) return skinny_argmax_slots(kind, M, N, K);
    return big_slots(kind, M, N, K);
}

// K slices of an EPI_PARTIAL launch (the O and down projections); the workspace holds
// slices x M x N fp32 partials.
int gemm_partial_slices(int dtype, int M, int N, int K) {
    if (dtype == CAD_DTYPE_F32) {
        const TilePlan t = tile_plan(EPI_PARTIAL, M, N, K, 1);
        const int tiles = t.nmt * t.nnt;
        int S = (2 * device_cu_count() + tiles - 1) / tiles;
        const int smax = K / 256 > 1 ? K / 256 : 1;
        return S < 1 ? 1 : (S > smax ? smax : S);
    }
    if (skinny_supports(EPI_PARTIAL, M, K)) return skinny_partial_slices(K);
    return big_partial_slices(M, N, K, device_cu_count());
}

// A bf16 QKV projection the weight-streaming kernel does not take runs as K-slice partials plus
// a row kernel for RoPE and the K/V append: its output is too narrow to fill the chip otherwise.
// (the unsplit tiled QKV projection takes ~21 us at any row count; split into K-slice partials
// plus the finishing row kernel it is faster up to 256 rows, and no faster beyond: at 704 rows
// the unsplit form measured 5-10 us faster per batched PLD round)
bool gemm_qkv_split(int dtype, int M, int K) {
    return dtype == CAD_DTYPE_BF16 && !skinny_supports(EPI_QKV, M, K) && M <= 256;
}

hipError_t launch_gemm(int dtype, int kind, const void* A, const void* W, int M, int N, int K, int slices,
                       EpiParams p, hipStream_t s) {
    if (dtype == CAD_DTYPE_BF16) {
        if (skinny_supports(kind, M, K)) return launch_skinny(kind, A, W, M, N, K, p, s);
        return launch_big(kind, A, W, M, N, K, slices, p, s);
    }
    switch (kind) {
        case EPI_QKV: return dispatch_f32<EPI_QKV>(A, W, M, N, K, 1, p, s);
        case EPI_SWIGLU: return dispatch_f32<EPI_SWIGLU>(A, W, M, N, K, 1, p, s);
        case EPI_ARGMAX: return dispatch_f32<EPI_ARGMAX>(A, W, M, N, K, 1, p, s);
        default: return dispatch_f32<EPI_PARTIAL>(A, W, M, N, K, slices, p, s);
    }
}
