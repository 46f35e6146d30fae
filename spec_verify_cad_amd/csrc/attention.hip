// Span attention: the Nq new rows of every sequence attend to the cached prefix plus the span
// rows their mask allows (causal span, or SwitchSD's block-triangular candidate mask), with
// grouped-query heads sharing one K/V stream.
//
// bf16 path (gfx950 MFMA, head_dim 64 or 128): split-L flash decoding.  A workgroup owns one
// (sequence, KV head, key chunk, query-row tile); the query rows of a tile are the
// (token, q head) pairs of the GQA group, so every K/V tile is read from HBM once per
// group.  Per 64-key tile: S^T = K . Q^T on MFMA (each lane then holds the scores of ONE
// query), online softmax with exp2, O^T += V^T . P^T on MFMA with P taken straight from
// registers (the MFMA k-slots are mapped onto the keys the lane already holds, and V is
// staged transposed in LDS to match).  P is split into bf16 hi + lo parts, two MFMAs, so
// the attention output carries fp32-level weights into its bf16 rounding point.  Partial (m, l, O) per chunk go to the workspace and a
// merge kernel combines them.
//
// fp32 path: one workgroup per (row, q head), plain two-pass softmax over all keys.
#include "cad_device.h"

namespace {

constexpr int KT = 64;          // keys per LDS tile
constexpr int WAVES = 4;

__device__ __forceinline__ bool key_allowed(int key, int len, int it, int mode, int Dblk) {
    if (key < len) return true;
    const int s = key - len;
    if (mode == CAD_MASK_BLOCK_TRI) {
        const int w = it / Dblk, j = it % Dblk;
        return s >= w * Dblk && s <= w * Dblk + j;
    }
    return s <= it;
}

// RPW = 16-query tiles per wave.  DH = head_dim.
template <int DH, int RPW>
__global__ __launch_bounds__(256) void k_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                   const uint16_t* __restrict__ vc, const int32_t* __restrict__ len_snap,
                                                   int Nq, int Hq, int Hkv, int cap, int mode, int Dblk,
                                                   int chunk, int nsplit, float* __restrict__ part_o,
                                                   float* __restrict__ part_ml) {
    constexpr int ROWS = WAVES * RPW * 16;      // query rows per workgroup
    constexpr int KPAD = 8, VPAD = 8;
    constexpr int DS = DH / 32;                 // MFMA k-steps over head_dim
    constexpr int DB = DH / 16;                 // 16-wide head_dim blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT][DH + KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[DH][KT + VPAD];

    const int split = blockIdx.x, rtile = blockIdx.y;
    const int bg = blockIdx.z, b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv, Rg = Nq * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    const bool ok = seq_ok(len_snap, b, Nq, cap);
    const int len = ok ? len_snap[b] : 0;
    const int row0 = rtile * ROWS;
    // rows of this tile cover tokens it in [row0/G, (row0+ROWS-1)/G]: keys beyond len+it_max are masked
    const int it_max = min(Nq - 1, (row0 + ROWS - 1) / G);
    const int kend_all = len + Nq;
    int kbeg = split * chunk;
    int kend = min(kbeg + chunk, min(kend_all, len + it_max + 1));
    if (!ok) kend = kbeg;                        // nothing to do: write empty partials

    // per-wave query fragments (B operand): lane holds Q[row = l16][dim 32*ks + 8*g4 .. +8]
    bf16x8_t qf[RPW][DS];
    int q_it[RPW];
    bool q_live[RPW];
#pragma unroll
    for (int rp = 0; rp < RPW; ++rp) {
        const int rho = row0 + (wave * RPW + rp) * 16 + l16;
        q_live[rp] = rho < Rg;
        const int it = q_live[rp] ? rho / G : 0, hh = q_live[rp] ? rho % G : 0;
        q_it[rp] = it;
        const uint16_t* qp = q + (((size_t)b * Nq + it) * Hq + g * G + hh) * DH;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            uint4 v = q_live[rp] && ok ? *(const uint4*)(qp + ks * 32 + g4 * 8) : make_uint4(0, 0, 0, 0);
            qf[rp][ks] = *(bf16x8_t*)&v;
        }
    }

    const float sl2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e)/sqrt(d)
    float m_run[RPW], l_run[RPW];
    f32x4_t oacc[RPW][DB];
#pragma unroll
    for (int rp = 0; rp < RPW; ++rp) {
        m_run[rp] = -INFINITY;
        l_run[rp] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rp][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const size_t head_off = ((size_t)b * Hkv + g) * cap * DH;
    const uint16_t* kbase = kc + head_off;
    const uint16_t* vbase = vc + head_off;

    for (int k0 = kbeg; k0 < kend; k0 += KT) {
        __syncthreads();
        // stage K [KT][DH] (row-major) and V^T [DH][KT]
        for (int c = tid; c < KT * DH / 8; c += 256) {
            const int kr = c / (DH / 8), dc = (c % (DH / 8)) * 8;
            const int key = k0 + kr;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (key < kend) {
                kv = *(const uint4*)(kbase + (size_t)key * DH + dc);
                vv = *(const uint4*)(vbase + (size_t)key * DH + dc);
            }
            *(uint4*)&Ks[kr][dc] = kv;
            const uint16_t* ve = (const uint16_t*)&vv;
#pragma unroll
            for (int e = 0; e < 8; ++e) Vt[dc + e][kr] = ve[e];
        }
        __syncthreads();

#pragma unroll
        for (int rp = 0; rp < RPW; ++rp) {
            // S^T[key][query]: 4 key blocks of 16; lane holds keys kb*16 + 4*g4 + i for query l16
            f32x4_t st[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                st[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DS; ++ks) {
                    const bf16x8_t kf = *(const bf16x8_t*)&Ks[kb * 16 + l16][ks * 32 + g4 * 8];
                    st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rp][ks], st[kb], 0, 0, 0);
                }
            }
            // mask + scale, tile max for this lane's query
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = k0 + kb * 16 + g4 * 4 + i;
                    const bool al = q_live[rp] && key < kend && key_allowed(key, len, q_it[rp], mode, Dblk);
                    const float sv = al ? st[kb][i] * sl2 : -INFINITY;
                    st[kb][i] = sv;
                    tmax = fmaxf(tmax, sv);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run[rp], tmax);
            const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run[rp] - m_new);
            float psum = 0.f;
            // P enters the PV MFMA as bf16 hi + bf16 lo (the rounding remainder), so the
            // weights keep about 16 significant bits instead of 8.
            bf16x8_t pf[2], pl[2];               // PV k-steps over 32 keys each
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = m_new == -INFINITY ? 0.f : exp2f(st[kb][i] - m_new);
                    const uint16_t ph = f32_to_bf16(pv);
                    const float rem = pv - bf16_to_f32(ph);
                    const uint16_t plo = f32_to_bf16(rem);
                    psum += pv;
                    // k-slot mapping of PV step kb/2: slots 8*g4+i <- key block 2*(kb/2), slots 8*g4+4+i <- the next
                    ((uint16_t*)&pf[kb >> 1])[(kb & 1) * 4 + i] = ph;
                    ((uint16_t*)&pl[kb >> 1])[(kb & 1) * 4 + i] = plo;
                }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            l_run[rp] = l_run[rp] * alpha + psum;
            m_run[rp] = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[rp][db] *= alpha;
            // O^T[dim][query] += V^T[dim][keys] . P^T[keys][query]
#pragma unroll
            for (int pk = 0; pk < 2; ++pk) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t* vrow = &Vt[db * 16 + l16][pk * 32];
                    uint2 lo = *(const uint2*)(vrow + g4 * 4);          // keys 32pk + 4g4 .. +3
                    uint2 hi = *(const uint2*)(vrow + 16 + g4 * 4);     // keys 32pk + 16 + 4g4 .. +3
                    uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    const bf16x8_t vf = *(bf16x8_t*)&vv;
                    oacc[rp][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[pk], oacc[rp][db], 0, 0, 0);
                    oacc[rp][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[pk], oacc[rp][db], 0, 0, 0);
                }
            }
        }
    }

    // partials: lane holds O^T[dim = db*16 + 4*g4 + i][query l16]
#pragma unroll
    for (int rp = 0; rp < RPW; ++rp) {
        const int rho = row0 + (wave * RPW + rp) * 16 + l16;
        if (rho >= Rg) continue;
        const size_t pidx = (((size_t)b * Hkv + g) * Rg + rho) * nsplit + split;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *(f32x4_t*)(part_o + pidx * DH + db * 16 + g4 * 4) = oacc[rp][db];
        if (g4 == 0) {
            part_ml[pidx * 2 + 0] = m_run[rp];
            part_ml[pidx * 2 + 1] = l_run[rp];
        }
    }
}

// Combine the split partials of one (row, q head): o = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
template <typename T>
__global__ __launch_bounds__(64) void k_attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                   const int32_t* __restrict__ len_snap, int Nq, int Hq, int Hkv,
                                                   int DH, int cap, int nsplit, T* __restrict__ o) {
    const int rowhead = blockIdx.x;                  // (b*Nq + it)*Hq + h
    const int h = rowhead % Hq, row = rowhead / Hq;
    const int b = row / Nq, it = row % Nq;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const int G = Hq / Hkv, g = h / G, hh = h % G;
    const int Rg = Nq * G, rho = it * G + hh;
    const size_t p0 = (((size_t)b * Hkv + g) * Rg + rho) * nsplit;
    float m = -INFINITY;
    for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_ml[(p0 + s) * 2]);
    float L = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float ms = part_ml[(p0 + s) * 2];
        if (ms != -INFINITY) L += exp2f(ms - m) * part_ml[(p0 + s) * 2 + 1];
    }
    for (int dd = threadIdx.x; dd < DH; dd += 64) {
        float acc = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float ms = part_ml[(p0 + s) * 2];
            if (ms != -INFINITY) acc += exp2f(ms - m) * part_o[(p0 + s) * DH + dd];
        }
        Elt<T>::st(o, (size_t)rowhead * DH + dd, acc / L);
    }
}

// fp32 (or any dtype) reference-style kernel: one workgroup per (row, q head); scores in LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_simple(const T* __restrict__ q, const T* __restrict__ kc,
                                                     const T* __restrict__ vc, const int32_t* __restrict__ len_snap,
                                                     int Nq, int Hq, int Hkv, int DH, int cap, int mode, int Dblk,
                                                     T* __restrict__ o) {
    extern __shared__ float sc[];                    // [len + Nq] scores, then scratch
    __shared__ float red[WAVES];
    const int rowhead = blockIdx.x, h = rowhead % Hq, row = rowhead / Hq;
    const int b = row / Nq, it = row % Nq;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const int len = len_snap[b], S = len + Nq;
    const int g = h / (Hq / Hkv);
    const T* qp = q + (size_t)rowhead * DH;
    const T* kb = kc + ((size_t)b * Hkv + g) * cap * DH;
    const T* vb = vc + ((size_t)b * Hkv + g) * cap * DH;
    const float scale = 1.0f / sqrtf((float)DH);
    float mx = -INFINITY;
    for (int key = threadIdx.x; key < S; key += 256) {
        float s = -INFINITY;
        if (key_allowed(key, len, it, mode, Dblk)) {
            float acc = 0.f;
            for (int dd = 0; dd < DH; ++dd) acc += Elt<T>::ld(qp, dd) * Elt<T>::ld(kb, (size_t)key * DH + dd);
            s = acc * scale;
        }
        sc[key] = s;
        mx = fmaxf(mx, s);
    }
    for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int key = threadIdx.x; key < S; key += 256) {
        const float e = sc[key] == -INFINITY ? 0.f : __expf(sc[key] - mx);
        sc[key] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    sum = red[0] + red[1] + red[2] + red[3];
    for (int dd = threadIdx.x; dd < DH; dd += 256) {
        float acc = 0.f;
        for (int key = 0; key < S; ++key)
            if (sc[key] != 0.f) acc += sc[key] * Elt<T>::ld(vb, (size_t)key * DH + dd);
        Elt<T>::st(o, (size_t)rowhead * DH + dd, acc / sum);
    }
}

}  // namespace

hipError_t launch_attention(const FwdDims& fd, const FwdBufs& wb, const void* kc, const void* vc, hipStream_t s) {
    if (fd.dtype == CAD_DTYPE_F32 || (fd.d != 64 && fd.d != 128)) {
        const size_t smem = (size_t)(fd.cap + fd.Nq) * sizeof(float);
        if (fd.dtype == CAD_DTYPE_F32)
            hipLaunchKernelGGL((k_attn_simple<float>), dim3(fd.M * fd.Hq), dim3(256), smem, s, (const float*)wb.q,
                               (const float*)kc, (const float*)vc, wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.d, fd.cap,
                               fd.mode, fd.Dblk, (float*)wb.o);
        else
            hipLaunchKernelGGL((k_attn_simple<uint16_t>), dim3(fd.M * fd.Hq), dim3(256), smem, s,
                               (const uint16_t*)wb.q, (const uint16_t*)kc, (const uint16_t*)vc, wb.len_snap, fd.Nq,
                               fd.Hq, fd.Hkv, fd.d, fd.cap, fd.mode, fd.Dblk, (uint16_t*)wb.o);
        return hipGetLastError();
    }
    const dim3 grid(fd.attn_splits, fd.attn_row_tiles, fd.B * fd.Hkv);
    const bool two = fd.attn_rows_per_wg == 128;
#define CAD_ATTN(DH, RPW)                                                                                        \
    hipLaunchKernelGGL((k_attn_bf16<DH, RPW>), grid, dim3(256), 0, s, (const uint16_t*)wb.q, (const uint16_t*)kc, \
                       (const uint16_t*)vc, wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.mode, fd.Dblk,          \
                       fd.attn_chunk, fd.attn_splits, wb.part_o, wb.part_ml)
    if (fd.d == 128) { if (two) CAD_ATTN(128, 2); else CAD_ATTN(128, 1); }
    else { if (two) CAD_ATTN(64, 2); else CAD_ATTN(64, 1); }
#undef CAD_ATTN
    return hipGetLastError();
}

bool attention_uses_merge(const FwdDims& fd) {
    return !(fd.dtype == CAD_DTYPE_F32 || (fd.d != 64 && fd.d != 128));
}

hipError_t launch_attention_merge(const FwdDims& fd, const FwdBufs& wb, hipStream_t s) {
    hipLaunchKernelGGL((k_attn_merge<uint16_t>), dim3(fd.M * fd.Hq), dim3(64), 0, s, wb.part_o, wb.part_ml,
                       wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.d, fd.cap, fd.attn_splits, (uint16_t*)wb.o);
    return hipGetLastError();
}
