// Span attention: the Nq new rows of every sequence attend to the cached prefix plus the span
// rows their mask allows (causal span, or SwitchSD's block-triangular candidate mask), with
// grouped-query heads sharing one K/V stream.
//
// bf16 path (gfx950 MFMA, head_dim 64 or 128): split-L flash decoding with no LDS.  A
// workgroup owns one (sequence, KV head, key chunk, 64-row tile); the rows of a tile are the
// (token, q head) pairs of the GQA group, so every K/V byte of a chunk is fetched from HBM once
// per group (the four waves of a workgroup share it through L1).  Each wave takes 16 rows and
// walks its keys 32 at a time, loading MFMA operands straight from the cache:
//   S^T = K . Q^T   A = 16 keys x 32 dims of the K cache (16 contiguous bytes per lane),
//                   B = the wave's query fragments (loaded once);
//   O^T += V^T . P^T  A = 16 dims x 32 keys of the dim-major V cache, B = P^T taken from the
//                   score registers: the MFMA k-slots 8g+i / 8g+4+i are mapped to keys 4g+i /
//                   16+4g+i, which are exactly the scores lane (g, r) holds, so P never moves
//                   between lanes, and V^T is read with the same key order (two 8-byte loads).
// Online softmax runs in registers with exp2; P enters the PV product as bf16 hi + bf16 lo
// (the rounding remainder), two MFMAs, so the weights keep about 16 significant bits.  With
// one key chunk the wave writes the normalised output; otherwise it writes (m, l, O) partials
// and a merge kernel combines them.
//
// fp32 path: one workgroup per (row, q head), plain two-pass softmax over all keys.
#include "cad_device.h"

namespace {

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

// Keys per split for a sequence of len cached rows and Nq new rows: the live keys spread
// evenly over the nsplit splits, in multiples of 32 and at least 64, so splits past the live
// range get no keys.  Computed on the device from the cache length the forward captured.
__device__ __forceinline__ int split_chunk(int len, int Nq, int nsplit) {
    const int S = len + Nq;
    int c = (S + nsplit - 1) / nsplit;
    c = (c + 31) & ~31;
    return c < 64 ? 64 : c;
}

// four bf16 of one V row (keys key0..key0+3, key0 a multiple of 4); keys at or past kend read
// as zero.  Branch-free: a group wholly past kend reads slot 0 instead (cap is a multiple of 4,
// so a load never crosses the end of a row), so all loads of a step issue back to back.
__device__ __forceinline__ uint2 v4(const uint16_t* vrow, int key0, int kend) {
    const int n = kend - key0;                       // valid keys in the group
    uint2 w = *(const uint2*)(vrow + (n > 0 ? key0 : 0));   // keys key0 .. key0+3, low half first
    w.x &= n >= 2 ? 0xFFFFFFFFu : (n == 1 ? 0xFFFFu : 0u);
    w.y &= n >= 4 ? 0xFFFFFFFFu : (n == 3 ? 0xFFFFu : 0u);
    return w;
}

template <int DH>
__global__ __launch_bounds__(256) void k_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                   const uint16_t* __restrict__ vc, const int32_t* __restrict__ len_snap,
                                                   int Nq, int Hq, int Hkv, int cap, int mode, int Dblk,
                                                   int nsplit, float* __restrict__ part_o,
                                                   float* __restrict__ part_ml, uint16_t* __restrict__ o_out) {
    constexpr int DS = DH / 32;                 // MFMA k-steps over head_dim
    constexpr int DB = DH / 16;                 // 16-wide head_dim blocks of the output
    const int split = blockIdx.x, rtile = blockIdx.y;
    const int bg = blockIdx.z, b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv, Rg = Nq * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int wrow0 = rtile * (WAVES * 16) + wave * 16;
    if (wrow0 >= Rg) return;                    // no rows for this wave (no barriers below)
    const bool ok = seq_ok(len_snap, b, Nq, cap);
    const int len = ok ? len_snap[b] : 0;
    const int rho = wrow0 + l16;
    const bool qlive = rho < Rg;
    const int it = qlive ? rho / G : 0, hh = qlive ? rho % G : 0;
    // keys past len + (last token of the wave) are masked for every row of the wave
    const int it_max = min(Nq - 1, min(wrow0 + 15, Rg - 1) / G);
    const int chunk = split_chunk(len, Nq, nsplit);
    const int kbeg = split * chunk;
    int kend = min(kbeg + chunk, len + it_max + 1);
    if (!ok) kend = kbeg;

    bf16x8_t qf[DS];
    {
        const uint16_t* qp = q + (((size_t)b * Nq + it) * Hq + g * G + hh) * DH;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            uint4 v = qlive && ok ? *(const uint4*)(qp + ks * 32 + g4 * 8) : make_uint4(0, 0, 0, 0);
            qf[ks] = *(bf16x8_t*)&v;
        }
    }

    const float sl2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e)/sqrt(d)
    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const size_t head = (size_t)b * Hkv + g;
    const uint16_t* kbase = kc + head * cap * DH;
    const uint16_t* vbase = vc + head * DH * cap;          // dim-major: row = one dim over all slots

    // Operands of one 32-key step.  Keys at or past kend load from slot 0 (always a valid
    // address) and are masked afterwards, so a step can be fetched before it is known to be
    // needed: the loop keeps the next step's loads in flight while it computes the current one.
    struct StepOps { bf16x8_t kf[2][DS]; bf16x8_t vf[DB]; };
    auto load = [&](int k0, StepOps& op) {
        // K fragments: lane (key l16, g4) of key block kb
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = k0 + kb * 16 + l16;
            const uint16_t* kp = kbase + (size_t)(key < kend ? key : 0) * DH + g4 * 8;
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) {
                uint4 v = *(const uint4*)(kp + ks * 32);
                op.kf[kb][ks] = *(bf16x8_t*)&v;
            }
        }
        // V^T fragments: lane (dim db*16 + l16, g4) takes keys 4g4..+3 and 16+4g4..+3
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t* vrow = vbase + (size_t)(db * 16 + l16) * cap;
            const uint2 lo = v4(vrow, k0 + 4 * g4, kend), hi = v4(vrow, k0 + 16 + 4 * g4, kend);
            uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
            op.vf[db] = *(bf16x8_t*)&vv;
        }
    };
    auto compute = [&](int k0, const StepOps& op) {
        // S^T[key][query]: lane holds keys kb*16 + 4*g4 + i of query l16
        f32x4_t st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            st[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DS; ++ks)
                st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kf[kb][ks], qf[ks], st[kb], 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = k0 + kb * 16 + g4 * 4 + i;
                const bool al = qlive && key < kend && key_allowed(key, len, it, mode, Dblk);
                const float sv = al ? st[kb][i] * sl2 : -INFINITY;
                st[kb][i] = sv;
                tmax = fmaxf(tmax, sv);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
        float psum = 0.f;
        // P^T fragment: k-slot 8*g4 + i <- key 4*g4 + i (block 0), 8*g4 + 4 + i <- key 16 + 4*g4 + i
        bf16x8_t ph, pl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = m_new == -INFINITY ? 0.f : exp2f(st[kb][i] - m_new);
                const uint16_t hb = f32_to_bf16(pv);
                const uint16_t lb = f32_to_bf16(pv - bf16_to_f32(hb));
                psum += pv;
                ((uint16_t*)&ph)[kb * 4 + i] = hb;
                ((uint16_t*)&pl)[kb * 4 + i] = lb;
            }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            oacc[db] *= alpha;
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.vf[db], ph, oacc[db], 0, 0, 0);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.vf[db], pl, oacc[db], 0, 0, 0);
        }
    };

    StepOps opa, opb;
    load(kbeg, opa);
    for (int k0 = kbeg; k0 < kend; k0 += 64) {
        load(k0 + 32, opb);
        compute(k0, opa);
        if (k0 + 32 >= kend) break;
        load(k0 + 64, opa);
        compute(k0 + 32, opb);
    }

    if (!qlive) return;
    // lane holds O^T[dim = db*16 + 4*g4 + i][query l16]
    if (nsplit == 1) {
        if (!ok) return;
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t* op = o_out + (((size_t)b * Nq + it) * Hq + g * G + hh) * DH;
#pragma unroll
        for (int db = 0; db < DB; ++db) st4(op + db * 16 + g4 * 4, oacc[db] * inv);
        return;
    }
    const size_t pidx = (head * Rg + rho) * nsplit + split;
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4_t*)(part_o + pidx * DH + db * 16 + g4 * 4) = oacc[db];
    if (g4 == 0) {
        part_ml[pidx * 2 + 0] = m_run;
        part_ml[pidx * 2 + 1] = l_run;
    }
}

// Combine the split partials of one (row, q head): o = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
// Only splits that held keys for the sequence are read.  The 256 threads form NG groups of DH/4
// threads (four dims each); group j sums splits j, j + NG, ... in order, and the groups are added
// in order, so the result does not depend on scheduling.  The O loads of the first SB splits of
// every group are issued before the weights are known.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                   const int32_t* __restrict__ len_snap, int Nq, int Hq, int Hkv,
                                                   int cap, int nsplit, T* __restrict__ o) {
    constexpr int TPG = DH / 4, NG = 256 / TPG, SB = 8;
    __shared__ float wgt[256];
    __shared__ float red[2][4];
    __shared__ float4 gacc[NG][TPG];
    const int rowhead = blockIdx.x;                  // (b*Nq + it)*Hq + h
    const int h = rowhead % Hq, row = rowhead / Hq;
    const int b = row / Nq, it = row % Nq;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const int len = len_snap[b];
    const int chunk = split_chunk(len, Nq, nsplit);
    const int live = min(nsplit, (len + Nq + chunk - 1) / chunk);
    const int G = Hq / Hkv, g = h / G, hh = h % G;
    const int Rg = Nq * G, rho = it * G + hh;
    const size_t p0 = (((size_t)b * Hkv + g) * Rg + rho) * nsplit;
    const int tid = threadIdx.x, grp = tid / TPG, q = tid % TPG;
    const int lane = tid & 63, wave = tid >> 6;

    float4 ov[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        const int sp = min(grp + NG * j, live - 1);
        ov[j] = *(const float4*)(part_o + (p0 + sp) * DH + 4 * q);
    }
    float m = -INFINITY;
    for (int sp = tid; sp < live; sp += 256) m = fmaxf(m, part_ml[(p0 + sp) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) red[0][wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float lsum = 0.f;
    for (int sp = tid; sp < live; sp += 256) {
        const float2 ml = *(const float2*)(part_ml + (p0 + sp) * 2);
        const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - m);
        wgt[sp] = w;
        lsum += w * ml.y;
    }
    lsum = wave_sum(lsum);
    if (lane == 0) red[1][wave] = lsum;
    __syncthreads();
    const float L = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0;; j0 += SB) {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int sp = grp + NG * (j0 + j);
            const float w = sp < live ? wgt[sp] : 0.f;
            acc.x += w * ov[j].x;
            acc.y += w * ov[j].y;
            acc.z += w * ov[j].z;
            acc.w += w * ov[j].w;
        }
        if (grp + NG * (j0 + SB) >= live) break;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int sp = min(grp + NG * (j0 + SB + j), live - 1);
            ov[j] = *(const float4*)(part_o + (p0 + sp) * DH + 4 * q);
        }
    }
    gacc[grp][q] = acc;
    __syncthreads();
    if (tid < TPG) {
        float4 t = gacc[0][tid];
#pragma unroll
        for (int j = 1; j < NG; ++j) {
            const float4 u = gacc[j][tid];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const size_t ob = (size_t)rowhead * DH + 4 * tid;
        Elt<T>::st(o, ob + 0, t.x * inv);
        Elt<T>::st(o, ob + 1, t.y * inv);
        Elt<T>::st(o, ob + 2, t.z * inv);
        Elt<T>::st(o, ob + 3, t.w * inv);
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
    const T* vb = vc + ((size_t)b * Hkv + g) * DH * cap;      // dim-major
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
            if (sc[key] != 0.f) acc += sc[key] * Elt<T>::ld(vb, (size_t)dd * cap + key);
        Elt<T>::st(o, (size_t)rowhead * DH + dd, acc / sum);
    }
}

bool mfma_path(const FwdDims& fd) { return !(fd.dtype == CAD_DTYPE_F32 || (fd.d != 64 && fd.d != 128)); }

}  // namespace

// Split plan of the MFMA path: 64-row tiles of each GQA group and enough key splits for about
// two workgroups per CU (each split at least 64 keys of a full cache); the keys of a split
// follow from the sequence's length on the device.
void attention_plan(FwdDims* fd, int cus) {
    const int G = fd->Hq / fd->Hkv, Rg = fd->Nq * G;
    fd->attn_rows_per_wg = WAVES * 16;
    fd->attn_row_tiles = (Rg + fd->attn_rows_per_wg - 1) / fd->attn_rows_per_wg;
    const long units = (long)fd->B * fd->Hkv * fd->attn_row_tiles;
    const long want = 2L * cus;
    long splits = (want + units - 1) / units;
    const long most = (fd->cap + fd->Nq + 63) / 64;       // splits of at least 64 keys
    if (splits > most) splits = most;
    if (splits > 256) splits = 256;                      // the merge holds at most 256 split weights
    if (splits < 1) splits = 1;
    fd->attn_splits = (int)splits;
    fd->attn_chunk = 0;                                  // per sequence, from its length, on the device
}

hipError_t launch_attention(const FwdDims& fd, const FwdBufs& wb, const void* kc, const void* vc, hipStream_t s) {
    if (!mfma_path(fd)) {
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
    if (fd.d == 128)
        hipLaunchKernelGGL((k_attn_bf16<128>), grid, dim3(WAVES * 64), 0, s, (const uint16_t*)wb.q, (const uint16_t*)kc,
                           (const uint16_t*)vc, wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.mode, fd.Dblk,
                           fd.attn_splits, wb.part_o, wb.part_ml, (uint16_t*)wb.o);
    else
        hipLaunchKernelGGL((k_attn_bf16<64>), grid, dim3(WAVES * 64), 0, s, (const uint16_t*)wb.q, (const uint16_t*)kc,
                           (const uint16_t*)vc, wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.mode, fd.Dblk,
                           fd.attn_splits, wb.part_o, wb.part_ml, (uint16_t*)wb.o);
    return hipGetLastError();
}

bool attention_uses_merge(const FwdDims& fd) { return mfma_path(fd) && fd.attn_splits > 1; }

hipError_t launch_attention_merge(const FwdDims& fd, const FwdBufs& wb, hipStream_t s) {
    if (fd.d == 128)
        hipLaunchKernelGGL((k_attn_merge<uint16_t, 128>), dim3(fd.M * fd.Hq), dim3(256), 0, s, wb.part_o, wb.part_ml,
                           wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, (uint16_t*)wb.o);
    else
        hipLaunchKernelGGL((k_attn_merge<uint16_t, 64>), dim3(fd.M * fd.Hq), dim3(256), 0, s, wb.part_o, wb.part_ml,
                           wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, (uint16_t*)wb.o);
    return hipGetLastError();
}
