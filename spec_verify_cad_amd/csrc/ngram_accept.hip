// Integer kernels around the span forward.
//
// k_ngram: prompt-lookup draft search (PLD page, "The n-gram match, precisely"; SwitchSD's
// kappa-gram gate with recency-ranked candidates).  One workgroup of 1024 threads per sequence
// scans the candidate starts newest-first in chunks of 8192 (eight consecutive starts per thread,
// the chunk's token window staged in LDS so the loads are coalesced, and the next chunk's window
// fetched into registers while the current one is compared), ranks the hits of a chunk by a
// block-wide prefix count in descending start order and stops as soon as W hits are known.
//
// k_accept: greedy left-to-right acceptance (PLD page, "Verification in a single parallel
// pass") or the longest validated candidate of a block verify (SwitchSD), then the commit:
// emitted tokens appended to the history, cache length advanced, and in block mode the
// winner's accepted K/V entries moved down to the slots right after the prefix.
#include "cad_device.h"

namespace {

constexpr int NG_NT = 1024;      // threads of the scan workgroup
constexpr int NG_Q = 8;          // candidate starts per thread per chunk
constexpr int CH = NG_NT * NG_Q; // candidate starts per scan chunk
constexpr int MAXN = 64;
constexpr int NG_L = (CH + MAXN + NG_NT - 1) / NG_NT;   // window tokens each thread fetches per chunk

// Suffix lengths n_hi down to n_lo are tried in turn and the hits of the first length that has
// any are kept (n_hi == n_lo: the plain lookup); match_n (nullable) gets that length, 0 if none.
__global__ __launch_bounds__(NG_NT) void k_ngram(const int32_t* __restrict__ ctx, int64_t stride,
                                                 const int32_t* __restrict__ ctx_len, int n_hi, int n_lo, int W,
                                                 int D, int with_current, int32_t* __restrict__ draft,
                                                 int32_t* __restrict__ draft_len, int32_t* __restrict__ match_pos,
                                                 int32_t* __restrict__ match_n) {
    __shared__ int32_t win[CH + MAXN];
    __shared__ int32_t suf[MAXN];
    __shared__ int wsum[NG_NT / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* c = ctx + (size_t)b * stride;
    int len = ctx_len[b];
    len = len < 0 ? 0 : (len > stride ? (int)stride : len);
    const int rowlen = with_current + W * D;
    int32_t* drow = draft + (size_t)b * rowlen;
    for (int e = tid; e < rowlen; e += NG_NT) drow[e] = (e == 0 && with_current) ? (len > 0 ? c[len - 1] : 0) : 0;
    for (int w = tid; w < W; w += NG_NT) {
        draft_len[b * W + w] = 0;
        if (match_pos) match_pos[b * W + w] = -1;
    }
    if (match_n && tid == 0) match_n[b] = 0;
    for (int n = n_hi; n >= n_lo; --n) {
    if (len < n + 1) continue;
    __syncthreads();                                     // the previous length's suffix is no longer read
    for (int k = tid; k < n; k += NG_NT) suf[k] = c[len - n + k];
    // the window of a chunk (starts lo..hi and their n tokens) is fetched into registers one
    // chunk ahead, every load in flight at once; positions before 0 read position 0 and become -1
    int32_t pre[NG_L];
    auto fetch = [&](int lo_) {
#pragma unroll
        for (int i = 0; i < NG_L; ++i) {
            const int e = min(tid + i * NG_NT, CH + n - 2), pos = lo_ + e;
            const int32_t v = c[pos > 0 ? pos : 0];
            pre[i] = pos >= 0 ? v : -1;
        }
    };
    int found = 0;
    fetch(len - n - CH);
    for (int hi = len - n - 1; hi >= 0 && found < W; hi -= CH) {
        const int lo = hi - CH + 1;                      // window covers starts lo..hi and their n tokens
        __syncthreads();                                 // the previous chunk's window is no longer read
#pragma unroll
        for (int i = 0; i < NG_L; ++i) {
            const int e = tid + i * NG_NT;
            if (e < CH + n - 1) win[e] = pre[i];
        }
        fetch(lo - CH);                                  // the next chunk's window, in flight meanwhile
        __syncthreads();
        // thread t takes starts hi - NG_Q*t - q, q < NG_Q (descending in thread order, then in q)
        int hits = 0;
#pragma unroll
        for (int q = 0; q < NG_Q; ++q) {
            const int j = hi - NG_Q * tid - q;
            bool hit = j >= 0;
            for (int k = 0; k < n && hit; ++k) hit = win[j - lo + k] == suf[k];
            hits |= (int)hit << q;
        }
        const int cnt = __popc(hits);
        int incl = cnt;                                  // inclusive scan over the wave's lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = found;
        int total = found;
        for (int w = 0; w < NG_NT / 64; ++w) {
            before += w < wave ? wsum[w] : 0;
            total += wsum[w];
        }
        int rank = before + incl - cnt;
#pragma unroll
        for (int q = 0; q < NG_Q; ++q) {
            if (!((hits >> q) & 1)) continue;
            if (rank < W) {
                const int j = hi - NG_Q * tid - q;
                const int dl = min(D, len - (j + n));
                int32_t* dst = drow + with_current + rank * D;
                for (int e = 0; e < dl; ++e) dst[e] = c[j + n + e];
                draft_len[b * W + rank] = dl;
                if (match_pos) match_pos[b * W + rank] = j;
            }
            ++rank;
        }
        found = total;                                   // the same value in every thread
    }
    if (found > 0) {
        if (match_n && tid == 0) match_n[b] = n;
        return;
    }
    }
}

__global__ __launch_bounds__(256) void k_accept(const int32_t* __restrict__ draft, int with_current,
                                                const int32_t* __restrict__ draft_len, const int32_t* __restrict__ pred,
                                                const int32_t* __restrict__ first_pred, int W, int D, int mode,
                                                int32_t* __restrict__ accepted, int32_t* __restrict__ best_w,
                                                int32_t* __restrict__ emitted, int32_t* __restrict__ n_emitted,
                                                int32_t* __restrict__ ctx, int64_t ctx_stride,
                                                int32_t* __restrict__ ctx_len, int ctx_cap, void* kc, void* vc,
                                                int32_t* __restrict__ kv_len, int32_t* __restrict__ kv_err,
                                                int Hkv, int d, int esz, int cap) {
    __shared__ int sa, sw, sctx, slen, sskip;
    __shared__ int32_t em[65];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int rowlen = with_current + W * D;
    const int32_t* drow = draft + (size_t)b * rowlen + with_current;
    if (tid == 0) {
        int skip = kv_err && kv_err[b] != 0;
        int a_best = 0, w_best = 0;
        if (mode == CAD_MASK_CAUSAL_SPAN) {
            const int32_t* pr = pred + (size_t)b * (1 + D);
            const int dl = min(max(draft_len[b], 0), D);          // a length past D reads no further
            int a = 0;
            while (a < dl && drow[a] == pr[a]) ++a;
            a_best = a;
            for (int e = 0; e < a; ++e) em[e] = drow[e];
            em[a] = pr[a];
        } else {
            const int32_t* pr = pred + (size_t)b * W * D;
            const int fp = first_pred[b];
            for (int w = 0; w < W; ++w) {
                const int dl = min(max(draft_len[b * W + w], 0), D);
                int a = 0;
                while (a < dl && drow[w * D + a] == (a == 0 ? fp : pr[w * D + a - 1])) ++a;
                if (a > a_best) { a_best = a; w_best = w; }
            }
            for (int e = 0; e < a_best; ++e) em[e] = drow[w_best * D + e];
            em[a_best] = a_best == 0 ? fp : pr[w_best * D + a_best - 1];
        }
        const int cl = ctx_len ? ctx_len[b] : 0;
        if (!skip && ctx && (cl < 0 || cl + a_best + 1 > ctx_cap)) {
            skip = 1;
            if (kv_err) kv_err[b] = CAD_ECAPACITY;
        }
        const int kl = kv_len ? kv_len[b] : 0;
        // the verify forward wrote rows kl .. kl+rows-1: refuse a length that could not hold them
        const int rows = mode == CAD_MASK_CAUSAL_SPAN ? 1 + D : W * D;
        if (!skip && kv_len && (kl < 0 || kl + rows > cap)) {
            skip = 1;
            if (kv_err) kv_err[b] = CAD_ECAPACITY;
        }
        sa = a_best; sw = w_best; sctx = cl; sskip = skip;
        slen = kl;
    }
    __syncthreads();
    if (sskip) {
        // a skipped sequence reports nothing accepted and nothing emitted (n_emitted = 0 marks it:
        // a sequence that ran always emits at least one token); its lengths stay unchanged
        for (int e = tid; e <= D; e += 256) emitted[(size_t)b * (D + 1) + e] = 0;
        if (tid == 0) {
            accepted[b] = 0;
            if (best_w) best_w[b] = 0;
            n_emitted[b] = 0;
        }
        return;
    }
    const int a = sa, w = sw;
    for (int e = tid; e <= D; e += 256) emitted[(size_t)b * (D + 1) + e] = e <= a ? em[e] : 0;
    if (ctx)
        for (int e = tid; e <= a; e += 256) ctx[(size_t)b * ctx_stride + sctx + e] = em[e];
    if (mode == CAD_MASK_BLOCK_TRI && kc && w > 0 && a > 0) {
        // move the winner's rows len + w*D + j -> len + j (j < a); source and destination never
        // overlap (w*D >= D >= a).  K rows are whole [d] rows; V is dim-major, so each of its
        // d rows per head moves a elements.
        const int len = slen;
        const int per_row = d * esz / 16;                         // 16-byte chunks per K row
        const int ktotal = Hkv * a * per_row;
        for (int e = tid; e < ktotal; e += 256) {
            const int g = e / (a * per_row), j = (e / per_row) % a, ck = e % per_row;
            uint4* base = (uint4*)kc;
            const size_t head = ((size_t)b * Hkv + g) * cap;
            base[(head + len + j) * per_row + ck] = base[(head + len + (size_t)w * D + j) * per_row + ck];
        }
        const int vtotal = Hkv * d * a;
        for (int e = tid; e < vtotal; e += 256) {
            const int g = e / (d * a), dim = (e / a) % d, j = e % a;
            const size_t row = (((size_t)b * Hkv + g) * d + dim) * cap;
            if (esz == 2)
                ((uint16_t*)vc)[row + len + j] = ((const uint16_t*)vc)[row + len + (size_t)w * D + j];
            else
                ((float*)vc)[row + len + j] = ((const float*)vc)[row + len + (size_t)w * D + j];
        }
    }
    __syncthreads();
    if (tid == 0) {
        accepted[b] = a;
        if (best_w) best_w[b] = w;
        n_emitted[b] = a + 1;
        if (ctx) ctx_len[b] = sctx + a + 1;
        if (kv_len) kv_len[b] = slen + (mode == CAD_MASK_CAUSAL_SPAN ? a + 1 : a);
    }
}

// Block-verify commit of the other layers of a stack: after k_accept has committed the first
// layer (accepted[b] = a*, best_w[b] = w*, kv_len[b] = len + a*; n_emitted[b] = 0 for a skipped
// sequence), the winner's first a* K/V slots of each further layer move from len + w*D + j to
// len + j, exactly as k_accept moved the first layer's.  Grid: (B, layers of this launch).
constexpr int CL_MAX = 16;
struct LayerKV { void* k[CL_MAX]; void* v[CL_MAX]; };
__global__ __launch_bounds__(256) void k_compact_layers(LayerKV lk, const int32_t* __restrict__ accepted,
                                                        const int32_t* __restrict__ best_w,
                                                        const int32_t* __restrict__ n_emitted,
                                                        const int32_t* __restrict__ kv_len, int D, int Hkv, int d,
                                                        int esz, int cap) {
    const int b = blockIdx.x, l = blockIdx.y, tid = threadIdx.x;
    const int a = accepted[b], w = best_w[b];
    if (n_emitted[b] == 0 || a <= 0 || w <= 0) return;
    const int len = kv_len[b] - a;
    if (len < 0 || len + (size_t)(w + 1) * D > (size_t)cap) return;   // not a length k_accept committed
    uint4* kb = (uint4*)lk.k[l];
    const int per_row = d * esz / 16;
    for (int e = tid; e < Hkv * a * per_row; e += 256) {
        const int g = e / (a * per_row), j = (e / per_row) % a, ck = e % per_row;
        const size_t head = ((size_t)b * Hkv + g) * cap;
        kb[(head + len + j) * per_row + ck] = kb[(head + len + (size_t)w * D + j) * per_row + ck];
    }
    for (int e = tid; e < Hkv * d * a; e += 256) {
        const int g = e / (d * a), dim = (e / a) % d, j = e % a;
        const size_t row = (((size_t)b * Hkv + g) * d + dim) * cap;
        if (esz == 2)
            ((uint16_t*)lk.v[l])[row + len + j] = ((const uint16_t*)lk.v[l])[row + len + (size_t)w * D + j];
        else
            ((float*)lk.v[l])[row + len + j] = ((const float*)lk.v[l])[row + len + (size_t)w * D + j];
    }
}

}  // namespace

hipError_t launch_compact_layers(const cad_kv_desc* kvs, int n_layers, int B, int D, const int32_t* accepted,
                                 const int32_t* best_w, const int32_t* n_emitted, hipStream_t s) {
    const int esz = kvs[0].dtype == CAD_DTYPE_F32 ? 4 : 2;
    for (int l0 = 1; l0 < n_layers; l0 += CL_MAX) {
        LayerKV lk;
        const int n = n_layers - l0 < CL_MAX ? n_layers - l0 : CL_MAX;
        for (int i = 0; i < CL_MAX; ++i) {
            lk.k[i] = i < n ? kvs[l0 + i].k : nullptr;
            lk.v[i] = i < n ? kvs[l0 + i].v : nullptr;
        }
        hipLaunchKernelGGL(k_compact_layers, dim3(B, n), dim3(256), 0, s, lk, accepted, best_w, n_emitted, kvs[0].len,
                           D, kvs[0].n_kv_heads, kvs[0].head_dim, esz, kvs[0].cap);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_ngram(const int32_t* ctx, int64_t stride, const int32_t* ctx_len, int B, int n_hi, int n_lo,
                        int W, int D, int with_current, int32_t* draft, int32_t* draft_len, int32_t* match_pos,
                        int32_t* match_n, hipStream_t s) {
    hipLaunchKernelGGL(k_ngram, dim3(B), dim3(NG_NT), 0, s, ctx, stride, ctx_len, n_hi, n_lo, W, D, with_current,
                       draft, draft_len, match_pos, match_n);
    return hipGetLastError();
}

hipError_t launch_accept(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                         const int32_t* first_pred, int B, int W, int D, int mode, int32_t* accepted,
                         int32_t* best_w, int32_t* emitted, int32_t* n_emitted, int32_t* ctx, int64_t ctx_stride,
                         int32_t* ctx_len, int ctx_cap, const cad_kv_desc* kv, hipStream_t s) {
    const int esz = kv && kv->dtype == CAD_DTYPE_F32 ? 4 : 2;
    hipLaunchKernelGGL(k_accept, dim3(B), dim3(256), 0, s, draft, with_current, draft_len, pred, first_pred, W, D,
                       mode, accepted, best_w, emitted, n_emitted, ctx, ctx_stride, ctx_len, ctx_cap,
                       kv ? kv->k : nullptr, kv ? kv->v : nullptr, kv ? kv->len : nullptr, kv ? kv->err : nullptr,
                       kv ? kv->n_kv_heads : 0, kv ? kv->head_dim : 0, esz, kv ? kv->cap : 0);
    return hipGetLastError();
}
