// Projection GEMM for many token rows (M > 32): Y[M, N] = A[M, K] . W[N, K]^T on gfx950 MFMA.
//
// A workgroup of WN x WM waves computes a BN (features) x BM (tokens) tile; wave (wn, wm) owns a
// (BN/WN) x (BM/WM) sub-tile held as FT x TT accumulators of v_mfma_f32_16x16x32_bf16 (A operand
// = W rows, B operand = token rows; lane (r, g) holds features 4g..4g+3 of token r of each block).
// K advances 64 at a time through two LDS buffers: while the waves multiply out of one buffer,
// the next stage sits in registers on its way to the other and the stage after that is being
// fetched from HBM, so there is one barrier per stage; the column-tile loop splits each stage
// into two MFMA halves around the barrier so that every LDS read and write overlaps multiplies.  Eight waves share a tile, two per SIMD,
// so one wave's LDS and MFMA latencies hide behind the other's work.  Every epilogue runs from
// registers:
//   QKV     the wave's features are whole heads, a rotation pair (i, i + d/2) sits in the same
//           lane (blocks fb and fb + d/32), RoPE from the per-row (cos, sin) table; q to the
//           workspace, k to its cache row, v to the dim-major cache;
//   SWIGLU  the wave's first FT/2 blocks are gate rows and the last FT/2 the matching up rows;
//   ARGMAX  per-token max over the wave's features (lane values, then the 4 lanes of a token),
//           merged over the WN waves through LDS into one (max, index) slot per column tile;
//   PARTIAL fp32 partial sums of one K slice, 16 bytes per lane store.
// Workgroups are dealt to XCDs round-robin; the unit order gives each XCD a contiguous run, and
// consecutive units are the row tiles (then K slices) of one column tile, so they share its W in L2.
//
// Balanced LM head (BAL): the vocabulary is cut into one contiguous range of 16-row blocks per
// CU instead of BN-row column tiles (594 tiles of 256 rows on 256 CUs would run 3 rounds with
// the last one 30 % full).  A workgroup walks its range in chunks of BN rows with the load
// pipeline running on across chunk boundaries; a wave whose rows of a chunk all lie past the
// range end skips its multiplies (the waves of one feature half sit on different SIMDs, so the
// short last chunk costs about half a chunk).  Each chunk leaves one (max, index) slot per row.
#include <algorithm>

#include "cad_device.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK64 = 64;
// column tiles read their operands through buffer resources of byte offsets: every operand must
// stay below this size
constexpr size_t kPipeMaxBytes = 0x7FFFFFF0u;
constexpr int BAL_MAX_CHUNKS = 4;
// register stages of the balanced LM head: 3 for 64-token tiles, 2 for 128 (measured; the
// column-tile schedule uses 2 and 1)
constexpr int BAL_RS64 = 3, BAL_RS128 = 2;

// chunks of BN rows in the longest of G balanced ranges over N rows (ranges are whole 16-row blocks)
__host__ __device__ inline int bal_chunks(int N, int G, int BN) {
    const int NB = (N + 15) / 16, per = (NB + G - 1) / G;
    return (per * 16 + BN - 1) / BN;
}

template <int KIND, int BN, int BM, int WN, int WM, int BK>
struct BigCfg {
    static constexpr int LDK = BK;                            // LDS row pitch (XOR-swizzled chunks)
    static constexpr int WTN = BN / WN, WTM = BM / WM;        // wave tile (features, tokens)
    static constexpr int FT = WTN / 16, TT = WTM / 16;
    static constexpr int NT = WN * WM * 64;                   // threads
    static constexpr int WCH = BN * (BK / 8) / NT;            // 16-byte W chunks per thread per stage
    static constexpr int ACH = BM * (BK / 8) / NT;            // 16-byte A chunks per thread per stage
    static constexpr int STAGE = (BN + BM) * LDK;             // elements per LDS stage
    static constexpr size_t SMEM = (size_t)2 * STAGE * sizeof(uint16_t);
};

// W row of tile row tr (0..BN-1) of column tile nt.  SwiGLU: within each wave's WTN rows the
// first half are gate rows and the second half the matching up rows.
template <int KIND, int BN, int WTN>
__device__ __forceinline__ int big_w_row(int tr, int nt, int N, int ffn, bool& valid) {
    if constexpr (KIND == EPI_SWIGLU) {
        const int wn = tr / WTN, f = tr % WTN, half = WTN / 2;
        const int F = nt * (BN / 2) + wn * half + (f % half);
        valid = F < ffn;
        return f < half ? F : ffn + F;
    } else {
        const int r = nt * BN + tr;
        valid = r < N;
        return r;
    }
}

__device__ __forceinline__ int xcd_unit(int bid, int grid) { return (bid % 8) * (grid / 8) + bid / 8; }

// QKV epilogue of one wave: blocks ft with (ft mod 2*HALF) < HALF hold first-half dims of a head,
// their rotation partners sit in block ft + HALF of the same lane.
template <int FT, int TT, int HALF>
__device__ __forceinline__ void qkv_epilogue(const f32x4_t (&acc)[FT][TT], const EpiParams& p, int t0, int fbase,
                                             int M, int N, int l16, int g4) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int tok = t0 + tt * 16 + l16;
        if (tok >= M) continue;
        const int b = tok / p.Nq, it = tok % p.Nq;
        if (!seq_ok(p.len_snap, b, p.Nq, p.cap)) continue;
        const size_t slot = (size_t)p.len_snap[b] + it;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
            if ((ft % (2 * HALF)) >= HALF) continue;         // handled with its first-half partner
            const int n1 = fbase + ft * 16 + g4 * 4;         // feature of element 0 (first half)
            if (n1 >= N) continue;
            const int head = n1 / p.d + p.head_off, i0 = n1 % p.d;
            const f32x4_t x1 = acc[ft][tt], x2 = acc[ft + HALF][tt];
            if (head >= p.Hq + p.Hkv) {                      // V: dim-major cache, stored unrotated
                uint16_t* vp = (uint16_t*)p.vc +
                               (((size_t)b * p.Hkv + (head - p.Hq - p.Hkv)) * p.d + i0) * p.cap + slot;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vp[(size_t)i * p.cap] = f32_to_bf16(x1[i]);
                    vp[(size_t)(i + p.d / 2) * p.cap] = f32_to_bf16(x2[i]);
                }
                continue;
            }
            const float2* cs = p.rope_cs + (size_t)tok * (p.d / 2) + i0;
            f32x4_t y1, y2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float2 t = cs[i];
                y1[i] = x1[i] * t.x - x2[i] * t.y;
                y2[i] = x2[i] * t.x + x1[i] * t.y;
            }
            uint16_t* dst = head < p.Hq
                                ? (uint16_t*)p.q_out + ((size_t)tok * p.Hq + head) * p.d
                                : (uint16_t*)p.kc + (((size_t)b * p.Hkv + (head - p.Hq)) * p.cap + slot) * p.d;
            st4(dst + i0, y1);
            st4(dst + i0 + p.d / 2, y2);
        }
    }
}

// Epilogue of one BN x BM column tile from the accumulators: wave (wn, wm)
// holds features wn*WTN + ft*16 + 4*g4 + i of tokens m0 + wm*WTM + tt*16 + l16.
template <int KIND, int BN, int BM, int WN, int WM, int FT, int TT>
__device__ __forceinline__ void big_epilogue(const f32x4_t (&acc)[FT][TT], const EpiParams& p, int M, int N,
                                                int ffn, int m0, int nt, int ks, int tid, int wn, int wm, int l16,
                                                int g4) {
    constexpr int WTN = BN / WN, WTM = BM / WM, NT = WN * WM * 64;
    const int fbase = nt * BN + wn * WTN;                 // first feature (plain layouts)
    if constexpr (KIND == EPI_PARTIAL) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int tok = m0 + wm * WTM + tt * 16 + l16;
            if (tok >= M) continue;
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                const int n = fbase + ft * 16 + g4 * 4;
                if (n < N) *(f32x4_t*)(p.part + ((size_t)ks * M + tok) * N + n) = acc[ft][tt];
            }
        }
    } else if constexpr (KIND == EPI_SWIGLU) {
        constexpr int H = FT / 2;
        const int F0 = nt * (BN / 2) + wn * (WTN / 2);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int tok = m0 + wm * WTM + tt * 16 + l16;
            if (tok >= M || !seq_ok(p.len_snap, tok / p.Nq, p.Nq, p.cap)) continue;
#pragma unroll
            for (int ft = 0; ft < H; ++ft) {
                const int F = F0 + ft * 16 + g4 * 4;
                if (F >= ffn) continue;
                f32x4_t a;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float g = acc[ft][tt][i];
                    a[i] = g / (1.0f + __expf(-g)) * acc[ft + H][tt][i];
                }
                st4((uint16_t*)p.act + (size_t)tok * ffn + F, a);
            }
        }
    } else if constexpr (KIND == EPI_QKV) {
        // the pair offset d/32 (blocks) must be a compile-time index into acc
        if (p.d == 128) qkv_epilogue<FT, TT, 4>(acc, p, m0 + wm * WTM, fbase, M, N, l16, g4);
        else if (p.d == 64) qkv_epilogue<FT, TT, 2>(acc, p, m0 + wm * WTM, fbase, M, N, l16, g4);
        else qkv_epilogue<FT, TT, 1>(acc, p, m0 + wm * WTM, fbase, M, N, l16, g4);
    } else if constexpr (KIND == EPI_SAMPLE) {
        // per row: Gumbel-perturbed maxima and the log-sum-exp over this tile's ids, merged over
        // the lane groups of a wave, then over the WN waves that share the rows
        __shared__ float4 sred[WN][BM][2];
        // wave-uniform: this wave's columns all inside the vocabulary and no debug logits.  Then
        // every row is scanned without per-value tests (a row past M takes row 0's draft and
        // position; its state is never stored).
        const bool plain = !p.logits && fbase + WTN <= N;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int tok = m0 + wm * WTM + tt * 16 + l16;
            SampleState st;
            sample_init(st);
            if (plain) {
                const SampleRow sr = sample_row(p, tok < M ? tok : 0);
#pragma unroll
                for (int ft = 0; ft < FT; ++ft) {
                    const int n0 = fbase + ft * 16 + g4 * 4;
                    const uint4 w = sample_bits(p, sr, n0);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sample_add(st, acc[ft][tt][i] * p.inv_temp, gumbel(ws[i]), n0 + i, sr.draft);
                }
            } else if (tok < M) {
                const SampleRow sr = sample_row(p, tok);
#pragma unroll
                for (int ft = 0; ft < FT; ++ft) {
                    const int n0 = fbase + ft * 16 + g4 * 4;
                    if (n0 >= N) continue;
                    const uint4 w = sample_bits(p, sr, n0);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n0 + i < N) sample_add(st, acc[ft][tt][i] * p.inv_temp, gumbel(ws[i]), n0 + i, sr.draft);
                }
                if (p.logits)
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int n = fbase + ft * 16 + g4 * 4 + i;
                            if (n < N) p.logits[(size_t)tok * N + n] = acc[ft][tt][i];
                        }
            }
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) sample_merge(st, sample_shfl_xor(st, o));
            if (g4 == 0) sample_store(&sred[wn][wm * WTM + tt * 16 + l16][0], st);
            // one token tile's sampling state live at a time (the 256-row tile fits its registers)
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        for (int r = tid; r < BM; r += NT) {
            const int tok = m0 + r;
            if (tok >= M) continue;
            SampleState st = sample_load(&sred[0][r][0]);
#pragma unroll
            for (int w = 1; w < WN; ++w) sample_merge(st, sample_load(&sred[w][r][0]));
            sample_store(p.samp_part + ((size_t)tok * p.amax_slots + nt) * 2, st);
        }
    } else {                                                 // EPI_ARGMAX
        __shared__ float2 red[WN][BM];
        __shared__ float rsec[WN][BM];                         // runner-up values (top-2 gap asked)
        const bool top2 = p.amax_sec != nullptr;
        // wave-uniform: this wave's columns all lie inside the vocabulary and no debug output is
        // asked for.  Then each lane scans its values with one compare and two selects apiece and
        // no branches (rows past M are scanned too; their results are never stored).  The general
        // scan below costs several times that in branches per value, which at 128 values per lane
        // weighed as much as a fifth of the whole launch.
        const bool plain = !top2 && !p.logits && fbase + WTN <= N;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int tok = m0 + wm * WTM + tt * 16 + l16;
            float best = -INFINITY, second = -INFINITY;
            int bi = 0x7fffffff;
            if (plain) {
                int off = -1;                                  // first column of the maximum
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = acc[ft][tt][i];
                        if (v > best) { best = v; off = ft * 16 + i; }
                    }
                if (off >= 0) bi = fbase + g4 * 4 + off;
            } else if (tok < M) {
#pragma unroll
                for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = fbase + ft * 16 + g4 * 4 + i;       // increasing along the lane
                        if (n < N) {
                            const float v = acc[ft][tt][i];
                            if (top2) second = fmaxf(second, fminf(best, v));
                            if (v > best) { best = v; bi = n; }
                            if (p.logits) p.logits[(size_t)tok * N + n] = v;
                        }
                    }
            }
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float v2 = __shfl_xor(best, o, 64);
                const int i2 = __shfl_xor(bi, o, 64);
                if (top2) second = second_merge(best, second, v2, __shfl_xor(second, o, 64));
                argmax_merge(best, bi, v2, i2);
            }
            if (g4 == 0) {
                red[wn][wm * WTM + tt * 16 + l16] = make_float2(best, __int_as_float(bi));
                if (top2) rsec[wn][wm * WTM + tt * 16 + l16] = second;
            }
        }
        __syncthreads();
        for (int r = tid; r < BM; r += NT) {
            const int tok = m0 + r;
            if (tok >= M || !seq_ok(p.len_snap, tok / p.Nq, p.Nq, p.cap)) continue;
            float best = red[0][r].x, second = top2 ? rsec[0][r] : -INFINITY;
            int bi = __float_as_int(red[0][r].y);
#pragma unroll
            for (int w = 1; w < WN; ++w) {
                if (top2) second = second_merge(best, second, red[w][r].x, rsec[w][r]);
                argmax_merge(best, bi, red[w][r].x, __float_as_int(red[w][r].y));
            }
            p.amax_part[(size_t)tok * p.amax_slots + nt] = make_float2(best, __int_as_float(bi));
            if (top2) p.amax_sec[(size_t)tok * p.amax_slots + nt] = second;
        }
    }
}

// BAL: 0 = column tiles, 1 = balanced ranges, 2 = balanced ranges with the debug outputs (logits
// and/or the runner-up values of the top-2 gap)
template <int KIND, int BN, int BM, int WN, int WM, int BK, int RS, int BAL>
__global__ __launch_bounds__(WN * WM * 64) void k_gemm_big(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                     int M, int N, int K, int nmt, int nnt, int S, int ffn,
                                                     EpiParams p) {
    using C = BigCfg<KIND, BN, BM, WN, WM, BK>;
    constexpr int LDK = C::LDK;
    constexpr int FT = C::FT, TT = C::TT, WCH = C::WCH, ACH = C::ACH, NT = C::NT;
    static_assert(BAL || BK == 64, "the column-tile pipeline takes K steps of 64 (two MFMA halves)");
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];   // 2 stages of [BN + BM][LDK]

    const int total = nmt * nnt * S;
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    if (unit >= total) return;
    const int ks = unit % S, tile = unit / S;
    const int mt = tile % nmt, nt = tile / nmt;
    const int m0 = mt * BM;
    const int kbeg = ks * p.k_slice, kend = min(K, kbeg + p.k_slice);
    const int nk = (kend - kbeg + BK - 1) / BK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // (balanced ranges: the waves of one wn sit on different SIMDs, so a chunk whose second half
    // is past the range end still keeps every SIMD busy)
    const int wn = BAL ? wave / WM : wave % WN, wm = BAL ? wave % WM : wave / WN;
    const int l16 = lane & 15, g4 = lane >> 4;

    // per-thread global sources as 32-bit element offsets (row base + chunk offset); invalid rows
    // read row 0 and are zeroed.  (Every operand here has fewer than 2^31 elements.)
    uint32_t woff[WCH], aoff[ACH];
    uint32_t wmask = 0, amask = 0;
#pragma unroll
    for (int c = 0; c < WCH; ++c) {
        const int ch = tid + c * NT, tr = ch / (BK / 8);
        bool v;
        const int r = big_w_row<KIND, BN, C::WTN>(tr, nt, N, ffn, v);
        wmask |= (uint32_t)v << c;
        woff[c] = (uint32_t)(v ? r : 0) * (uint32_t)K + (ch % (BK / 8)) * 8;
    }
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int ch = tid + c * NT, r = ch / (BK / 8);
        const bool v = m0 + r < M;
        amask |= (uint32_t)v << c;
        aoff[c] = (uint32_t)(v ? m0 + r : 0) * (uint32_t)K + (ch % (BK / 8)) * 8;
    }
    const int kchunk = (tid % (BK / 8)) * 8;                  // same k offset for every chunk of a thread
    // A stage of the balanced schedule in registers: raw loads plus their validity bits.  Every
    // load is unconditional from a valid address (no load sits in a branch, so the wait counts stay
    // exact) and the masking happens when the stage is written to LDS, so the loads of a stage
    // stay in flight until then.
    struct Stage { uint4 w[WCH], a[ACH]; uint32_t wok, aok; };
    // 16-byte chunk position of chunk c of tile row r: the chunk index XOR the row's low three
    // bits, so the 16 rows an MFMA fragment read touches spread over every bank group (rows are
    // 16-aligned in every read, so r mod 16 is all the swizzle needs)
    auto sw = [](int r, int c) { return c ^ (r & 7); };
    auto masked = [](uint4 t, uint32_t ok) {
        const uint32_t m = 0u - ok;
        return make_uint4(t.x & m, t.y & m, t.z & m, t.w & m);
    };
    auto store_lds = [&](int buf, const Stage& r) {
        uint16_t* Ws = smem + buf * C::STAGE;
        uint16_t* As = Ws + BN * LDK;
#pragma unroll
        for (int c = 0; c < WCH; ++c) {
            const int ch = tid + c * NT;
            *(uint4*)(Ws + (ch / (BK / 8)) * LDK + sw(ch / (BK / 8), ch % (BK / 8)) * 8) = masked(r.w[c], (r.wok >> c) & 1);
        }
#pragma unroll
        for (int c = 0; c < ACH; ++c) {
            const int ch = tid + c * NT;
            *(uint4*)(As + (ch / (BK / 8)) * LDK + sw(ch / (BK / 8), ch % (BK / 8)) * 8) = masked(r.a[c], (r.aok >> c) & 1);
        }
    };

    f32x4_t acc[FT][TT];
#pragma unroll
    for (int i = 0; i < FT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const uint16_t* Ws = smem + buf * C::STAGE;
        const uint16_t* As = Ws + BN * LDK;
        // the compiler's single-wave small-GEMM interleave of LDS reads and MFMAs (measured 1-2 %
        // faster than the multi-wave one on the 256 x 256 and 256 x 128 tiles, and than none)
        __builtin_amdgcn_iglp_opt(1);
#pragma unroll
        for (int kq = 0; kq < BK / 32; ++kq) {
            bf16x8_t af[FT], bfr[TT];
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
                af[ft] = *(const bf16x8_t*)(Ws + (wn * C::WTN + ft * 16 + l16) * LDK + sw(l16, kq * 4 + g4) * 8);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                bfr[tt] = *(const bf16x8_t*)(As + (wm * C::WTM + tt * 16 + l16) * LDK + sw(l16, kq * 4 + g4) * 8);
#pragma unroll
            for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[ft][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ft], bfr[tt], acc[ft][tt], 0, 0, 0);
        }
    };

    // Balanced schedule: RS register stages in a ring.  Stage kt is loaded into slot kt % RS, RS
    // stages ahead, and at step kt written to LDS buffer kt & 1, then (after the barrier)
    // multiplied.  Buffer kt & 1 was last read at step kt - 2, and every wave has passed step
    // kt - 1's barrier since, so one barrier per step suffices.  The loop is unrolled over a
    // multiple of RS and of 2 so every slot and buffer index is a constant and the oldest loads
    // always sit in the slot written next; loads are issued unconditionally (a stage past the
    // slice reads valid addresses and is masked to zero), because a load inside a branch makes
    // the compiler's wait counts at the join conservative and drains the pipeline before every
    // LDS write.

    constexpr int UNR = RS % 2 ? 2 * RS : RS;
    if constexpr (BAL) {
        // range nt of nnt: vocabulary rows [r0, r1), chunk c = rows r0 + c*BN + (0..BN-1)
        static_assert(KIND == EPI_ARGMAX, "balanced ranges are an LM-head schedule");
        __shared__ float2 bred[BAL_MAX_CHUNKS][WN][BM];
        __shared__ float bsec[BAL == 2 ? BAL_MAX_CHUNKS : 1][WN][BM];   // runner-up values (debug form)
        const int NB = (N + 15) >> 4;
        const int r0 = (int)((long long)nt * NB / nnt) * 16;
        const int r1 = min(N, (int)((long long)(nt + 1) * NB / nnt) * 16);
        const int nch = (r1 - r0 + BN - 1) / BN;
        const int cpw = bal_chunks(N, nnt, BN);
        const int T = nch * nk;
        const int wn_s = __builtin_amdgcn_readfirstlane(wn);               // wave-uniform: scalar branches
        // W chunk c of this thread: tile row tid / (BK/8) + c * NT / (BK/8), column kchunk
        static_assert(NT % (BK / 8) == 0, "every W chunk of a thread has the same column");
        const int wtr0 = tid / (BK / 8);
        // global step t = chunk t / nk, K step t % nk; steps past the last chunk read valid
        // addresses and are masked like rows past the range end
        auto load_bal = [&](int t, Stage& r) {
            const int cc = t / nk;
            const int k0 = kbeg + (t - cc * nk) * BK;
            const int rb = r0 + cc * BN;
            const bool kin = k0 + kchunk < kend;
            const int row0 = rb + wtr0;
            uint32_t wok = 0;
#pragma unroll
            for (int c = 0; c < WCH; ++c) wok |= (uint32_t)(kin && row0 + c * (NT / (BK / 8)) < r1) << c;
            r.wok = wok;
            r.aok = kin ? amask : 0u;
#pragma unroll
            for (int c = 0; c < WCH; ++c) {
                const bool ok = (wok >> c) & 1;
                const uint32_t off = (uint32_t)(row0 + c * (NT / (BK / 8))) * (uint32_t)K + (uint32_t)k0;
                r.w[c] = *(const uint4*)(W + (ok ? off : 0u) + kchunk);
                if constexpr (RS > 1) __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int c = 0; c < ACH; ++c) {
                r.a[c] = *(const uint4*)(A + aoff[c] + (((r.aok >> c) & 1) ? k0 : 0));
                if constexpr (RS > 1) __builtin_amdgcn_sched_barrier(0);
            }
        };
        // per-chunk (max, lowest index) of each token over this wave's rows, into LDS only (no
        // global store inside the K loop but the debug logits, which have an instantiation of
        // their own)
        auto chunk_argmax = [&](int cc) {
            const int rb = r0 + cc * BN;
            // wave-uniform: all of this wave's rows of the chunk lie inside the range (and no debug
            // output): the branch-free scan of the column-tile epilogue
            const bool plain = BAL == 1 && rb + (wn_s + 1) * C::WTN <= r1;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int tok = m0 + wm * C::WTM + tt * 16 + l16;
                float best = -INFINITY, second = -INFINITY;
                int bi = 0x7fffffff;
                if (plain) {
                    int off = -1;
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = acc[ft][tt][i];
                            if (v > best) { best = v; off = ft * 16 + i; }
                        }
                    if (off >= 0) bi = rb + wn * C::WTN + g4 * 4 + off;
                } else if (tok < M) {
#pragma unroll
                    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int n = rb + wn * C::WTN + ft * 16 + g4 * 4 + i;   // increasing along the lane
                            if (n < r1) {
                                const float v = acc[ft][tt][i];
                                if constexpr (BAL == 2) second = fmaxf(second, fminf(best, v));
                                if (v > best) { best = v; bi = n; }
                                if constexpr (BAL == 2)
                                    if (p.logits) p.logits[(size_t)tok * N + n] = v;
                            }
                        }
                }
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float v2 = __shfl_xor(best, o, 64);
                    const int i2 = __shfl_xor(bi, o, 64);
                    if constexpr (BAL == 2) second = second_merge(best, second, v2, __shfl_xor(second, o, 64));
                    argmax_merge(best, bi, v2, i2);
                }
                if (g4 == 0) {
                    bred[cc][wn][wm * C::WTM + tt * 16 + l16] = make_float2(best, __int_as_float(bi));
                    if constexpr (BAL == 2) bsec[cc][wn][wm * C::WTM + tt * 16 + l16] = second;
                }
            }
        };
        Stage r[RS];
#pragma unroll
        for (int i = 0; i < RS; ++i) load_bal(i, r[i]);
        for (int t0 = 0; t0 < T; t0 += UNR) {
#pragma unroll
            for (int j = 0; j < UNR; ++j) {
                const int t = t0 + j;
                if (t >= T) break;
                store_lds(j & 1, r[j % RS]);
                load_bal(t + RS, r[j % RS]);
                __syncthreads();
                const int cc = t / nk;
                // a wave whose rows all lie past the range end skips the multiply
                if (wn_s * C::WTN < r1 - (r0 + cc * BN)) compute(j & 1);
                if (t - cc * nk == nk - 1) {
                    chunk_argmax(cc);
#pragma unroll
                    for (int a = 0; a < FT; ++a)
#pragma unroll
                        for (int b = 0; b < TT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        __syncthreads();
        // one slot per chunk of every range (cpw per range), empty slots for chunks past its end
        for (int cc = 0; cc < cpw; ++cc)
            for (int rr = tid; rr < BM; rr += NT) {
                const int tok = m0 + rr;
                if (tok >= M || !seq_ok(p.len_snap, tok / p.Nq, p.Nq, p.cap)) continue;
                float best = -INFINITY, second = -INFINITY;
                int bi = 0x7fffffff;
                if (cc < nch)
#pragma unroll
                    for (int w = 0; w < WN; ++w) {
                        if constexpr (BAL == 2) second = second_merge(best, second, bred[cc][w][rr].x, bsec[cc][w][rr]);
                        argmax_merge(best, bi, bred[cc][w][rr].x, __float_as_int(bred[cc][w][rr].y));
                    }
                p.amax_part[(size_t)tok * p.amax_slots + nt * cpw + cc] = make_float2(best, __int_as_float(bi));
                if constexpr (BAL == 2)
                    if (p.amax_sec) p.amax_sec[(size_t)tok * p.amax_slots + nt * cpw + cc] = second;
            }
        return;
    }
    {
        // Column tiles: one register stage, pipelined across the K halves of a step.  Step t
        // multiplies K half 0 out of registers while it reads half 1's fragments from LDS buffer
        // t & 1, writes stage t + 1 to buffer (t + 1) & 1 and fetches stage t + 2; after the
        // step's one barrier it multiplies half 1 while it reads half 0 of step t + 1 from the
        // buffer just written.  Every LDS read and write thus overlaps the multiplies.  Buffer
        // (t + 1) & 1 was last read in step t - 1's first half, before that step's barrier, and
        // buffer t & 1 is written again only after step t's barrier, so one barrier per step is
        // enough.  A fragment register is read again as soon as its last multiply is issued.
        // Global loads go through buffer resources whose range check returns zero, so rows past
        // the operand and K past the slice cost no traffic and need no masking.
        constexpr uint32_t OOB = 0x7FFFFFF0u;           // buffer size; offsets from here read zero
        const auto wres = __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)OOB, 0x00020000);
        const auto ares = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)OOB, 0x00020000);
        uint32_t wb[WCH], ab[ACH];                      // byte offsets at k = 0, OOB for rows outside
#pragma unroll
        for (int c = 0; c < WCH; ++c) wb[c] = ((wmask >> c) & 1) ? 2u * woff[c] : OOB;
#pragma unroll
        for (int c = 0; c < ACH; ++c) ab[c] = ((amask >> c) & 1) ? 2u * aoff[c] : OOB;
        u32x4_t sw_[WCH], sa_[ACH];                     // the stage in flight
        auto fetch = [&](int k0) {
            const uint32_t kb = k0 + kchunk < kend ? 2u * (uint32_t)k0 : OOB;
#pragma unroll
            for (int c = 0; c < WCH; ++c) sw_[c] = __builtin_amdgcn_raw_buffer_load_b128(wres, wb[c] + kb, 0, 0);
#pragma unroll
            for (int c = 0; c < ACH; ++c) sa_[c] = __builtin_amdgcn_raw_buffer_load_b128(ares, ab[c] + kb, 0, 0);
        };
        // this thread's stage chunks: tile row tid / 8 + c * NT / 8, chunk tid % 8; the swizzle
        // depends on the row's low three bits only, the same for every c
        const int srow = tid / (BK / 8), sch = tid % (BK / 8);
        const int soff = srow * LDK + sw(srow, sch) * 8;
        constexpr int RSTEP = NT / (BK / 8) * LDK;      // elements between a thread's chunks
        auto put = [&](uint16_t* Ws, int c) {
            if (c < WCH) *(u32x4_t*)(Ws + soff + c * RSTEP) = sw_[c];
            else *(u32x4_t*)(Ws + BN * LDK + soff + (c - WCH) * RSTEP) = sa_[c - WCH];
        };
        auto rd_a = [&](const uint16_t* Ws, int kq, int ft) {
            return *(const bf16x8_t*)(Ws + (wn * C::WTN + ft * 16 + l16) * LDK + sw(l16, kq * 4 + g4) * 8);
        };
        auto rd_b = [&](const uint16_t* Ws, int kq, int tt) {
            return *(const bf16x8_t*)(Ws + BN * LDK + (wm * C::WTM + tt * 16 + l16) * LDK + sw(l16, kq * 4 + g4) * 8);
        };
        constexpr int NS = WCH + ACH;                   // stage chunks per thread
        bf16x8_t fa[FT], fb0[TT], fb1[TT];              // W fragments; token fragments of the two halves
        // the multiplies of one K half out of fa / fu; fa is refilled from (Rs, rkq) block by block
        // as it frees up and the other half's token fragments go to fn; with STORE the stage is
        // written to Ws and the next one fetched from k0n meanwhile (Rs and Ws are different buffers)
        auto half = [&](const uint16_t* __restrict__ Rs, int rkq, const bf16x8_t(&fu)[TT], bf16x8_t(&fn)[TT],
                        bool store, uint16_t* __restrict__ Ws, int k0n) {
            if (store) {
#pragma unroll
                for (int c = 0; c < NS; ++c) put(Ws, c);
                fetch(k0n);
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[ft][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ft], fu[tt], acc[ft][tt], 0, 0, 0);
                fa[ft] = rd_a(Rs, rkq, ft);
                if (ft < TT) fn[ft] = rd_b(Rs, rkq, ft);
            }
            // issue pattern: per feature block its multiplies with the block's share of stage chunks
            // (write, then refetch of that register) between them, then the block's fragment reads
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                const int c0 = ft * NS / FT, c1 = (ft + 1) * NS / FT;   // stage chunks of this block
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
                    if (store && tt < c1 - c0) {
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);      // LDS write
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // global load
                    }
                }
                if (store)
                    for (int c = TT; c < c1 - c0; ++c) {
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS reads
                if (ft < TT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        };
        // prologue: stage 0 in LDS buffer 0, stage 1 in flight, half 0 of step 0 in registers
        fetch(kbeg);
#pragma unroll
        for (int c = 0; c < NS; ++c) put(smem, c);
        fetch(kbeg + BK);
        __syncthreads();
        // (in the order the loop reads them, so the wait counts at the loop head agree)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
            fa[ft] = rd_a(smem, 0, ft);
            __builtin_amdgcn_sched_barrier(0);
            if (ft < TT) fb0[ft] = rd_b(smem, 0, ft);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int kt = 0; kt < nk; ++kt) {
            uint16_t* cur = smem + (kt & 1) * C::STAGE;
            uint16_t* nxt = smem + ((kt + 1) & 1) * C::STAGE;
            half(cur, 1, fb0, fb1, true, nxt, kbeg + (kt + 2) * BK);
            __syncthreads();
            half(nxt, 0, fb1, fb0, false, nullptr, 0);
        }
        big_epilogue<KIND, BN, BM, WN, WM>(acc, p, M, N, ffn, m0, nt, ks, tid, wn, wm, l16, g4);
    }
}

struct BigPlan { int BN, BM, nmt, nnt, S, k_slice, grid; bool bal; };

template <int KIND, int BN, int BM, int WN, int WM, int BK, int RS, int BAL = 0>
hipError_t go_big(const void* A, const void* W, int M, int N, int K, int ffn, const BigPlan& t, const EpiParams& p,
                  hipStream_t s) {
    auto kern = k_gemm_big<KIND, BN, BM, WN, WM, BK, RS, BAL>;
    constexpr size_t smem = BigCfg<KIND, BN, BM, WN, WM, BK>::SMEM;
    if (!BAL) {
        const size_t wrows = KIND == EPI_SWIGLU ? 2 * (size_t)ffn : (size_t)N;
        if (wrows * K * 2 >= kPipeMaxBytes || (size_t)M * K * 2 >= kPipeMaxBytes) return hipErrorInvalidValue;
    }
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(kern, dim3(t.grid), dim3(WN * WM * 64), smem, s, (const uint16_t*)A, (const uint16_t*)W, M, N, K,
                       t.nmt, t.nnt, t.S, ffn, p);
    return hipGetLastError();
}

}  // namespace

// Tile choice: 256 features per workgroup tile (two waves of 128 across it); 64, 128 or 256
// tokens.  The narrow QKV projection and the K-slice partial projections take 128 x 64 tiles
// (one wave of 128 features, so a QKV wave holds whole heads of up to 128 dims) to spread over
// more workgroups (measured on the 1.5B shape for gate/up: 64-row tiles up to 128 rows, 128-row
// tiles up to 256, 256-row tiles beyond; 192 features wide while one round holds the tiles, else
// 256).
BigPlan big_plan(int kind, int M, int N, int K, int slices) {
    BigPlan t;
    t.BN = 256;
    t.BM = M <= 64 ? 64 : M <= 128 ? 128 : 256;
    // gate/up: 256 x 64 tiles up to 128 rows (more workgroups), 256 x 128 up to 256 rows (at
    // 256 rows one round of 140 workgroups took 35 us, 560 128 x 64 tiles in two rounds 44 us)
    if (kind == EPI_SWIGLU && M <= 128) t.BM = 64;
    if (kind == EPI_SWIGLU && M > 128 && M <= 256) t.BM = 128;
    // beyond 256 rows: 192 x 256 tiles while they fit the CUs in one round (at 512 rows, 188
    // workgroups: 46 us against 52 us for 140 256 x 256 tiles), else 256 x 256 (at 704 rows 282
    // 192-wide tiles would need a second round)
    if (kind == EPI_SWIGLU && M > 256 && (long)((M + 255) / 256) * ((N / 2 + 95) / 96) <= device_cu_count())
        t.BN = 192;
    // 65-256 rows: 192-wide tiles as well while they fit one round (188 workgroups instead of 144
    // on the 1.5B shape: 27.9 -> 24.7 us at 128 rows, 33.3 -> 29.1 us at 256)
    if (kind == EPI_SWIGLU && M <= 256 && (long)((M + t.BM - 1) / t.BM) * ((N / 2 + 95) / 96) <= device_cu_count())
        t.BN = 192;
    if (kind == EPI_QKV || kind == EPI_PARTIAL) {
        // narrow outputs: 128 x 64 tiles give more workgroups (and QKV one head per wave); for the
        // K-slice partials they also mean fewer slices, so less partial traffic for the row
        // kernel that adds them
        t.BN = 128;
        t.BM = 64;
    }
    t.nmt = (M + t.BM - 1) / t.BM;
    t.nnt = kind == EPI_SWIGLU ? (N / 2 + t.BN / 2 - 1) / (t.BN / 2) : (N + t.BN - 1) / t.BN;
    t.S = kind == EPI_PARTIAL ? slices : 1;
    t.k_slice = ((K + t.S - 1) / t.S + BK64 - 1) / BK64 * BK64;
    // (only while the LM head is bound by the weight stream: at 256 rows and more the column
    // tiles' rounds measured faster than balanced ranges)
    t.bal = kind == EPI_ARGMAX && t.BM <= 128;
    if (t.bal) {
        // one range per CU, at least 24 blocks per range (small vocabularies) and at most
        // BAL_MAX_CHUNKS chunks per range
        const int NB = (N + 15) / 16, bpc = t.BN / 16;
        int G = std::min(device_cu_count(), (NB + 23) / 24);
        G = std::max(G, (NB + BAL_MAX_CHUNKS * bpc - 1) / (BAL_MAX_CHUNKS * bpc));
        t.nnt = std::max(G, 1);
    }
    const int total = t.nmt * t.nnt * t.S;
    t.grid = (total + 7) / 8 * 8;
    return t;
}

int big_slots(int kind, int M, int N, int K) {
    const BigPlan t = big_plan(kind, M, N, K, 1);
    return t.bal ? t.nnt * bal_chunks(N, t.nnt, t.BN) : t.nnt;
}

int big_partial_slices(int M, int N, int K, int cus) {
    const BigPlan t = big_plan(EPI_PARTIAL, M, N, K, 1);
    const int tiles = t.nmt * t.nnt;
    // as many slices as two resident workgroups per CU take in one round (the 128 x 64 partial
    // tile runs two per CU): at 512 rows the down projection took 44 us with one per CU, 33 with two
    int S = 2 * cus / tiles;
    const int smax = K / 256 > 1 ? K / 256 : 1;              // at least 256 of K per slice
    return S < 1 ? 1 : (S > smax ? smax : S);
}

template <int KIND>
hipError_t big_dispatch(const void* A, const void* W, int M, int N, int K, int slices, EpiParams p, hipStream_t s) {
    const BigPlan t = big_plan(KIND, M, N, K, slices);
    p.k_slice = t.k_slice;
    const int ffn = KIND == EPI_SWIGLU ? p.ffn : 0;
    if (t.BN == 128) return go_big<KIND, 128, 64, 1, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
    if constexpr (KIND == EPI_SWIGLU)
        if (t.BN == 192) {
            if (t.BM == 64) return go_big<KIND, 192, 64, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
            if (t.BM == 128) return go_big<KIND, 192, 128, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
            return go_big<KIND, 192, 256, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
        }
    if constexpr (KIND == EPI_ARGMAX) {
        // debug outputs (logits, runner-up values) have an instantiation of their own
        const bool dbg = p.logits || p.amax_sec;
        if (t.bal && t.BM == 64)
            return dbg ? go_big<KIND, 256, 64, 2, 4, 64, BAL_RS64, 2>(A, W, M, N, K, ffn, t, p, s)
                       : go_big<KIND, 256, 64, 2, 4, 64, BAL_RS64, 1>(A, W, M, N, K, ffn, t, p, s);
        if (t.bal)
            return dbg ? go_big<KIND, 256, 128, 2, 4, 64, BAL_RS128, 2>(A, W, M, N, K, ffn, t, p, s)
                       : go_big<KIND, 256, 128, 2, 4, 64, BAL_RS128, 1>(A, W, M, N, K, ffn, t, p, s);
    }
    switch (t.BM) {
        case 64: return go_big<KIND, 256, 64, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
        case 128: return go_big<KIND, 256, 128, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
        default: return go_big<KIND, 256, 256, 2, 4, 64, 1>(A, W, M, N, K, ffn, t, p, s);
    }
}

hipError_t launch_big(int kind, const void* A, const void* W, int M, int N, int K, int slices, const EpiParams& p,
                      hipStream_t s) {
    switch (kind) {
        case EPI_QKV: return big_dispatch<EPI_QKV>(A, W, M, N, K, 1, p, s);
        case EPI_SWIGLU: return big_dispatch<EPI_SWIGLU>(A, W, M, N, K, 1, p, s);
        case EPI_ARGMAX: return big_dispatch<EPI_ARGMAX>(A, W, M, N, K, 1, p, s);
        case EPI_SAMPLE: return big_dispatch<EPI_SAMPLE>(A, W, M, N, K, 1, p, s);
        default: return big_dispatch<EPI_PARTIAL>(A, W, M, N, K, slices, p, s);
    }
}
