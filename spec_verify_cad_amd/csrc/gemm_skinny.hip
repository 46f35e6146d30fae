// Weight-streaming projection GEMM for few token rows (M <= 64): Y[M, N] = A[M, K] . W[N, K]^T.
//
// With a handful of rows every weight is used by at most 32 multiply-adds, so the kernel is a
// pure stream of W from HBM: nothing of W goes through LDS.  A unit of work is one 16-feature
// tile of W over one K slice; the NW waves of a workgroup split the slice and each lane loads
// 32 contiguous bytes of a W row per 64-element super-step (the 4 lanes of a row cover one
// 128-byte line).  The MFMA k-index is permuted to match (v_mfma_f32_16x16x32_bf16 sums over
// k, so A and B only have to agree on the order): lane (r, g) feeds W[r][s*64 + 16g + 8j .. +8]
// in sub-step j, and the token operand is loaded from A with the same offsets.  Workgroups are
// persistent and walk the units with a grid stride that is a multiple of the slice count, so a
// workgroup always works on the same K slice: its token fragments are loaded into registers
// once, and only W streams.  The LM head, whose workgroups walk many units, keeps two W buffers:
// the next unit's loads are in flight while the current one is multiplied and finished.  The
// waves' partial tiles are
// summed through LDS and the wave that owns a 16-token tile runs the epilogue from registers:
// lane (r, g) then holds features 4g..4g+3 of token r.
//
// Feature tiles: QKV tiles hold 8 rotation pairs of one head (dims pb*8 + 0..7 and their
// partners d/2 + pb*8 + 0..7), so RoPE needs one lane exchange; SwiGLU tiles hold 8 gate rows
// and the 8 matching up rows; LM-head and partial tiles are 16 consecutive rows.
#include "cad_device.h"

namespace {

template <int KIND>
__device__ __forceinline__ int w_row(int tile, int f, int N, const EpiParams& p, bool& valid) {
    if constexpr (KIND == EPI_QKV) {
        const int tph = p.d / 16, hl = tile / tph, pb = tile % tph;
        valid = true;
        return hl * p.d + (f < 8 ? pb * 8 + f : p.d / 2 + pb * 8 + (f - 8));
    } else if constexpr (KIND == EPI_SWIGLU) {
        const int F = tile * 8 + (f & 7);
        valid = F < p.ffn;
        return f < 8 ? F : p.ffn + F;
    } else {
        const int r = tile * 16 + f;
        valid = r < N;
        return r;
    }
}

template <int KIND, int TT, int SSW, int NW, bool DB>
__global__ __launch_bounds__(NW * 64) void k_skinny(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                    int M, int N, int K, int ntiles, int S, EpiParams p) {
    __shared__ f32x4_t red[NW][TT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    constexpr int KS = NW * SSW * 64;                 // K elements of one slice
    const int units = ntiles * S, G = gridDim.x;
    int u = blockIdx.x;
    if (u >= units) return;
    // the grid is a multiple of S, so every unit of this workgroup has the same K slice and
    // the token fragments are loaded once
    const int ks = u % S;
    const int kb = ks * KS + wave * SSW * 64 + g4 * 16;
    uint4 xf[TT][SSW][2];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int tok = tt * 16 + l16;
        const uint16_t* xrow = A + (size_t)(tok < M ? tok : 0) * K;
#pragma unroll
        for (int s = 0; s < SSW; ++s)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int k = kb + s * 64 + j * 8;
                const bool ok = tok < M && k < K;
                const uint4 t = *(const uint4*)(xrow + (ok ? k : 0));   // valid address, zeroed if masked
                xf[tt][s][j] = ok ? t : make_uint4(0, 0, 0, 0);
            }
    }

    // W fragments of one unit.  Every load is unconditional from a valid address: a row past N
    // reads row 0 and a column past K column 0.  Their values are not masked: a column past K
    // meets a zero token fragment (finite weights times zero add nothing) and a row past N is never
    // stored, so no load sits in a branch and the wait counts stay exact across units.
    auto load_w = [&](int uu, uint4 (&wf)[SSW][2]) {
        bool wv;
        const int wr = w_row<KIND>(uu / S, l16, N, p, wv);
        const uint16_t* wrow = W + (size_t)(wv ? wr : 0) * K;
#pragma unroll
        for (int s = 0; s < SSW; ++s)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int k = kb + s * 64 + j * 8;
                wf[s][j] = *(const uint4*)(wrow + (k < K ? k : 0));
            }
        // every load of the unit is issued before anything that uses one (left to itself the
        // scheduler interleaves them with the multiplies and keeps two in flight)
        __builtin_amdgcn_sched_barrier(0);
    };
    // the epilogue row of this lane and whether its sequence runs (read once, not per unit)
    const int my_tok = wave * 16 + l16;
    const bool my_live = wave < TT && my_tok < M && seq_ok(p.len_snap, my_tok / p.Nq, p.Nq, p.cap);

    float best = -INFINITY;                           // LM head: this lane's running (max, index)
    int bidx = 0x7fffffff;
    float second = -INFINITY;                         // and runner-up value
    SampleState sst;                                  // sampled LM head: this lane's running state
    SampleRow srow;
    if constexpr (KIND == EPI_SAMPLE) {
        sample_init(sst);
        const int tok = wave * 16 + l16;
        srow = sample_row(p, tok < M && wave < TT ? tok : 0);
    }

    auto compute = [&](int uu, const uint4 (&wf)[SSW][2]) {
        const int tile = uu / S;
        f32x4_t acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SSW; ++s)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)&wf[s][j],
                                                                      *(const bf16x8_t*)&xf[tt][s][j], acc[tt], 0, 0, 0);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) red[wave][tt][lane] = acc[tt];
        __syncthreads();
        if (wave < TT) {
            f32x4_t c = red[0][wave][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) c += red[w][wave][lane];
            const int tok = my_tok;
            const bool live = my_live;
            if constexpr (KIND == EPI_PARTIAL) {
                const int n = tile * 16 + g4 * 4;
                if (tok < M && n < N) *(f32x4_t*)(p.part + ((size_t)ks * M + tok) * N + n) = c;
            } else if constexpr (KIND == EPI_ARGMAX) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = tile * 16 + g4 * 4 + i;
                    if (live && n < N) {
                        second = fmaxf(second, fminf(best, c[i]));
                        if (c[i] > best) { best = c[i]; bidx = n; }   // n increases along a lane
                        if (p.logits) p.logits[(size_t)tok * N + n] = c[i];
                    }
                }
            } else if constexpr (KIND == EPI_SAMPLE) {
                if (live) {
                    const int n0 = tile * 16 + g4 * 4;
                    const uint4 w = sample_bits(p, srow, n0);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = n0 + i;
                        if (n < N) {
                            sample_add(sst, c[i] * p.inv_temp, gumbel(ws[i]), n, srow.draft);
                            if (p.logits) p.logits[(size_t)tok * N + n] = c[i];
                        }
                    }
                }
            } else {
                f32x4_t o;                                   // partner features (lane g4 ^ 2)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(c[i], 32, 64);
                if constexpr (KIND == EPI_SWIGLU) {
                    const int F = tile * 8 + g4 * 4;
                    if (live && g4 < 2 && F < p.ffn) {
                        f32x4_t a;
#pragma unroll
                        for (int i = 0; i < 4; ++i) a[i] = c[i] / (1.0f + __expf(-c[i])) * o[i];
                        st4((uint16_t*)p.act + (size_t)tok * p.ffn + F, a);
                    }
                } else {                                     // EPI_QKV
                    if (live) {
                        const int tph = p.d / 16, half = p.d / 2;
                        const int head = tile / tph + p.head_off, pb = tile % tph;
                        const bool first = g4 < 2;
                        const int i0 = pb * 8 + (g4 & 1) * 4;        // pair index of element 0
                        const int dim = first ? i0 : half + i0;
                        const int b = tok / p.Nq, it = tok % p.Nq;
                        const size_t slot = (size_t)p.len_snap[b] + it;
                        f32x4_t y;
                        if (head >= p.Hq + p.Hkv) {
                            y = c;
                        } else {
                            const float2* cs = p.rope_cs + (size_t)tok * half + i0;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float2 t = cs[i];
                                y[i] = first ? c[i] * t.x - o[i] * t.y : c[i] * t.x + o[i] * t.y;
                            }
                        }
                        if (head < p.Hq) {
                            st4((uint16_t*)p.q_out + ((size_t)tok * p.Hq + head) * p.d + dim, y);
                        } else if (head < p.Hq + p.Hkv) {
                            st4((uint16_t*)p.kc + (((size_t)b * p.Hkv + (head - p.Hq)) * p.cap + slot) * p.d + dim, y);
                        } else {                                 // V cache is dim-major [d][cap]
                            uint16_t* vp = (uint16_t*)p.vc +
                                           (((size_t)b * p.Hkv + (head - p.Hq - p.Hkv)) * p.d + dim) * p.cap + slot;
#pragma unroll
                            for (int i = 0; i < 4; ++i) vp[(size_t)i * p.cap] = f32_to_bf16(y[i]);
                        }
                    }
                }
            }
        }
        __syncthreads();
    };

    if constexpr (DB) {
        // two W buffers: the loads of the next unit are in flight while this one is reduced and
        // finished (a finished workgroup re-reads a unit once, from L2).  One exit, at the top:
        // with exits between the halves the compiler's wait counts at the loop head were merged
        // conservatively and drained the prefetch before issuing the next one.
        // (the 64-row form, 8 waves of 3 super-steps, measured 1.5 us slower in this shape at 64
        // rows and keeps the loop with exits between the halves)
        uint4 wa[SSW][2], wb[SSW][2];
        load_w(u, wa);                              // wa: unit u
        if constexpr (TT <= 2) {
            for (; u + G < units; u += 2 * G) {
                load_w(u + G, wb);
                compute(u, wa);
                const int u2 = u + 2 * G;
                load_w(u2 < units ? u2 : u + G, wa);
                compute(u + G, wb);
            }
            if (u < units) compute(u, wa);
        } else {
            while (true) {
                const int u1 = u + G;
                load_w(u1 < units ? u1 : u, wb);
                compute(u, wa);
                if (u1 >= units) break;
                const int u2 = u1 + G;
                load_w(u2 < units ? u2 : u1, wa);
                compute(u1, wb);
                if (u2 >= units) break;
                u = u2;
            }
        }
    } else {
        uint4 wa[SSW][2];
        for (; u < units; u += G) {
            load_w(u, wa);
            compute(u, wa);
        }
    }

    if constexpr (KIND == EPI_SAMPLE) {
        if (wave < TT) {
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) sample_merge(sst, sample_shfl_xor(sst, o));
            const int tok = wave * 16 + l16;
            if (g4 == 0 && tok < M) sample_store(p.samp_part + ((size_t)tok * p.amax_slots + blockIdx.x) * 2, sst);
        }
    }
    if constexpr (KIND == EPI_ARGMAX) {
        if (wave < TT) {
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float v2 = __shfl_xor(best, o, 64);
                const int i2 = __shfl_xor(bidx, o, 64);
                second = second_merge(best, second, v2, __shfl_xor(second, o, 64));
                argmax_merge(best, bidx, v2, i2);
            }
            const int tok = wave * 16 + l16;
            if (g4 == 0 && tok < M) {
                p.amax_part[(size_t)tok * p.amax_slots + blockIdx.x] = make_float2(best, __int_as_float(bidx));
                if (p.amax_sec) p.amax_sec[(size_t)tok * p.amax_slots + blockIdx.x] = second;
            }
        }
    }
}

// persistent grid: resident workgroups (occupancy, capped at kWgPerCu per CU), rounded down
// to a multiple of the slice count; cached per instantiation
constexpr int kWgPerCu = 2;
template <int KIND, int TT, int SSW, int NW, bool DB>
int skinny_grid(int units, int S) {
    static int per_cu = 0;
    if (per_cu == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_skinny<KIND, TT, SSW, NW, DB>, NW * 64, 0) != hipSuccess ||
            n <= 0)
            n = 1;
        per_cu = n < kWgPerCu ? n : kWgPerCu;
    }
    int g = device_cu_count() * per_cu;
    g = g < units ? g : units;
    g = g / S * S;
    return g < S ? S : g;
}

// Two W buffers (the next unit's loads in flight while this one is multiplied and finished) for
// the LM head, whose workgroups walk many units: 79.6 / 85.2 us at 8 / 32 rows against 82.8 / 90.7
// single-buffered (and 78.8 / 82.8 us once the loop lost its mid-loop exits), and for gate/up at
// 33-64 rows (23.7 -> 21.0 us).  At fewer rows the projections have one or two units per
// workgroup, where the second buffer mostly re-reads a unit (gate/up at 8 rows 15.0 -> 16.0 us),
// and the 7-super-step two-tile form of the 7B shape spills with it, so those keep one buffer.
template <int KIND, int TT, int SSW>
constexpr bool two_buffers() {
    return (KIND == EPI_ARGMAX && TT * SSW <= 12) || (KIND == EPI_SWIGLU && TT == 4);
}

template <int KIND, int TT, int SSW, int NW, bool DB = two_buffers<KIND, TT, SSW>()>
hipError_t go(const void* A, const void* W, int M, int N, int K, int ntiles, int S, const EpiParams& p,
              hipStream_t s) {
    const int grid = skinny_grid<KIND, TT, SSW, NW, DB>(ntiles * S, S);
    hipLaunchKernelGGL((k_skinny<KIND, TT, SSW, NW, DB>), dim3(grid), dim3(NW * 64), 0, s, (const uint16_t*)A,
                       (const uint16_t*)W, M, N, K, ntiles, S, p);
    return hipGetLastError();
}

// Variant for a full-K epilogue: the K of one unit must cover all of K.  With 64 token rows
// (TT = 4) the token fragments take 4x the registers, so the slice is spread over 8 waves of
// 3 super-steps (K <= 1536).
template <int KIND, int TT>
hipError_t go_full(const void* A, const void* W, int M, int N, int K, int ntiles, const EpiParams& p, hipStream_t s) {
    if constexpr (TT == 4) {
        if (K <= 8 * 3 * 64) return go<KIND, 4, 3, 8>(A, W, M, N, K, ntiles, 1, p, s);
        return hipErrorInvalidValue;
    } else {
        if (K <= 4 * 6 * 64) return go<KIND, TT, 6, 4>(A, W, M, N, K, ntiles, 1, p, s);
        if (K <= 8 * 7 * 64) return go<KIND, TT, 7, 8>(A, W, M, N, K, ntiles, 1, p, s);
        return hipErrorInvalidValue;
    }
}

template <int KIND, int TT>
int full_grid(int K, int ntiles) {
    if constexpr (TT == 4) {
        return skinny_grid<KIND, 4, 3, 8, two_buffers<KIND, 4, 3>()>(ntiles, 1);
    } else {
        if (K <= 4 * 6 * 64) return skinny_grid<KIND, TT, 6, 4, two_buffers<KIND, TT, 6>()>(ntiles, 1);
        return skinny_grid<KIND, TT, 7, 8, two_buffers<KIND, TT, 7>()>(ntiles, 1);
    }
}

}  // namespace

int skinny_argmax_slots(int kind, int M, int N, int K) {
    const int nt = (N + 15) / 16;
    if (kind == EPI_SAMPLE) {
        if (M > 32) return full_grid<EPI_SAMPLE, 4>(K, nt);
        return M > 16 ? full_grid<EPI_SAMPLE, 2>(K, nt) : full_grid<EPI_SAMPLE, 1>(K, nt);
    }
    if (M > 32) return full_grid<EPI_ARGMAX, 4>(K, nt);
    return M > 16 ? full_grid<EPI_ARGMAX, 2>(K, nt) : full_grid<EPI_ARGMAX, 1>(K, nt);
}

constexpr int kSkinnyPartialSlice = 4 * 3 * 64;   // K per slice of the partial-sum variant

int skinny_partial_slices(int K) { return (K + kSkinnyPartialSlice - 1) / kSkinnyPartialSlice; }

// Rows 33..64 take the 8-wave, 3-super-step variant (one workgroup per CU), the argmax LM head
// included (85.5 us at 64 rows against 101.5 us on the LDS-tiled balanced-range kernel).  Beyond 64
// rows the LM head stays on the tiled kernel: two workgroups of 64 rows walking the same W units
// on one XCD took 131.8 us at 128 rows against 109.6 us (a CU pulls ~27 GB/s in this form, and
// each then reads the whole 3.6 MB of its stream).
bool skinny_supports(int kind, int M, int K) {
    if (M > 64 || (M > 32 && kind == EPI_SAMPLE)) return false;
    if (kind == EPI_PARTIAL) return true;
    return K <= (M > 32 ? 8 * 3 * 64 : 8 * 7 * 64);
}

template <int KIND>
static hipError_t full_tt(const void* A, const void* W, int M, int N, int K, int nt, const EpiParams& p,
                          hipStream_t s) {
    if (M > 32) return go_full<KIND, 4>(A, W, M, N, K, nt, p, s);
    if (M > 16) return go_full<KIND, 2>(A, W, M, N, K, nt, p, s);
    return go_full<KIND, 1>(A, W, M, N, K, nt, p, s);
}

hipError_t launch_skinny(int kind, const void* A, const void* W, int M, int N, int K, const EpiParams& p,
                         hipStream_t s) {
    switch (kind) {
        case EPI_QKV: return full_tt<EPI_QKV>(A, W, M, N, K, N / 16, p, s);
        case EPI_SWIGLU: return full_tt<EPI_SWIGLU>(A, W, M, N, K, (p.ffn + 7) / 8, p, s);
        case EPI_ARGMAX: return full_tt<EPI_ARGMAX>(A, W, M, N, K, (N + 15) / 16, p, s);
        case EPI_SAMPLE: return full_tt<EPI_SAMPLE>(A, W, M, N, K, (N + 15) / 16, p, s);
        default: {
            const int nt = (N + 15) / 16, S = skinny_partial_slices(K);
            if (M > 32) return go<EPI_PARTIAL, 4, 3, 4>(A, W, M, N, K, nt, S, p, s);
            if (M > 16) return go<EPI_PARTIAL, 2, 3, 4>(A, W, M, N, K, nt, S, p, s);
            return go<EPI_PARTIAL, 1, 3, 4>(A, W, M, N, K, nt, S, p, s);
        }
    }
}
