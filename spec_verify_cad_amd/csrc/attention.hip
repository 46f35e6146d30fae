// Span attention: the Nq new rows of every sequence attend to the cached prefix plus the span
// rows their mask allows (causal span, or SwitchSD's block-triangular candidate mask), with
// grouped-query heads sharing one K/V stream.
//
// bf16 path (gfx950 MFMA, head_dim 64 or 128): split-L flash decoding with LDS-staged K/V
// tiles.  A workgroup owns one (sequence, KV head, key split, row tile); the rows of a tile are
// the (token, q head) pairs of the GQA group, so the K/V of a split is fetched once for all of
// them.  64-row tiles (4 waves) copy 64-key tiles through registers (K rows, and the dim-major
// V rows with each lane's 8 keys gathered into one 16-byte chunk) into two swizzled LDS
// buffers, the next tile in flight while the current one is multiplied; 80- and 128-row tiles
// (10 and 8 waves) copy K and V straight from the cache into three LDS buffers each, two tiles
// ahead.  Each wave takes 16 rows in 32-key steps:
//   S^T = K . Q^T   A = 16 keys x 32 dims of the K tile, B = the wave's query fragments;
//   O^T += V^T . P^T  A = 16 dims x 32 keys of the V tile, B = P^T taken from the score
//                   registers: MFMA k-slots 8g+i / 8g+4+i carry the keys of the scores lane
//                   (g, r) holds, so P never moves between lanes (4g+i / 16+4g+i on the
//                   register-staged tiles; 8g+i / 8g+4+i, the K rows taken in a permuted order,
//                   on the direct-copy tiles, whose V chunks are then plain runs of 8 keys).
// Online softmax runs in registers with exp2 and wavefront max/sum reductions; P enters the PV
// product as bf16 hi + bf16 lo (the rounding remainder), two MFMAs, so the weights keep about
// 16 significant bits.  With one split the wave writes the normalised output; otherwise it
// writes (m, l, O) partials and a merge kernel combines them.
//
// fp32 path: one workgroup per (row, q head), plain two-pass softmax over all keys.
#include <type_traits>

#include "cad_device.h"

namespace {

constexpr int WAVES = 4;

template <int MODE>
__device__ __forceinline__ bool key_allowed(int key, int len, int it, int Dblk) {
    if (key < len) return true;
    const int s = key - len;
    if constexpr (MODE == CAD_MASK_BLOCK_TRI) {
        const int w = it / Dblk, j = it % Dblk;
        return s >= w * Dblk && s <= w * Dblk + j;
    }
    return s <= it;
}
__device__ __forceinline__ bool key_allowed(int key, int len, int it, int mode, int Dblk) {
    return mode == CAD_MASK_BLOCK_TRI ? key_allowed<CAD_MASK_BLOCK_TRI>(key, len, it, Dblk)
                                      : key_allowed<CAD_MASK_CAUSAL_SPAN>(key, len, it, Dblk);
}

// Keys per split for a sequence of len cached rows and Nq new rows: the live keys spread
// evenly over the nsplit splits in whole 64-key tiles, so splits past the live range get no
// keys.  Computed on the device from the cache length the forward captured.
__device__ __forceinline__ int split_chunk(int len, int Nq, int nsplit) {
    const int S = len + Nq;
    int c = (S + nsplit - 1) / nsplit;
    return (c + 63) & ~63;
}

// Swizzled 16-byte chunk positions in the LDS tiles (reads of 16 consecutive rows at one chunk
// index, and writes of whole rows, touch every bank once).
//   K tile [TK keys][DH]: chunk c of key row r; V tile [DH dims][TK keys]: chunk c of dim row r.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int DH>
__device__ __forceinline__ int swz_k(int r, int c) {
    if constexpr (DH == 128) return c ^ (r & 15);       // 256-byte rows
    else return c ^ ((r >> 1) & 7);                     // 128-byte rows
}
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ ((r >> 1) & 7); }   // 128-byte rows
// K swizzle for the permuted score order of the two-tile-lead tiles (below): the 16 rows one
// 16-lane group reads, keys 8q + 4h + r (q, r = 0..3, h fixed), land in 16 distinct bank groups
template <int DH>
__device__ __forceinline__ int swz_kp(int r, int c) {
    if constexpr (DH == 128) return c ^ ((r & 3) | ((r >> 1) & 12));
    else return c ^ (((r >> 1) & 1) | ((r >> 2) & 6));
}

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes at voff land at lds + 16 i
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t res, uint32_t lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voff, 0, 0, 0);
}

// NPH key phases: with NPH = 2 the waves form NWV/2 row blocks twice over, and phase p takes
// keys 32p .. 32p+31 of every tile (its own running maximum and sums); the two phases' states
// are combined through LDS at the end.  This halves each wave's chain per tile for groups whose
// rows fill few waves (the PLD verify: 66 rows, five row blocks).
template <int DH, int MODE, int NWV, int NPH = 1>
// (4-wave tiles run two workgroups per CU: the register budget must leave two waves per SIMD)
__global__ __launch_bounds__(NWV * 64, NWV == 4 ? 2 : 1) void k_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                   const uint16_t* __restrict__ vc, const int32_t* __restrict__ len_snap,
                                                   int Nq, int Hq, int Hkv, int cap, int Dblk,
                                                   int nsplit, float* __restrict__ part_o,
                                                   float* __restrict__ part_ml, uint16_t* __restrict__ o_out) {
    constexpr int DS = DH / 32;                 // MFMA k-steps over head_dim
    constexpr int DB = DH / 16;                 // 16-wide head_dim blocks of the output
    constexpr int TK = 64;                      // keys per LDS tile (two 32-key MFMA steps)
    constexpr int KCH = DH / 8;                 // 16-byte chunks of a K row
    constexpr int NT = NWV * 64;                // threads; NWV waves of 16 rows each (per phase)
    constexpr int NRW = NWV / NPH;              // row blocks
    constexpr int KB = 4 / NPH;                 // 16-key score blocks of a wave per tile
    constexpr int KTOT = TK * KCH, VTOT = DH * (TK / 4);     // 16-byte K chunks, 4-key V groups per tile
    constexpr int KLD = (KTOT + NT - 1) / NT;   // K chunks each thread copies per tile
    constexpr int VLD = (VTOT + NT - 1) / NT;   // 4-key V groups each thread copies per tile
    static_assert(NPH == 1 || NPH == 2, "one or two key phases");
    // DEEP (8- and 10-wave tiles, one workgroup per CU): K and V tiles land in LDS straight from
    // memory, two steps ahead of their use, in three buffers each (separate variables, each a
    // compile-time choice in every copy of the unrolled loop); otherwise K and V come through
    // registers one tile ahead into two buffers each.
    constexpr bool DEEP = NWV >= 8;
    constexpr int KSZ = TK * KCH, VSZ = DH * (TK / 8);
    __shared__ u32x4_t ks0[DEEP ? KSZ : 1], ks1[DEEP ? KSZ : 1], ks2[DEEP ? KSZ : 1];
    __shared__ u32x4_t vs0[DEEP ? VSZ : 1], vs1[DEEP ? VSZ : 1], vs2[DEEP ? VSZ : 1];
    __shared__ u32x4_t ksr[DEEP ? 1 : 2][DEEP ? 1 : KSZ];
    __shared__ u32x4_t vsr[DEEP ? 1 : 2][DEEP ? 1 : VSZ];

    auto KS = [&](int i) __attribute__((always_inline)) -> u32x4_t* {
        if constexpr (DEEP) return i == 0 ? ks0 : (i == 1 ? ks1 : ks2);
        else return ksr[i];
    };
    auto VS = [&](int i) __attribute__((always_inline)) -> u32x4_t* {
        if constexpr (DEEP) return i == 0 ? vs0 : (i == 1 ? vs1 : vs2);
        else return vsr[i];
    };
    const int split = blockIdx.x, rtile = blockIdx.y;
    const int bg = blockIdx.z, b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv, Rg = Nq * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int rw = wave % NRW, ph = __builtin_amdgcn_readfirstlane(wave / NRW);   // row block, key phase

    const int wg_row0 = rtile * (NRW * 16);
    const int wrow0 = wg_row0 + rw * 16;
    const bool wlive = wrow0 < Rg;              // a wave without rows still copies tiles
    const bool ok = seq_ok(len_snap, b, Nq, cap);
    const int len = ok ? len_snap[b] : 0;
    const int rho = wrow0 + l16;
    const bool qlive = rho < Rg;
    const int it = qlive ? rho / G : 0, hh = qlive ? rho % G : 0;
    // keys past len + (last token of the workgroup's rows) are masked for all of its rows
    const int it_max = min(Nq - 1, min(wg_row0 + NRW * 16 - 1, Rg - 1) / G);
    const int chunk = split_chunk(len, Nq, nsplit);
    const int kbeg = split * chunk;
    int kend = min(kbeg + chunk, len + it_max + 1);
    if (!ok) kend = kbeg;
    if constexpr (DEEP) kend = __builtin_amdgcn_readfirstlane(kend);   // (uniform loop exits)

    bf16x8_t qf[DS];
    {
        const uint16_t* qp = q + (((size_t)b * Nq + it) * Hq + g * G + hh) * DH;
#pragma unroll
        for (int d = 0; d < DS; ++d) {
            // unconditional (a lane without a row reads row 0's q, finite, and writes nothing):
            // a load inside a branch would make the wait counts of the loop below conservative
            uint4 v = *(const uint4*)(qp + d * 32 + g4 * 8);
            qf[d] = *(bf16x8_t*)&v;
        }
    }

    const float sl2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e)/sqrt(d)
    // m_run: the query's reference maximum (log2 units), shared by its 4 lanes; it may trail the
    // running maximum by up to RESCALE, so weights stay <= 2^RESCALE and the accumulators are
    // rescaled only when some lane of the wave exceeds that.  It starts at a finite M_NONE (below
    // any score), so a weight exp2(s - m_run) needs no guard: a masked score (-inf) gives 0, and
    // the first visible score triggers a rescale; M_NONE is reported as -inf.  l_lane: this
    // lane's share of the weight sum (its 8 keys of every step), summed over the 4 lanes at the end.
    constexpr float RESCALE = 8.f, M_NONE = -1e30f;
    float m_run = M_NONE, l_lane = 0.f;
    f32x4_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // keys this lane's query sees, below kend: [0, vis_a) and [vis_lo, vis_hi] (causal: the
    // cached prefix and the span up to the query's own position; block mode: the prefix and the
    // query's candidate block up to its position in it); none for a lane without a query
    int vis_a, vis_lo, vis_hi;
    if constexpr (MODE == CAD_MASK_BLOCK_TRI) {
        const int w = it / Dblk, j = it % Dblk;
        vis_a = min(kend, len);
        vis_lo = len + w * Dblk;
        vis_hi = min(kend - 1, len + w * Dblk + j);
    } else {
        vis_a = min(kend, len + it + 1);
        vis_lo = 1;
        vis_hi = 0;
    }
    if (!qlive) { vis_a = INT_MIN / 2; vis_lo = 1; vis_hi = 0; }

    const size_t head = (size_t)b * Hkv + g;
    const uint16_t* kbase = kc + head * cap * DH;
    const uint16_t* vbase = vc + head * DH * cap;          // dim-major: row = one dim over all slots

    // (4-wave tiles) K/V in registers on their way to LDS.  K runs one tile ahead of V: during step t the K rows
    // of tile t + 2 and the V rows of tile t + 1 are fetched, so that step t can multiply tile
    // t + 1's scores while it turns tile t's scores into weights.  The loads stay in program order
    // (a scheduling barrier after each), so the compiler's wait counts at the loop head, which
    // merge the issue order of the prologue and of the previous step, wait for the oldest loads
    // only.  Every load is issued unconditionally from a valid address: a K row past kend reads
    // slot 0 (its scores are masked), a V group past kend reads slot 0 and is zeroed (so masked
    // keys add exactly zero); cap is a multiple of 4, so an 8-byte V group never crosses the end
    // of a row.
    struct Tile { u32x4_t k[KLD]; u32x2_t v[VLD]; };
    // (when the thread count does not divide a tile, the surplus threads of the last round load
    // a clamped, valid chunk and store nothing)
    auto load_k = [&](int tk0, Tile& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int id = min(tid + NT * i, KTOT - 1), key = tk0 + id / KCH;
            r.k[i] = *(const u32x4_t*)(kbase + (size_t)(key < kend ? key : 0) * DH + (id % KCH) * 8);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto load_v = [&](int tv0, auto& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int id = min(tid + NT * i, VTOT - 1), key0 = tv0 + 4 * (id % (TK / 4));
            r.v[i] = *(const u32x2_t*)(vbase + (size_t)(id / (TK / 4)) * cap + (key0 < kend ? key0 : 0));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto load = [&](int tk0, int tv0, Tile& r) __attribute__((always_inline)) {
        load_k(tk0, r);
        load_v(tv0, r);
    };
    // V tile layout: the 8 keys an MFMA lane needs (4g..4g+3 and 16+4g..16+4g+3 of a 32-key step)
    // form one 16-byte chunk, chunk kq*4 + g of the dim row.  (K into buffer kb, V of the tile at
    // tv0 into buffer vb.)
    auto store_k = [&](int kb, const Tile& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int id = tid + NT * i, key = id / KCH;
            if (KTOT % NT == 0 || id < KTOT) KS(kb)[key * KCH + swz_k<DH>(key, id % KCH)] = r.k[i];
        }
    };
    auto store_v = [&](int tv0, int vb, const auto& r) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int id = tid + NT * i, row = id / (TK / 4), grp = id % (TK / 4);
            if (VTOT % NT != 0 && id >= VTOT) continue;
            const int n = kend - (tv0 + 4 * grp);                  // valid keys of the group
            u32x2_t w = r.v[i];
            w.x &= n >= 2 ? 0xFFFFFFFFu : (n == 1 ? 0xFFFFu : 0u);
            w.y &= n >= 4 ? 0xFFFFFFFFu : (n == 3 ? 0xFFFFu : 0u);
            const int kq = grp >> 3, gq = grp & 7;
            const int c = swz_v(row, kq * 4 + (gq & 3));
            ((u32x2_t*)VS(vb))[(row * (TK / 8) + c) * 2 + (gq >> 2)] = w;
        }
    };
    auto store = [&](int tv0, int kb, int vb, const Tile& r) __attribute__((always_inline)) {
        store_k(kb, r);
        store_v(tv0, vb, r);
    };
    // Copies of the two-tile lead (DEEP, below): 1 KB blocks of a tile go from the cache straight
    // into an LDS buffer, one buffer load per wave and block, lane i's 16 bytes at block offset
    // 16 i; each lane fetches the logical chunk that the swizzle places at its slot (the
    // swizzles are their own inverses).  Each copy reads through a buffer resource based at the
    // tile's first key, with per-lane byte offsets fixed for the whole loop (the compiler waits
    // for a load in flight before its address register is rewritten).  With more waves than
    // blocks some waves repeat a block.  K rows past kend hold whatever the cache holds (their
    // scores are masked); V keys past kend are zeroed in LDS before the tile's value product
    // (vzero); whatever lies past the cache's end reads zero.  V is dim-major: a 64-key tile is
    // DH rows of 128 bytes, chunk c holding keys 8c .. 8c + 7 (the permuted score order makes
    // these a lane's eight weights).
    constexpr int KBLK = KSZ / 64, KD = (KBLK + NWV - 1) / NWV;
    constexpr int VBLK = VSZ / 64, VD = (VBLK + NWV - 1) / NWV;
    uint32_t koff[KD], voff[VD];
#pragma unroll
    for (int j = 0; j < KD; ++j) {
        const int e = ((__builtin_amdgcn_readfirstlane(wave) * KD + j) % KBLK) * 64 + lane, key = e / KCH;
        koff[j] = (key * DH + swz_kp<DH>(key, e % KCH) * 8) * 2;
    }
#pragma unroll
    for (int j = 0; j < VD; ++j) {
        const int e = ((__builtin_amdgcn_readfirstlane(wave) * VD + j) % VBLK) * 64 + lane, row = e / (TK / 8);
        voff[j] = (row * cap + swz_v(row, e % (TK / 8)) * 8) * 2;
    }
    // (the LDS address passes through readfirstlane, an integer: the compiler then does not tie
    // the copy to the buffer it fills and does not make reads of the other buffers wait for it;
    // the explicit counts before each barrier order them)
    auto lds_addr = [&](u32x4_t* p) __attribute__((always_inline)) -> uint32_t {
        return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p);
    };
    auto kdirect = [&](int tk0, int kb) __attribute__((always_inline)) {
        const auto res = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)tk0 * DH), (short)0,
                                                           max(0, cap - tk0) * DH * 2, 0x00020000);
#pragma unroll
        for (int j = 0; j < KD; ++j) {
            buf_to_lds16(res, lds_addr(&KS(kb)[((__builtin_amdgcn_readfirstlane(wave) * KD + j) % KBLK) * 64]), koff[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto vdirect = [&](int tv0, int vb) __attribute__((always_inline)) {
        const auto res = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + tv0), (short)0,
                                                           max(0, DH * cap - tv0) * 2, 0x00020000);
#pragma unroll
        for (int j = 0; j < VD; ++j) {
            buf_to_lds16(res, lds_addr(&VS(vb)[((__builtin_amdgcn_readfirstlane(wave) * VD + j) % VBLK) * 64]), voff[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // zero the keys >= kend of the V tile at tv0 in buffer vb (the tile that holds kend)
    auto vzero = [&](int tv0, int vb) __attribute__((always_inline)) {
        const int nv = kend - tv0;
        for (int id = tid; id < VSZ; id += NT) {
            const int row = id / (TK / 8), c = id % (TK / 8), n = nv - 8 * c;   // valid keys of the chunk
            if (n >= 8) continue;
            u32x4_t& w = VS(vb)[row * (TK / 8) + swz_v(row, c)];
            u32x4_t m;
#pragma unroll
            for (int q = 0; q < 4; ++q) m[q] = n >= 2 * q + 2 ? 0xFFFFFFFFu : (n == 2 * q + 1 ? 0xFFFFu : 0u);
            w &= m;
        }
    };
    // this wave's four (two with two key phases) 16-key score blocks of the K tile in buffer kb:
    // S^T = K . Q^T, score block kb of the tile is st[kb - ph*KB]
    auto scores = [&](int kb, f32x4_t(&st)[KB]) __attribute__((always_inline)) {
#pragma unroll
        for (int kbi = 0; kbi < KB; ++kbi) {
            const int bk = ph * KB + kbi;
            // DEEP: output row 4 g + i of blocks 2 kq, 2 kq + 1 is key 32 kq + 8 g + i, + 4 + i, so
            // each lane's eight weights of a 32-key step are eight consecutive keys
            const int key = DEEP ? (bk >> 1) * 32 + 8 * (l16 >> 2) + 4 * (bk & 1) + (l16 & 3) : bk * 16 + l16;
            st[kbi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < DS; ++d) {
                const int ch = DEEP ? swz_kp<DH>(key, d * 4 + g4) : swz_k<DH>(key, d * 4 + g4);
                const u32x4_t kv = KS(kb)[key * KCH + ch];
                st[kbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)&kv, qf[d], st[kbi], 0, 0, 0);
            }
        }
    };
    // mask the scores of the tile at keys k0.. (S^T[key][query]: lane holds keys
    // k0 + (ph*KB + kb)*16 + 4*g4 + i of query l16, or with the permuted order (DEEP) keys
    // k0 + 32*(bk >> 1) + 8*g4 + 4*(bk & 1) + i, bk = ph*KB + kb) to -inf outside the lane's visible keys and
    // return the lane's maximum in log2 units; the scores stay unscaled (the weights fold the
    // 1/sqrt(d) scale into their exponent).  One compare per score against per-tile bounds
    // (bitwise: short-circuit tests made the compiler branch per score).
    auto mask_max = [&](int k0, f32x4_t(&st)[KB]) __attribute__((always_inline)) {
        const int base = DEEP ? k0 + ph * (KB / 2) * 32 + g4 * 8 : k0 + ph * KB * 16 + g4 * 4;
        const int A = vis_a - base, L = vis_lo - base, H = vis_hi - base;
        float lmax = -INFINITY;
#pragma unroll
        for (int kbi = 0; kbi < KB; ++kbi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = DEEP ? (kbi >> 1) * 32 + (kbi & 1) * 4 + i : kbi * 16 + i;
                bool al = c < A;
                if constexpr (MODE == CAD_MASK_BLOCK_TRI) al = al | ((c >= L) & (c <= H));
                const float sv = al ? st[kbi][i] : -INFINITY;
                st[kbi][i] = sv;
                lmax = fmaxf(lmax, sv);
            }
        return lmax * sl2;
    };
    // lazy rescale: only when some lane of the wave exceeds the reference maximum by RESCALE
    auto rescale = [&](float lmax) __attribute__((always_inline)) {
        if (__ballot(lmax > m_run + RESCALE) != 0) {      // wave-uniform, rare after the first tile
            float tmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
    };
    // P^T fragment of keys 32kq ..: k-slot 8*g4 + i <- key 4*g4 + i (block 2kq), 8*g4 + 4 + i <-
    // key 16 + 4*g4 + i (block 2kq + 1); each weight as bf16 hi + bf16 lo (both round to nearest
    // even, two keys per conversion)
    auto weights = [&](int kqi, const f32x4_t(&st)[KB], bf16x8_t& phi, bf16x8_t& pl) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kb = 2 * kqi + (j >> 1), i = (j & 1) * 2;     // index into st
            const f32x2_t pv = f32x2_t{__builtin_amdgcn_exp2f(fmaf(st[kb][i], sl2, -m_run)),
                                       __builtin_amdgcn_exp2f(fmaf(st[kb][i + 1], sl2, -m_run))};
            const bf16x2_t h = __builtin_convertvector(pv, bf16x2_t);
            const bf16x2_t lo = __builtin_convertvector(pv - __builtin_convertvector(h, f32x2_t), bf16x2_t);
            l_lane += pv.x + pv.y;
            phi[2 * j] = h.x; phi[2 * j + 1] = h.y;
            pl[2 * j] = lo.x; pl[2 * j + 1] = lo.y;
        }
    };
    auto values = [&](int kqi, int vb, const bf16x8_t& phi, const bf16x8_t& pl) __attribute__((always_inline)) {
        const int kq = ph * (2 / NPH) + kqi;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int row = db * 16 + l16;
            const u32x4_t vv = VS(vb)[row * (TK / 8) + swz_v(row, kq * 4 + g4)];
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)&vv, phi, oacc[db], 0, 0, 0);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)&vv, pl, oacc[db], 0, 0, 0);
        }
    };
    // One 64-key step of tile t at keys k0 (its scores in cur, masked, the reference maximum
    // already updated; its V in buffer vb), with tile t + 1's scores (K in buffer kbn) going to
    // nxt: the weights of tile t are formed while tile t + 1's score MFMAs run, and tile t + 1's
    // mask and maximum while tile t's value MFMAs run; the issue order is pinned below.
    auto step = [&](int k0, int kbn, int vb, f32x4_t(&cur)[KB], f32x4_t(&nxt)[KB]) __attribute__((always_inline)) {
        constexpr int NKQ = 2 / NPH;
        bf16x8_t phi[NKQ], pl[NKQ];
#pragma unroll
        for (int kqi = 0; kqi < NKQ; ++kqi) weights(kqi, cur, phi[kqi], pl[kqi]);
        scores(kbn, nxt);
#pragma unroll
        for (int kqi = 0; kqi < NKQ; ++kqi) values(kqi, vb, phi[kqi], pl[kqi]);
        const float lmax = mask_max(k0 + TK, nxt);
        // issue pattern: the score reads, then each score MFMA with a share of the weight
        // arithmetic; then each value MFMA (its V read ahead) with a share of the masking
        constexpr int NS = KB * DS, NV = 2 * NKQ * DB;         // score and value MFMAs
#pragma unroll
        for (int i = 0; i < NS; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // K reads
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                          // VALU
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // V read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                          // VALU
        }
        rescale(lmax);
    };

    // tile t's weights and value products only (the last tile of a split)
    auto last = [&](int vb, const f32x4_t(&cur)[KB]) __attribute__((always_inline)) {
        constexpr int NKQ = 2 / NPH;
#pragma unroll
        for (int kqi = 0; kqi < NKQ; ++kqi) {
            bf16x8_t phi, pl;
            weights(kqi, cur, phi, pl);
            values(kqi, vb, phi, pl);
        }
    };

    f32x4_t st0[KB], st1[KB];
    Tile r, r1;
    if (NPH == 1 && kend - kbeg <= TK) {
        // one tile (every split of a short span): fetched, copied, scored and multiplied in turn
        // (the two-phase tile serves long histories only)
        if constexpr (DEEP) {
            kdirect(kbeg, 0);
            vdirect(kbeg, 0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (kend - kbeg < TK) {
                vzero(kbeg, 0);
                __syncthreads();
            }
        } else {
            load(kbeg, kbeg, r);
            store(kbeg, 0, 0, r);
            __syncthreads();
        }
        if (wlive) {
            scores(0, st0);
            rescale(mask_max(kbeg, st0));
            last(0, st0);
        }
    } else if constexpr (DEEP) {
        // Two tiles of lead.  Prologue: the K of tiles 0, 1, 2 into K buffers 0, 1, 2 and the V of
        // tiles 0, 1 into V buffers 0, 1, all issued together; tile 0's scores once its K has
        // landed.  Step t opens by copying tile t + 3's K into K buffer t % 3 (last read by tile
        // t's scores, in step t - 1) and tile t + 2's V into V buffer (t + 2) % 3 (last read by
        // tile t - 1's value product), then scores tile t + 1 out of K buffer (t + 1) % 3 and
        // multiplies tile t's V out of V buffer t % 3: every copy has two steps to land.  Before
        // the barrier that closes step t each wave waits for its LDS writes and for its share of
        // tile t + 2's K and tile t + 1's V, not for the copies issued after them (tile t + 3's K
        // and tile t + 2's V): the count is explicit and the barrier carries no memory fence (a
        // fence would wait for every copy into LDS); empty asm statements keep the compiler from
        // moving LDS accesses across it.  The tile that holds kend has its V keys past kend
        // zeroed before its value product.  The loop is unrolled six times (three buffers, two
        // score register sets), so every buffer is a compile-time choice in each copy.
        constexpr int WN = KD + VD, WN0 = 2 * KD + 2 * VD;
        static_assert(WN0 < 64, "vmcnt range");
        // s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt left open)
        constexpr int WAITK = (WN & 15) | (7 << 4) | ((WN >> 4) << 14);
        constexpr int WAIT0 = (WN0 & 15) | (7 << 4) | ((WN0 >> 4) << 14);
        constexpr int WAIT1 = (VD & 15) | (7 << 4) | ((VD >> 4) << 14);
        constexpr int WAITL = 15 | (7 << 4) | (3 << 14);                  // lgkmcnt(0) only
        auto bar = [&]() __attribute__((always_inline)) {
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            __asm__ volatile("" ::: "memory");
        };
        auto wait_bar = [&](auto w) __attribute__((always_inline)) {
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(decltype(w)::value);
            bar();
        };
        using std::integral_constant;
        kdirect(kbeg, 0);
        kdirect(kbeg + TK, 1);
        kdirect(kbeg + 2 * TK, 2);
        vdirect(kbeg, 0);
        vdirect(kbeg + TK, 1);
        wait_bar(integral_constant<int, WAIT0>{});         // tile 0's K
        if (wlive) {
            scores(0, st0);
            rescale(mask_max(kbeg, st0));
        }
        wait_bar(integral_constant<int, WAIT1>{});         // tiles 1 and 2's K, tile 0's V
        // one step at t0 = kbeg + (6i + P) TK; true once the split is done
        auto body = [&](auto pc, int t0) __attribute__((always_inline)) -> bool {
            constexpr int P = decltype(pc)::value;
            f32x4_t(&cur)[KB] = (P & 1) ? st1 : st0;
            f32x4_t(&nxt)[KB] = (P & 1) ? st0 : st1;
            if constexpr (NPH == 1) {
                if (t0 + TK >= kend) {
                    if (t0 + TK > kend) {
                        vzero(t0, P % 3);
                        wait_bar(integral_constant<int, WAITL>{});
                    }
                    if (wlive) last(P % 3, cur);
                    return true;
                }
            } else if (t0 >= kend) {
                return true;
            }
            kdirect(t0 + 3 * TK, P % 3);
            vdirect(t0 + 2 * TK, (P + 2) % 3);
            if constexpr (NPH == 2) {
                if (t0 + TK > kend) {
                    vzero(t0, P % 3);
                    wait_bar(integral_constant<int, WAITL>{});
                }
            }
            if (wlive) step(t0, (P + 1) % 3, P % 3, cur, nxt);
            wait_bar(integral_constant<int, WAITK>{});
            return false;
        };
        for (int t0 = kbeg;; t0 += 6 * TK) {
            if (body(integral_constant<int, 0>{}, t0)) break;
            if (body(integral_constant<int, 1>{}, t0 + TK)) break;
            if (body(integral_constant<int, 2>{}, t0 + 2 * TK)) break;
            if (body(integral_constant<int, 3>{}, t0 + 3 * TK)) break;
            if (body(integral_constant<int, 4>{}, t0 + 4 * TK)) break;
            if (body(integral_constant<int, 5>{}, t0 + 5 * TK)) break;
        }
        __builtin_amdgcn_s_waitcnt(0);                     // no copy may still write LDS below
    } else {
        // Prologue: tiles 0 and 1 fetched together (one memory round trip); tile 0's K through
        // buffer 0, its scores, mask and reference maximum; then tile 1's K to buffer 1 and tile
        // 0's V to buffer 0, with tile 2's K fetched behind tile 1's V.  Step t runs on K buffer
        // (t + 1) & 1 and V buffer t & 1; after it the K of tile t + 2 goes to buffer t & 1 (last
        // read by tile t's scores, in step t - 1) and the V of tile t + 1 to buffer (t + 1) & 1
        // (last read in step t - 1), both before the barrier that opens step t + 1.  The last
        // tile takes its weights and values only (one-phase tiles).  The loop is unrolled by two
        // so the score sets and buffers are constants.
        load(kbeg, kbeg, r);
        load(kbeg + TK, kbeg + TK, r1);
        store_k(0, r);
        __syncthreads();
        if (wlive) {
            scores(0, st0);
            rescale(mask_max(kbeg, st0));
        }
        store_k(1, r1);                                    // K of tile 1
        store_v(kbeg, 0, r);                               // V of tile 0
#pragma unroll
        for (int i = 0; i < VLD; ++i) r.v[i] = r1.v[i];   // tile 1's V, in flight
        load_k(kbeg + 2 * TK, r);
        __syncthreads();
        // (the two-phase tile keeps a full step for its last tile: the peeled form spilled
        // registers there, and its splits hold hundreds of tiles)
        for (int t0 = kbeg;;) {
            if constexpr (NPH == 1) {
                if (t0 + TK >= kend) {
                    if (wlive) last(0, st0);
                    break;
                }
            } else if (t0 >= kend) {
                break;
            }
            if (wlive) step(t0, 1, 0, st0, st1);
            store(t0 + TK, 0, 1, r);
            load(t0 + 3 * TK, t0 + 2 * TK, r);
            __syncthreads();
            t0 += TK;
            if constexpr (NPH == 1) {
                if (t0 + TK >= kend) {
                    if (wlive) last(1, st1);
                    break;
                }
            } else if (t0 >= kend) {
                break;
            }
            if (wlive) step(t0, 0, 1, st1, st0);
            store(t0 + TK, 1, 0, r);
            load(t0 + 3 * TK, t0 + 2 * TK, r);
            __syncthreads();
            t0 += TK;
        }
    }

    float l_run = l_lane + __shfl_xor(l_lane, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if constexpr (NPH == 2) {
        // phase 1 hands (m, l, O) to phase 0 of the same row block and lane through the K/V
        // buffers (free once every wave has left the loop), a quarter of O in each of four:
        // O = O0 2^(m0-m) + O1 2^(m1-m)
        __shared__ float2 ml1[NRW * 64];
        constexpr int DQ = DB / 4;
        static_assert(DB % 4 == 0 && NRW * 64 * DQ * sizeof(f32x4_t) <= KSZ * sizeof(u32x4_t) &&
                      NRW * 64 * DQ * sizeof(f32x4_t) <= VSZ * sizeof(u32x4_t), "O quarters fit the K/V buffers");
        f32x4_t* const oq[4] = {(f32x4_t*)KS(0), (f32x4_t*)KS(1), (f32x4_t*)VS(0), (f32x4_t*)VS(1)};
        const int slot = rw * 64 + lane;
        __syncthreads();
        if (ph == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oq[db / DQ][slot * DQ + db % DQ] = oacc[db];
            ml1[slot] = make_float2(m_run, l_run);
        }
        __syncthreads();
        if (ph == 1) return;
        const float2 o1ml = ml1[slot];
        const float m = fmaxf(m_run, o1ml.x);
        // (both maxima are finite, M_NONE at the least)
        const float a0 = __builtin_amdgcn_exp2f(m_run - m);
        const float a1 = __builtin_amdgcn_exp2f(o1ml.x - m);
        l_run = l_run * a0 + o1ml.y * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            oacc[db] = oacc[db] * a0 + oq[db / DQ][slot * DQ + db % DQ] * a1;
        m_run = m;
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
        part_ml[pidx * 2 + 0] = m_run == M_NONE ? -INFINITY : m_run;   // no visible key: -inf
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

// Merge for few splits (nsplit <= SMAX): DH/4 threads per (row, q head), four dims each, several
// pairs per workgroup and no LDS.  Every thread loads all the pair's (m, l) and its four dims of
// each split at once, then combines them in split order with the same weights as k_attn_merge.
template <typename T, int DH, int SMAX>
__global__ __launch_bounds__(256) void k_attn_merge_few(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        const int32_t* __restrict__ len_snap, int Nq, int Hq, int Hkv,
                                                        int cap, int nsplit, int pairs, T* __restrict__ o) {
    constexpr int TPG = DH / 4;
    const int rowhead = blockIdx.x * (256 / TPG) + threadIdx.x / TPG;   // (b*Nq + it)*Hq + h
    const int q = threadIdx.x % TPG;
    if (rowhead >= pairs) return;
    const int h = rowhead % Hq, row = rowhead / Hq;
    const int b = row / Nq, it = row % Nq;
    if (!seq_ok(len_snap, b, Nq, cap)) return;
    const int len = len_snap[b];
    const int chunk = split_chunk(len, Nq, nsplit);
    const int live = min(nsplit, (len + Nq + chunk - 1) / chunk);
    const int G = Hq / Hkv, g = h / G, hh = h % G;
    const int Rg = Nq * G, rho = it * G + hh;
    const size_t p0 = (((size_t)b * Hkv + g) * Rg + rho) * nsplit;
    float2 ml[SMAX];
    float4 ov[SMAX];
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int sp = min(j, live - 1);
        ml[j] = *(const float2*)(part_ml + (p0 + sp) * 2);
        ov[j] = *(const float4*)(part_o + (p0 + sp) * DH + 4 * q);
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < SMAX; ++j) m = j < live ? fmaxf(m, ml[j].x) : m;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const float w = (j >= live || ml[j].x == -INFINITY) ? 0.f : exp2f(ml[j].x - m);
        L += w * ml[j].y;
        acc.x += w * ov[j].x;
        acc.y += w * ov[j].y;
        acc.z += w * ov[j].z;
        acc.w += w * ov[j].w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t ob = (size_t)rowhead * DH + 4 * q;
    Elt<T>::st(o, ob + 0, acc.x * inv);
    Elt<T>::st(o, ob + 1, acc.y * inv);
    Elt<T>::st(o, ob + 2, acc.z * inv);
    Elt<T>::st(o, ob + 3, acc.w * inv);
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

// Split plan of the MFMA path: 64-row tiles of each GQA group and key splits: with few row tiles
// enough splits to fill the chip (each at least one 64-key tile of a full cache), otherwise as
// many as keep every workgroup resident (two per CU), at most 8.  The keys of a split follow
// from the sequence's length on the device.
void attention_plan(FwdDims* fd, int cus) {
    const int G = fd->Hq / fd->Hkv, Rg = fd->Nq * G;
    // 128-row tiles (8 waves) once a GQA group has more than 64 rows: the K/V of a split is then
    // fetched for twice the rows (a 66-row group, 6 heads x 11 positions, is one tile, not two)
    fd->attn_rows_per_wg = Rg > 64 ? 128 : 64;
    // a group of 65..80 rows (the PLD verify: 6 heads x 11 positions) takes 80-row tiles of five
    // row blocks in two key phases (ten waves, one workgroup per CU), not an 8-wave tile with
    // three idle waves
    if (Rg > 64 && Rg <= 80 && fd->d == 128) fd->attn_rows_per_wg = 80;
    fd->attn_row_tiles = (Rg + fd->attn_rows_per_wg - 1) / fd->attn_rows_per_wg;
    const long units = (long)fd->B * fd->Hkv * fd->attn_row_tiles;
    // resident workgroups: two 4-wave or one 8- or 10-wave workgroup per CU (registers and LDS)
    const long want = (fd->attn_rows_per_wg == 64 ? 2L : 1L) * cus;
    long splits = want / units;
    if (splits > 24) {
        // few row tiles (small spans): as many splits as fill the chip, the merge is cheap
        splits = (want + units - 1) / units;
        const long most = (fd->cap + fd->Nq + 63) / 64;  // splits of at least one 64-key tile
        if (splits > most) splits = most;
        if (splits > 256) splits = 256;                  // the merge holds at most 256 split weights
    } else if (splits > 8) {
        splits = 8;                                      // the merge without LDS takes up to 8
    }
    // (never more workgroups than stay resident: a second, nearly empty round costs a whole one)
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
    const bool tri = fd.mode == CAD_MASK_BLOCK_TRI;
    const int nt = fd.attn_rows_per_wg == 80 ? 640 : fd.attn_rows_per_wg / 16 * 64;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(nt), 0, s, (const uint16_t*)wb.q, (const uint16_t*)kc,
                           (const uint16_t*)vc, wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.Dblk, fd.attn_splits,
                           wb.part_o, wb.part_ml, (uint16_t*)wb.o);
    };
    const bool big = fd.attn_rows_per_wg == 128;
    if (fd.d == 128 && fd.attn_rows_per_wg == 80) {
        if (tri) go(k_attn_bf16<128, CAD_MASK_BLOCK_TRI, 10, 2>);
        else go(k_attn_bf16<128, CAD_MASK_CAUSAL_SPAN, 10, 2>);
    } else if (fd.d == 128) {
        if (tri) big ? go(k_attn_bf16<128, CAD_MASK_BLOCK_TRI, 8>) : go(k_attn_bf16<128, CAD_MASK_BLOCK_TRI, 4>);
        else big ? go(k_attn_bf16<128, CAD_MASK_CAUSAL_SPAN, 8>) : go(k_attn_bf16<128, CAD_MASK_CAUSAL_SPAN, 4>);
    } else {
        if (tri) big ? go(k_attn_bf16<64, CAD_MASK_BLOCK_TRI, 8>) : go(k_attn_bf16<64, CAD_MASK_BLOCK_TRI, 4>);
        else big ? go(k_attn_bf16<64, CAD_MASK_CAUSAL_SPAN, 8>) : go(k_attn_bf16<64, CAD_MASK_CAUSAL_SPAN, 4>);
    }
    return hipGetLastError();
}

bool attention_uses_merge(const FwdDims& fd) { return mfma_path(fd) && fd.attn_splits > 1; }

hipError_t launch_attention_merge(const FwdDims& fd, const FwdBufs& wb, hipStream_t s) {
    const int pairs = fd.M * fd.Hq;
    if (fd.attn_splits <= 8) {
        const int per = 256 / (fd.d / 4);
        const dim3 grid((pairs + per - 1) / per);
        if (fd.d == 128)
            hipLaunchKernelGGL((k_attn_merge_few<uint16_t, 128, 8>), grid, dim3(256), 0, s, wb.part_o, wb.part_ml,
                               wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, pairs, (uint16_t*)wb.o);
        else
            hipLaunchKernelGGL((k_attn_merge_few<uint16_t, 64, 8>), grid, dim3(256), 0, s, wb.part_o, wb.part_ml,
                               wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, pairs, (uint16_t*)wb.o);
        return hipGetLastError();
    }
    if (fd.d == 128)
        hipLaunchKernelGGL((k_attn_merge<uint16_t, 128>), dim3(pairs), dim3(256), 0, s, wb.part_o, wb.part_ml,
                           wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, (uint16_t*)wb.o);
    else
        hipLaunchKernelGGL((k_attn_merge<uint16_t, 64>), dim3(pairs), dim3(256), 0, s, wb.part_o, wb.part_ml,
                           wb.len_snap, fd.Nq, fd.Hq, fd.Hkv, fd.cap, fd.attn_splits, (uint16_t*)wb.o);
    return hipGetLastError();
}
