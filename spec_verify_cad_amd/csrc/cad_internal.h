// Host-side internal interface of libcad: shapes, workspace carve-up and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cad.h"

// Epilogue kinds of the projection GEMMs.
enum EpiKind { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };

// Everything a GEMM epilogue needs.  Unused fields are ignored by the other kinds.
struct EpiParams {
    int M, N;                       // output rows (tokens) and logical output columns
    const int32_t* len_snap;        // [B] cache length captured at the start of the forward
    int Nq, cap;
    // EPI_QKV: RoPE + q write + K/V append
    void* q_out; void* kc; void* vc;
    int Hq, Hkv, d, mode, Dblk, f_off;
    double rope_base;
    // EPI_RESID: out = resid + acc (fp32), optional rounded copy
    const float* resid; float* out_f32; void* out_t;
    // EPI_SWIGLU: act = rnd(silu(gate) * up)
    void* act; int ffn;
    // EPI_ARGMAX: per-(row, column tile) (max, index) partials, optional logits
    float2* part; int ntiles; float* logits;
};

// Tile plan of a projection GEMM (shared by workspace sizing and launch).
struct GemmPlan { int BM, BN, nmt, nnt, grid; };
GemmPlan gemm_plan(int dtype, int M, int N, bool swiglu);

// Per-forward derived sizes.
struct FwdDims {
    int B, Nq, M, h, Hq, Hkv, d, ffn, V, cap, mode, Dblk, dtype, esz;
    int qkv_n, lm_tiles, attn_splits, attn_chunk, attn_rows_per_wg, attn_row_tiles;
};

// Workspace carve-up (offsets are 256-byte aligned).
struct FwdBufs {
    int32_t* len_snap;
    float* x; void* u; void* q; void* o;
    float* part_o; float* part_ml;
    float* h1; void* u2; void* act; float* h2; void* u3;
    float2* amax_part;
    size_t total;
};

bool fwd_dims(const cad_layer_desc* L, int B, int Nq, int mode, int W, int D, int cap, FwdDims* fd);
FwdBufs fwd_carve(const FwdDims& fd, void* base, bool kv_only);

// Launchers: each returns hipSuccess or the launch error.
hipError_t launch_embed_norm(const FwdDims& fd, const int32_t* tokens, const void* embed, float eps,
                             const int32_t* kv_len, int32_t* err, const FwdBufs& wb, hipStream_t s);
hipError_t launch_rmsnorm(const FwdDims& fd, const float* in, void* out, float eps, const int32_t* len_snap,
                          hipStream_t s);
hipError_t launch_gemm(int dtype, int kind, const void* A, const void* W, int M, int N, int K,
                       const EpiParams& p, hipStream_t s);
hipError_t launch_attention(const FwdDims& fd, const FwdBufs& wb, const void* kc, const void* vc,
                            hipStream_t s);
hipError_t launch_attention_merge(const FwdDims& fd, const FwdBufs& wb, hipStream_t s);
bool attention_uses_merge(const FwdDims& fd);
hipError_t launch_argmax_final(const FwdDims& fd, const FwdBufs& wb, int32_t* argmax_out, hipStream_t s);
hipError_t launch_commit(const FwdDims& fd, const FwdBufs& wb, int32_t* kv_len, hipStream_t s);
hipError_t launch_ngram(const int32_t* ctx, int64_t stride, const int32_t* ctx_len, int B, int n, int W,
                        int D, int with_current, int32_t* draft, int32_t* draft_len, int32_t* match_pos,
                        hipStream_t s);
hipError_t launch_accept(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                         const int32_t* first_pred, int B, int W, int D, int mode, int32_t* accepted,
                         int32_t* best_w, int32_t* emitted, int32_t* n_emitted, int32_t* ctx, int64_t ctx_stride,
                         int32_t* ctx_len, int ctx_cap, const cad_kv_desc* kv, hipStream_t s);
