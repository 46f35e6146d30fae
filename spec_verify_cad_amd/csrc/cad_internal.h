// Host-side internal interface of libcad: shapes, workspace carve-up and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cad.h"

// Epilogue kinds of the projection GEMMs.
//   EPI_QKV     RoPE at the row's absolute position; q -> workspace, k/v appended to the cache
//   EPI_SWIGLU  act = rnd(silu(gate) * up); a tile holds matching gate and up features
//   EPI_ARGMAX  LM head: per-row (max, lowest index) partials, one slot per workgroup (or per
//               column tile); a small row kernel reduces the slots and commits the cache length
//   EPI_PARTIAL fp32 partial sums of one K slice, part[slice][row][feature]; the next row
//               kernel adds the slices (in slice order) to the residual stream
enum EpiKind { EPI_QKV = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2, EPI_PARTIAL = 3, EPI_SAMPLE = 4 };

// Everything a GEMM epilogue needs.  Unused fields are ignored by the other kinds.
struct EpiParams {
    int M, N;                       // output rows (tokens) and logical output features
    const int32_t* len_snap;        // [B] cache length captured by the first kernel of the forward
    int Nq, cap;
    // EPI_QKV
    void* q_out; void* kc; void* vc;
    int Hq, Hkv, d, head_off;       // head_off: first head the GEMM produces (Hq for a K/V-only pass)
    const float2* rope_cs;          // [M, d/2] (cos, sin) of each row's position
    // EPI_SWIGLU
    void* act; int ffn;
    // EPI_ARGMAX
    float2* amax_part;              // [M, slots] (max, index bits)
    float* amax_sec;                // [M, slots] runner-up value of each slot, nullable (top-2 gap)
    int amax_slots;
    float* logits;                  // nullable debug output [M, N]
    // EPI_SAMPLE (the LM head of a sampled forward): per (row, slot) two float4 of SampleState;
    // the slot index is that of the argmax slots (amax_slots per row)
    float4* samp_part;
    float inv_temp;
    uint32_t seed_lo, seed_hi;
    const int32_t* tokens;          // [M] the forward's input tokens (row r's draft is token r + 1)
    const int32_t* draft_len;       // [B] drafts per sequence, nullable (no drafts)
    int row_pos_last;               // rows are each sequence's last row (copy-commit mode)
    // EPI_PARTIAL
    float* part;                    // [S, M, N]
    int k_slice;                    // elements of K per slice (multiple of 64)
};

// Per-forward derived sizes.
struct FwdDims {
    int B, Nq, M, h, Hq, Hkv, d, ffn, V, cap, mode, Dblk, dtype, esz;
    int qkv_n;
    int attn_splits, attn_chunk, attn_rows_per_wg, attn_row_tiles;
    int o_slices, down_slices;      // K slices of the O and down projections (partials)
    int qkv_slices, kv_slices;      // K slices of a split QKV projection (all heads / K,V heads), 0 if not split
};

// Rotary inverse frequencies base^(-2i/d), i < d/2, computed in double on the host.
struct RopeFreqs { double inv[64]; };

// Workspace carve-up (offsets are 256-byte aligned).
struct FwdBufs {
    int32_t* len_snap;
    float2* amax_part; int amax_slots;
    float* amax_sec;                // runner-up per (row, slot) for the top-2 gap
    int amax_slots_last;            // slots per row of an LM head over one row per sequence
    float2* rope_cs;
    float* x; void* u; void* q; void* o;
    float* part_o; float* part_ml;
    float* h1; void* u2; void* act; float* h2; void* u3;
    float* part;                    // K-slice partials of the O and down projections
    float* qkv_part;                // K-slice partials of a split QKV projection
    float4* samp_part;              // sampled LM head: per (row, slot) two float4 (bf16 layers)
    int samp_slots, samp_slots_last;
    size_t total;
};

// Arguments of a sampled forward (stochastic verification).
struct SampleArgs {
    float temperature;
    uint64_t seed;
    const int32_t* draft_len;       // [B], nullable
};

bool fwd_dims(const cad_layer_desc* L, int B, int Nq, int mode, int W, int D, int cap, FwdDims* fd);
// the one-layer span forward of cad_span_forward (argument checks, launches) over a given workspace
int span_forward_internal(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B, int Nq,
                          int mode, int W, int D, int flags, int32_t* argmax_out, void* hidden_out, float* logits_out,
                          float* top2_gap, void* workspace, size_t workspace_bytes, hipStream_t stream);
FwdBufs fwd_carve(const FwdDims& fd, void* base, bool kv_only);

// number of compute units of the current device (cached per device)
int device_cu_count();

// Launchers: each returns hipSuccess or the launch error.
hipError_t launch_embed_norm(const FwdDims& fd, const int32_t* tokens, const void* embed, float eps,
                             const RopeFreqs& freqs, const int32_t* kv_len, int32_t* err, const FwdBufs& wb,
                             hipStream_t s);
// argmax over the LM head's slots of `rows` rows: all M rows, or (last_only) one per sequence
// (top2_gap, nullable: largest minus second-largest logit of each row, from the runner-up slots)
hipError_t launch_argmax_final(const FwdDims& fd, const FwdBufs& wb, bool last_only, int32_t* argmax_out,
                               float* top2_gap, int32_t* kv_len, hipStream_t s);
// normed rows are written for every row, or (last_only) compactly for each sequence's last row
// argmax over each row's allowed ids (final normed rows wb.u3 against those LM-head rows),
// with the commit of the cache lengths
// reduces a sampled LM head's slots per row and writes the row's prediction (kept draft,
// replacement draw or plain draw), with the commit of the cache lengths
hipError_t launch_sample_final(const FwdDims& fd, const FwdBufs& wb, bool last_only, const int32_t* tokens,
                               const SampleArgs& sa, int32_t* pred_out, int32_t* kv_len, hipStream_t s);
hipError_t launch_allowed_argmax(const FwdDims& fd, const FwdBufs& wb, const void* w_lm, const int32_t* allowed, int A,
                                 bool last_only, int32_t* argmax_out, float* logits_out, int32_t* kv_len,
                                 hipStream_t s);
hipError_t launch_resid_norm(const FwdDims& fd, const float* base, const float* part, int slices, float* out_f32,
                             void* out_t, void* normed, bool last_only, float eps, const int32_t* len_snap,
                             hipStream_t s);
// Projection GEMM Y[M, N] = A[M, K] . W[N, K]^T with a fused epilogue; picks the kernel
// (weight-streaming for few rows, LDS-tiled MFMA otherwise) and its K slicing.  For
// EPI_PARTIAL `slices` gives the number of K slices (p.k_slice is filled in).
hipError_t launch_gemm(int dtype, int kind, const void* A, const void* W, int M, int N, int K, int slices,
                       EpiParams p, hipStream_t s);
int gemm_partial_slices(int dtype, int M, int N, int K);
bool gemm_qkv_split(int dtype, int M, int K);
// RoPE + K/V append from the QKV projection's K-slice partials (the split form of EPI_QKV):
// row r, produced columns [0, N) = heads head_off .. head_off + N/d - 1
hipError_t launch_qkv_finish(const FwdDims& fd, const float* part, int slices, int N, int head_off,
                             const FwdBufs& wb, void* kc, void* vc, hipStream_t s);
// (max, index) partial slots per row written by an EPI_ARGMAX launch of this shape
int gemm_argmax_slots(int dtype, int M, int N, int K, int kind = EPI_ARGMAX);
void attention_plan(FwdDims* fd, int cus);
hipError_t launch_attention(const FwdDims& fd, const FwdBufs& wb, const void* kc, const void* vc,
                            hipStream_t s);
hipError_t launch_attention_merge(const FwdDims& fd, const FwdBufs& wb, hipStream_t s);
bool attention_uses_merge(const FwdDims& fd);
hipError_t launch_commit(const FwdDims& fd, const FwdBufs& wb, int32_t* kv_len, hipStream_t s);
hipError_t launch_ngram(const int32_t* ctx, int64_t stride, const int32_t* ctx_len, int B, int n_hi, int n_lo,
                        int W, int D, int with_current, int32_t* draft, int32_t* draft_len, int32_t* match_pos,
                        int32_t* match_n, hipStream_t s);
// block-verify commit of layers 1 .. n_layers-1 of a stack after launch_accept committed kvs[0]
hipError_t launch_compact_layers(const cad_kv_desc* kvs, int n_layers, int B, int D, const int32_t* accepted,
                                 const int32_t* best_w, const int32_t* n_emitted, hipStream_t s);
hipError_t launch_accept(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                         const int32_t* first_pred, int B, int W, int D, int mode, int32_t* accepted,
                         int32_t* best_w, int32_t* emitted, int32_t* n_emitted, int32_t* ctx, int64_t ctx_stride,
                         int32_t* ctx_len, int ctx_cap, const cad_kv_desc* kv, hipStream_t s);
