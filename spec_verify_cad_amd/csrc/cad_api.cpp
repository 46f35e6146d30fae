// C ABI of libcad: host-side argument checks, workspace sizing/carving and the launch
// sequence of the span forward.  Nothing here allocates, frees or synchronizes.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "cad_internal.h"

namespace {

// ---- opt-in per-stage profiler (diagnostics) ----
enum Stage {
    ST_EMBED_NORM, ST_QKV, ST_ATTN, ST_ATTN_MERGE, ST_O_PROJ, ST_NORM2, ST_GATE_UP, ST_DOWN, ST_NORM3, ST_LM_HEAD,
    ST_ARGMAX, ST_COMMIT, ST_QKV_FINISH, ST_ALLOWED, ST_COUNT
};
const char* kStageNames[ST_COUNT] = {"embed_norm", "qkv_rope_append", "attention", "attention_merge", "o_proj",
                                     "resid_rmsnorm_2", "gate_up_swiglu", "down_proj", "resid_rmsnorm_final",
                                     "lm_head_argmax", "argmax_final_commit", "commit", "qkv_rope_append_rows",
                                     "allowed_ids_argmax_commit"};
struct ProfRec { int stage; hipEvent_t a, b; };
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
size_t g_used = 0;

hipEvent_t prof_event() {
    if (g_used == g_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_pool.push_back(e);
    }
    return g_pool[g_used++];
}

// Run one launch, bracketed by events when profiling is on.
template <class F>
hipError_t stage(int id, hipStream_t s, F&& launch) {
    hipEvent_t a = nullptr;
    if (g_prof && (a = prof_event())) (void)hipEventRecord(a, s);
    const hipError_t e = launch();
    if (g_prof && a) {
        hipEvent_t b = prof_event();
        if (b) {
            (void)hipEventRecord(b, s);
            g_recs.push_back({id, a, b});
        }
    }
    return e;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr long long kMaxRows = 1LL << 24;          // rows of one forward (B * Nq)

bool layer_ok(const cad_layer_desc* L) {
    if (!L) return false;
    if (L->hidden <= 0 || L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->head_dim <= 0 || L->ffn <= 0 ||
        L->vocab <= 0)
        return false;
    if (L->dtype != CAD_DTYPE_BF16 && L->dtype != CAD_DTYPE_F32) return false;
    return true;
}

bool layer_supported(const cad_layer_desc* L) {
    if (L->n_q_heads % L->n_kv_heads) return false;
    if (L->head_dim != 32 && L->head_dim != 64 && L->head_dim != 128) return false;
    if (L->hidden % 8 || L->ffn % 8 || (L->n_q_heads * L->head_dim) % 8) return false;
    if (L->hidden > 8192) return false;           // row kernels keep a hidden row in registers
    return true;
}

}  // namespace

bool fwd_dims(const cad_layer_desc* L, int B, int Nq, int mode, int W, int D, int cap, FwdDims* fd) {
    if (!layer_ok(L) || B <= 0 || Nq <= 0 || cap <= 0) return false;
    if ((long long)B * Nq > kMaxRows) return false;        // M = B * Nq rows stays far inside int
    if (mode != CAD_MASK_CAUSAL_SPAN && mode != CAD_MASK_BLOCK_TRI) return false;
    if (mode == CAD_MASK_BLOCK_TRI && (W <= 0 || D <= 0 || (long)W * D != Nq)) return false;
    std::memset(fd, 0, sizeof(*fd));
    fd->B = B; fd->Nq = Nq; fd->M = B * Nq;
    fd->h = L->hidden; fd->Hq = L->n_q_heads; fd->Hkv = L->n_kv_heads; fd->d = L->head_dim;
    fd->ffn = L->ffn; fd->V = L->vocab; fd->cap = cap; fd->mode = mode;
    fd->Dblk = mode == CAD_MASK_BLOCK_TRI ? D : 1;
    fd->dtype = L->dtype; fd->esz = L->dtype == CAD_DTYPE_F32 ? 4 : 2;
    fd->qkv_n = (fd->Hq + 2 * fd->Hkv) * fd->d;
    fd->o_slices = gemm_partial_slices(fd->dtype, fd->M, fd->h, fd->Hq * fd->d);
    fd->down_slices = gemm_partial_slices(fd->dtype, fd->M, fd->h, fd->ffn);
    if (gemm_qkv_split(fd->dtype, fd->M, fd->h)) {
        fd->qkv_slices = gemm_partial_slices(fd->dtype, fd->M, fd->qkv_n, fd->h);
        fd->kv_slices = gemm_partial_slices(fd->dtype, fd->M, 2 * fd->Hkv * fd->d, fd->h);
    }
    attention_plan(fd, device_cu_count());
    return true;
}

FwdBufs fwd_carve(const FwdDims& fd, void* base, bool kv_only) {
    FwdBufs w;
    std::memset(&w, 0, sizeof(w));
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) -> void* {
        void* r = p ? p + off : nullptr;
        off += al256(bytes);
        return r;
    };
    const size_t M = fd.M, h = fd.h, e = fd.esz, qd = (size_t)fd.Hq * fd.d;
    w.len_snap = (int32_t*)take(fd.B * sizeof(int32_t));
    w.rope_cs = (float2*)take(M * (size_t)(fd.d / 2) * sizeof(float2));
    w.u = take(M * h * e);
    if (fd.qkv_slices) {
        const size_t full = (size_t)fd.qkv_slices * fd.qkv_n, kv = (size_t)fd.kv_slices * 2 * fd.Hkv * fd.d;
        w.qkv_part = (float*)take(M * (kv_only ? kv : std::max(full, kv)) * 4);
    }
    if (!kv_only) {
        w.amax_slots = gemm_argmax_slots(fd.dtype, fd.M, fd.V, fd.h);
        w.amax_slots_last = gemm_argmax_slots(fd.dtype, fd.B, fd.V, fd.h);
        const size_t sl = std::max(M * (size_t)w.amax_slots, (size_t)fd.B * w.amax_slots_last);
        w.amax_part = (float2*)take(sl * sizeof(float2));
        w.amax_sec = (float*)take(sl * sizeof(float));
        if (fd.dtype == CAD_DTYPE_BF16) {
            w.samp_slots = gemm_argmax_slots(fd.dtype, fd.M, fd.V, fd.h, EPI_SAMPLE);
            w.samp_slots_last = gemm_argmax_slots(fd.dtype, fd.B, fd.V, fd.h, EPI_SAMPLE);
            const size_t ss = std::max(M * (size_t)w.samp_slots, (size_t)fd.B * w.samp_slots_last);
            w.samp_part = (float4*)take(ss * 2 * sizeof(float4));
        }
        w.x = (float*)take(M * h * 4);
        w.q = take(M * qd * e);
        w.o = take(M * qd * e);
        if (fd.dtype == CAD_DTYPE_BF16 && (fd.d == 64 || fd.d == 128)) {
            w.part_o = (float*)take(M * fd.Hq * (size_t)fd.attn_splits * fd.d * 4);
            w.part_ml = (float*)take(M * fd.Hq * (size_t)fd.attn_splits * 2 * 4);
        }
        w.h1 = (float*)take(M * h * 4);
        w.u2 = take(M * h * e);
        w.act = take(M * (size_t)fd.ffn * e);
        w.h2 = (float*)take(M * h * 4);
        w.u3 = take(M * h * e);
        const int S = fd.o_slices > fd.down_slices ? fd.o_slices : fd.down_slices;
        w.part = (float*)take((size_t)S * M * h * 4);
    }
    w.total = off;
    return w;
}

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

extern "C" {

const char* cad_status_string(int st) {
    switch (st) {
        case CAD_OK: return "ok";
        case CAD_EINVAL: return "invalid argument";
        case CAD_EUNSUPPORTED: return "unsupported shape";
        case CAD_ECAPACITY: return "capacity exceeded";
        case CAD_EHIP: return "HIP launch failed";
        case CAD_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

int cad_version(void) { return 100; }

int cad_profile_enable(int on) {
    g_prof = on != 0;
    return CAD_OK;
}

int cad_profile_read(int max_stages, double* ms_sum, int* count) {
    if (!ms_sum || !count || max_stages <= 0) return CAD_EINVAL;
    int st = CAD_OK;
    for (const ProfRec& r : g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            st = CAD_EHIP;
            continue;
        }
        if (r.stage < max_stages) {
            ms_sum[r.stage] += ms;
            count[r.stage] += 1;
        }
    }
    g_recs.clear();
    g_used = 0;
    return st == CAD_OK ? ST_COUNT : st;
}

const char* cad_profile_stage_name(int stage) {
    return stage >= 0 && stage < ST_COUNT ? kStageNames[stage] : "unknown";
}

size_t cad_span_forward_workspace(const cad_layer_desc* L, int B, int Nq, int mode, int W, int D, int cap,
                                  int flags) {
    FwdDims fd;
    if (!fwd_dims(L, B, Nq, mode, W, D, cap, &fd)) return 0;
    return fwd_carve(fd, nullptr, (flags & CAD_KV_ONLY) != 0).total;
}

size_t cad_stack_span_forward_workspace(const cad_layer_desc* layers, int n_layers, int B, int Nq, int mode, int W,
                                        int D, int cap, int flags) {
    FwdDims fd;
    if (!layers || n_layers < 1 || n_layers > CAD_MAX_LAYERS || !fwd_dims(&layers[0], B, Nq, mode, W, D, cap, &fd))
        return 0;
    return fwd_carve(fd, nullptr, (flags & CAD_KV_ONLY) != 0 && n_layers == 1).total;
}

namespace {

// Layers of one stack must agree in every dimension and in their norm and rotary constants.
bool same_shape(const cad_layer_desc* a, const cad_layer_desc* b) {
    return a->hidden == b->hidden && a->n_q_heads == b->n_q_heads && a->n_kv_heads == b->n_kv_heads &&
           a->head_dim == b->head_dim && a->ffn == b->ffn && a->vocab == b->vocab && a->dtype == b->dtype &&
           a->rms_eps == b->rms_eps && a->rope_base == b->rope_base;
}

// The span forward through n_layers layers (1 for the one-layer model).  The embedding is the
// first layer's and the LM head the last layer's; layer l+1 takes layer l's residual output h2
// as its input x and that output's RMSNorm u3 as its normed input.  The cache lengths and error
// flags are those of kvs[0]; kvs[l] holds layer l's K/V.  allowed == nullptr: the full LM head
// and argmax (or each sequence's last row only, with CAD_LOGITS_LAST); otherwise the argmax over
// each row's A allowed ids.  CAD_KV_ONLY runs every layer but the last in full (their outputs
// feed the next layer's K/V) and only the K/V projection of the last.
int span_forward_impl(const cad_layer_desc* layers, int n_layers, const cad_kv_desc* kvs, const int32_t* tokens,
                      int B, int Nq, int mode, int W, int D, int flags, int32_t* argmax_out, void* hidden_out,
                      float* logits_out, float* top2_gap, const int32_t* allowed, int A, const SampleArgs* samp,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!layers || !kvs || !tokens || n_layers < 1) return CAD_EINVAL;
    if (flags & ~(CAD_COMMIT_ALL | CAD_KV_ONLY | CAD_LOGITS_LAST)) return CAD_EINVAL;
    const bool kv_only = (flags & CAD_KV_ONLY) != 0;
    const bool last_only = (flags & CAD_LOGITS_LAST) != 0;
    if (last_only && mode != CAD_MASK_CAUSAL_SPAN) return CAD_EINVAL;
    const cad_layer_desc* L0 = &layers[0];
    const cad_layer_desc* Lz = &layers[n_layers - 1];
    const cad_kv_desc* kv0 = &kvs[0];
    if (!kv0->len) return CAD_EINVAL;
    FwdDims fd;
    if (!fwd_dims(L0, B, Nq, mode, W, D, kv0->cap, &fd)) return CAD_EINVAL;
    for (int l = 0; l < n_layers; ++l) {
        const cad_layer_desc* L = &layers[l];
        const cad_kv_desc* kv = &kvs[l];
        const bool full = !kv_only || l < n_layers - 1;
        if (!same_shape(L, L0) || !L->w_qkv) return CAD_EINVAL;
        if (full && (!L->w_o || !L->w_gate_up || !L->w_down)) return CAD_EINVAL;
        if (!kv->k || !kv->v || kv->B != B || kv->cap != kv0->cap) return CAD_EINVAL;
        if (kv->n_kv_heads != L->n_kv_heads || kv->head_dim != L->head_dim || kv->dtype != L->dtype) return CAD_EINVAL;
    }
    if (!L0->embed) return CAD_EINVAL;
    if (samp && (kv_only || mode != CAD_MASK_CAUSAL_SPAN || !(samp->temperature > 0.f) ||
                 !std::isfinite(samp->temperature)))
        return CAD_EINVAL;
    if (samp && L0->dtype != CAD_DTYPE_BF16) return CAD_EUNSUPPORTED;
    if (!kv_only && (!Lz->w_lm || !argmax_out)) return CAD_EINVAL;
    if (!layer_supported(L0) || kv0->cap % 4) return CAD_EUNSUPPORTED;
    if ((long)fd.M * fd.h > (1L << 31) || (long)fd.M * fd.ffn > (1L << 31)) return CAD_EUNSUPPORTED;
    const bool attends = !kv_only || n_layers > 1;
    const bool simple_attn = fd.dtype == CAD_DTYPE_F32 || (fd.d != 64 && fd.d != 128);
    if (attends && simple_attn && (size_t)(fd.cap + fd.Nq) * 4 > 64 * 1024) return CAD_EUNSUPPORTED;
    // the tiled attention addresses one head's K or V cache with 32-bit byte offsets
    if (attends && !simple_attn && (size_t)fd.cap * fd.d * 2 > 0x7FFFFFFFu) return CAD_EUNSUPPORTED;
    const FwdBufs wb = fwd_carve(fd, workspace, kv_only && n_layers == 1);
    if (!workspace || workspace_bytes < wb.total || ((uintptr_t)workspace & 255)) return CAD_EWORKSPACE;

    RopeFreqs freqs;
    for (int i = 0; i < fd.d / 2; ++i) freqs.inv[i] = std::pow(L0->rope_base, -2.0 * i / fd.d);
    if (stage(ST_EMBED_NORM, stream, [&] {
            return launch_embed_norm(fd, tokens, L0->embed, L0->rms_eps, freqs, kv0->len, kv0->err, wb, stream);
        }) != hipSuccess)
        return CAD_EHIP;

    const size_t h = fd.h;
    EpiParams base;
    std::memset(&base, 0, sizeof(base));
    base.M = fd.M; base.len_snap = wb.len_snap; base.Nq = fd.Nq; base.cap = fd.cap;
    base.Hq = fd.Hq; base.Hkv = fd.Hkv; base.d = fd.d; base.rope_cs = wb.rope_cs;
    // the residual stream alternates between two buffer pairs: layer l reads (x, u) and writes
    // (h2, u3) when l is even, the other way round when l is odd
    FwdBufs lb = wb;
    for (int l = 0; l < n_layers; ++l) {
        const cad_layer_desc* L = &layers[l];
        const cad_kv_desc* kv = &kvs[l];
        const bool last = l == n_layers - 1;
        if (l & 1) {
            lb.x = wb.h2; lb.u = wb.u3; lb.h2 = wb.x; lb.u3 = wb.u;
        } else {
            lb.x = wb.x; lb.u = wb.u; lb.h2 = wb.h2; lb.u3 = wb.u3;
        }
        EpiParams p = base;
        p.q_out = lb.q; p.kc = kv->k; p.vc = kv->v;
        const bool kv_rows_only = kv_only && last;
        // QKV projection + RoPE + K/V append (K/V rows only for the last layer of a cache prefill)
        {
            EpiParams pq = p;
            const char* w = (const char*)L->w_qkv;
            int N = fd.qkv_n;
            if (kv_rows_only) {
                pq.head_off = fd.Hq;
                w += (size_t)fd.Hq * fd.d * h * fd.esz;
                N = 2 * fd.Hkv * fd.d;
            }
            pq.N = N;
            if (fd.qkv_slices) {
                // split form: K-slice partials, then RoPE + K/V append per row
                const int S = kv_rows_only ? fd.kv_slices : fd.qkv_slices;
                pq.part = wb.qkv_part;
                if (stage(ST_QKV, stream, [&] {
                        return launch_gemm(fd.dtype, EPI_PARTIAL, lb.u, w, fd.M, N, fd.h, S, pq, stream);
                    }) != hipSuccess)
                    return CAD_EHIP;
                if (stage(ST_QKV_FINISH, stream, [&] {
                        return launch_qkv_finish(fd, wb.qkv_part, S, N, pq.head_off, lb, kv->k, kv->v, stream);
                    }) != hipSuccess)
                    return CAD_EHIP;
            } else if (stage(ST_QKV, stream, [&] {
                           return launch_gemm(fd.dtype, EPI_QKV, lb.u, w, fd.M, N, fd.h, 1, pq, stream);
                       }) != hipSuccess) {
                return CAD_EHIP;
            }
        }
        if (kv_rows_only) {
            if ((flags & CAD_COMMIT_ALL) &&
                stage(ST_COMMIT, stream, [&] { return launch_commit(fd, wb, kv0->len, stream); }) != hipSuccess)
                return CAD_EHIP;
            return CAD_OK;
        }
        if (stage(ST_ATTN, stream, [&] { return launch_attention(fd, lb, kv->k, kv->v, stream); }) != hipSuccess)
            return CAD_EHIP;
        if (attention_uses_merge(fd) &&
            stage(ST_ATTN_MERGE, stream, [&] { return launch_attention_merge(fd, lb, stream); }) != hipSuccess)
            return CAD_EHIP;
        // O projection (K-slice partials) -> h1 = x + o.Wo^T, u2 = RMSNorm(h1)
        EpiParams po = p;
        po.N = fd.h; po.part = wb.part;
        if (stage(ST_O_PROJ, stream, [&] {
                return launch_gemm(fd.dtype, EPI_PARTIAL, lb.o, L->w_o, fd.M, fd.h, fd.Hq * fd.d, fd.o_slices, po,
                                   stream);
            }) != hipSuccess)
            return CAD_EHIP;
        if (stage(ST_NORM2, stream, [&] {
                return launch_resid_norm(fd, lb.x, wb.part, fd.o_slices, wb.h1, nullptr, wb.u2, false, L->rms_eps,
                                         wb.len_snap, stream);
            }) != hipSuccess)
            return CAD_EHIP;
        EpiParams pg = p;
        pg.N = 2 * fd.ffn; pg.act = wb.act; pg.ffn = fd.ffn;
        if (stage(ST_GATE_UP, stream, [&] {
                return launch_gemm(fd.dtype, EPI_SWIGLU, wb.u2, L->w_gate_up, fd.M, 2 * fd.ffn, fd.h, 1, pg, stream);
            }) != hipSuccess)
            return CAD_EHIP;
        // down projection (K-slice partials) -> h2 = h1 + act.Wd^T, u3 = RMSNorm(h2); the last
        // layer also writes hidden_out = rnd(h2), and with CAD_LOGITS_LAST normalises only each
        // sequence's last row
        EpiParams pd = p;
        pd.N = fd.h; pd.part = wb.part;
        if (stage(ST_DOWN, stream, [&] {
                return launch_gemm(fd.dtype, EPI_PARTIAL, wb.act, L->w_down, fd.M, fd.h, fd.ffn, fd.down_slices, pd,
                                   stream);
            }) != hipSuccess)
            return CAD_EHIP;
        if (stage(ST_NORM3, stream, [&] {
                return launch_resid_norm(fd, wb.h1, wb.part, fd.down_slices, lb.h2, last ? hidden_out : nullptr,
                                         lb.u3, last && last_only, L->rms_eps, wb.len_snap, stream);
            }) != hipSuccess)
            return CAD_EHIP;
    }
    if (allowed) {
        // grammar-masked step: logits of the allowed ids only, argmax, commit
        if (stage(ST_ALLOWED, stream, [&] {
                return launch_allowed_argmax(fd, lb, Lz->w_lm, allowed, A, last_only, argmax_out, logits_out,
                                             (flags & CAD_COMMIT_ALL) ? kv0->len : nullptr, stream);
            }) != hipSuccess)
            return CAD_EHIP;
        return CAD_OK;
    }
    // LM head + argmax partials, then the per-row reduction (+ commit of the cache lengths).
    // Copy-commit mode: u3 holds one row per sequence (row b = the sequence's last row).
    EpiParams pl = base;
    const int lm_rows = last_only ? fd.B : fd.M;
    pl.M = lm_rows; pl.Nq = last_only ? 1 : fd.Nq;
    pl.N = fd.V; pl.amax_part = wb.amax_part; pl.amax_slots = last_only ? wb.amax_slots_last : wb.amax_slots;
    pl.amax_sec = top2_gap ? wb.amax_sec : nullptr;
    pl.logits = logits_out;
    if (samp) {
        // sampled LM head: the slots hold sampling states; rows know their sequence, position
        // and draft through the forward's own geometry
        pl.Nq = fd.Nq;
        pl.amax_slots = last_only ? wb.samp_slots_last : wb.samp_slots;
        pl.samp_part = wb.samp_part;
        pl.inv_temp = 1.0f / samp->temperature;
        pl.seed_lo = (uint32_t)(samp->seed & 0xFFFFFFFFu);
        pl.seed_hi = (uint32_t)(samp->seed >> 32);
        pl.tokens = tokens;
        pl.draft_len = samp->draft_len;
        pl.row_pos_last = last_only ? 1 : 0;
        if (stage(ST_LM_HEAD, stream, [&] {
                return launch_gemm(fd.dtype, EPI_SAMPLE, lb.u3, Lz->w_lm, lm_rows, fd.V, fd.h, 1, pl, stream);
            }) != hipSuccess)
            return CAD_EHIP;
        if (stage(ST_ARGMAX, stream, [&] {
                return launch_sample_final(fd, wb, last_only, tokens, *samp, argmax_out,
                                           (flags & CAD_COMMIT_ALL) ? kv0->len : nullptr, stream);
            }) != hipSuccess)
            return CAD_EHIP;
        return CAD_OK;
    }
    if (stage(ST_LM_HEAD, stream, [&] {
            return launch_gemm(fd.dtype, EPI_ARGMAX, lb.u3, Lz->w_lm, lm_rows, fd.V, fd.h, 1, pl, stream);
        }) != hipSuccess)
        return CAD_EHIP;
    if (stage(ST_ARGMAX, stream, [&] {
            return launch_argmax_final(fd, wb, last_only, argmax_out, top2_gap,
                                       (flags & CAD_COMMIT_ALL) ? kv0->len : nullptr, stream);
        }) != hipSuccess)
        return CAD_EHIP;
    return CAD_OK;
}

}  // namespace

}  // extern "C"

int span_forward_internal(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B, int Nq,
                          int mode, int W, int D, int flags, int32_t* argmax_out, void* hidden_out, float* logits_out,
                          float* top2_gap, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return span_forward_impl(L, 1, kv, tokens, B, Nq, mode, W, D, flags, argmax_out, hidden_out, logits_out, top2_gap,
                             nullptr, 0, nullptr, workspace, workspace_bytes, stream);
}

extern "C" {

int cad_span_forward(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B, int Nq,
                     int mode, int W, int D, int flags, int32_t* argmax_out, void* hidden_out, float* logits_out,
                     float* top2_gap, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return span_forward_impl(L, 1, kv, tokens, B, Nq, mode, W, D, flags, argmax_out, hidden_out, logits_out, top2_gap,
                             nullptr, 0, nullptr, workspace, workspace_bytes, stream);
}

int cad_span_forward_allowed(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B, int Nq,
                             int flags, const int32_t* allowed, int A, int32_t* argmax_out, float* logits_out,
                             void* hidden_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!allowed || !argmax_out) return CAD_EINVAL;
    if (A < 1 || A > CAD_MAX_ALLOWED) return CAD_EUNSUPPORTED;
    if (flags & ~(CAD_COMMIT_ALL | CAD_LOGITS_LAST)) return CAD_EINVAL;
    if (!L || !kv) return CAD_EINVAL;
    return span_forward_impl(L, 1, kv, tokens, B, Nq, CAD_MASK_CAUSAL_SPAN, 1, 1, flags, argmax_out, hidden_out,
                             logits_out, nullptr, allowed, A, nullptr, workspace, workspace_bytes, stream);
}

int cad_span_forward_sampled(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B, int Nq,
                             int flags, float temperature, uint64_t seed, const int32_t* draft_len, int32_t* pred_out,
                             float* logits_out, void* hidden_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!L || !kv || !pred_out) return CAD_EINVAL;
    if (flags & ~(CAD_COMMIT_ALL | CAD_LOGITS_LAST)) return CAD_EINVAL;
    const SampleArgs sa{temperature, seed, draft_len};
    return span_forward_impl(L, 1, kv, tokens, B, Nq, CAD_MASK_CAUSAL_SPAN, 1, 1, flags, pred_out, hidden_out,
                             logits_out, nullptr, nullptr, 0, &sa, workspace, workspace_bytes, stream);
}

int cad_stack_span_forward_allowed(const cad_layer_desc* layers, int n_layers, const cad_kv_desc* kvs,
                                   const int32_t* tokens, int B, int Nq, int flags, const int32_t* allowed, int A,
                                   int32_t* argmax_out, float* logits_out, void* hidden_out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (n_layers < 1 || n_layers > CAD_MAX_LAYERS) return CAD_EINVAL;
    if (!allowed || !argmax_out) return CAD_EINVAL;
    if (A < 1 || A > CAD_MAX_ALLOWED) return CAD_EUNSUPPORTED;
    if (flags & ~(CAD_COMMIT_ALL | CAD_LOGITS_LAST)) return CAD_EINVAL;
    return span_forward_impl(layers, n_layers, kvs, tokens, B, Nq, CAD_MASK_CAUSAL_SPAN, 1, 1, flags, argmax_out,
                             hidden_out, logits_out, nullptr, allowed, A, nullptr, workspace, workspace_bytes, stream);
}

int cad_stack_span_forward_sampled(const cad_layer_desc* layers, int n_layers, const cad_kv_desc* kvs,
                                   const int32_t* tokens, int B, int Nq, int flags, float temperature, uint64_t seed,
                                   const int32_t* draft_len, int32_t* pred_out, float* logits_out, void* hidden_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n_layers < 1 || n_layers > CAD_MAX_LAYERS || !pred_out) return CAD_EINVAL;
    if (flags & ~(CAD_COMMIT_ALL | CAD_LOGITS_LAST)) return CAD_EINVAL;
    const SampleArgs sa{temperature, seed, draft_len};
    return span_forward_impl(layers, n_layers, kvs, tokens, B, Nq, CAD_MASK_CAUSAL_SPAN, 1, 1, flags, pred_out,
                             hidden_out, logits_out, nullptr, nullptr, 0, &sa, workspace, workspace_bytes, stream);
}

int cad_stack_span_forward(const cad_layer_desc* layers, int n_layers, const cad_kv_desc* kvs, const int32_t* tokens,
                           int B, int Nq, int mode, int W, int D, int flags, int32_t* argmax_out, void* hidden_out,
                           float* logits_out, float* top2_gap, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (n_layers < 1 || n_layers > CAD_MAX_LAYERS) return CAD_EINVAL;
    return span_forward_impl(layers, n_layers, kvs, tokens, B, Nq, mode, W, D, flags, argmax_out, hidden_out,
                             logits_out, top2_gap, nullptr, 0, nullptr, workspace, workspace_bytes, stream);
}

int cad_ngram_lookup(const int32_t* ctx, int64_t ctx_stride, const int32_t* ctx_len, int B, int n, int W, int D,
                     int with_current, int32_t* draft, int32_t* draft_len, int32_t* match_pos, hipStream_t stream) {
    if (!ctx || !ctx_len || !draft || !draft_len) return CAD_EINVAL;
    if (B <= 0 || n <= 0 || W <= 0 || D <= 0 || ctx_stride <= 0) return CAD_EINVAL;
    if (with_current != 0 && with_current != 1) return CAD_EINVAL;
    if (W > 8 || D > 64 || n > 64 || ctx_stride > 0x7fffffff) return CAD_EUNSUPPORTED;
    return launch_ngram(ctx, ctx_stride, ctx_len, B, n, n, W, D, with_current, draft, draft_len, match_pos, nullptr,
                        stream) == hipSuccess
               ? CAD_OK
               : CAD_EHIP;
}

int cad_ngram_lookup_longest(const int32_t* ctx, int64_t ctx_stride, const int32_t* ctx_len, int B, int n_max,
                             int n_min, int W, int D, int with_current, int32_t* draft, int32_t* draft_len,
                             int32_t* match_pos, int32_t* match_n, hipStream_t stream) {
    if (!ctx || !ctx_len || !draft || !draft_len) return CAD_EINVAL;
    if (B <= 0 || n_min <= 0 || n_max < n_min || W <= 0 || D <= 0 || ctx_stride <= 0) return CAD_EINVAL;
    if (with_current != 0 && with_current != 1) return CAD_EINVAL;
    if (W > 8 || D > 64 || n_max > 64 || ctx_stride > 0x7fffffff) return CAD_EUNSUPPORTED;
    return launch_ngram(ctx, ctx_stride, ctx_len, B, n_max, n_min, W, D, with_current, draft, draft_len, match_pos,
                        match_n, stream) == hipSuccess
               ? CAD_OK
               : CAD_EHIP;
}

}  // extern "C"

namespace {

// Host-side checks shared by the one-layer and the stack accept scan.
int accept_args_ok(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                   const int32_t* first_pred, int B, int W, int D, int mode, const int32_t* accepted,
                   const int32_t* emitted, const int32_t* n_emitted, const int32_t* ctx, int64_t ctx_stride,
                   const int32_t* ctx_len, int ctx_cap, const cad_kv_desc* kv) {
    if (!draft || !draft_len || !pred || !accepted || !emitted || !n_emitted) return CAD_EINVAL;
    if (B <= 0 || W <= 0 || D <= 0) return CAD_EINVAL;
    if (mode == CAD_MASK_CAUSAL_SPAN) {
        if (W != 1 || with_current != 1) return CAD_EINVAL;
    } else if (mode == CAD_MASK_BLOCK_TRI) {
        if (!first_pred || with_current != 0) return CAD_EINVAL;
    } else {
        return CAD_EINVAL;
    }
    if (ctx && (!ctx_len || ctx_stride <= 0 || ctx_cap <= 0 || ctx_cap > ctx_stride)) return CAD_EINVAL;
    if (kv && (!kv->len || kv->B != B)) return CAD_EINVAL;
    if (kv && mode == CAD_MASK_BLOCK_TRI &&
        (!kv->k || !kv->v || kv->n_kv_heads <= 0 || (kv->head_dim != 32 && kv->head_dim != 64 &&
                                                      kv->head_dim != 128)))
        return CAD_EINVAL;
    if (W > 8 || D > 64 || (kv && kv->cap % 4)) return CAD_EUNSUPPORTED;
    return CAD_OK;
}

}  // namespace

extern "C" {

int cad_accept_scan(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                    const int32_t* first_pred, int B, int W, int D, int mode, int32_t* accepted, int32_t* best_w,
                    int32_t* emitted, int32_t* n_emitted, int32_t* ctx, int64_t ctx_stride, int32_t* ctx_len,
                    int ctx_cap, const cad_kv_desc* kv, hipStream_t stream) {
    const int st = accept_args_ok(draft, with_current, draft_len, pred, first_pred, B, W, D, mode, accepted, emitted,
                                  n_emitted, ctx, ctx_stride, ctx_len, ctx_cap, kv);
    if (st != CAD_OK) return st;
    return launch_accept(draft, with_current, draft_len, pred, first_pred, B, W, D, mode, accepted, best_w, emitted,
                         n_emitted, ctx, ctx_stride, ctx_len, ctx_cap, kv, stream) == hipSuccess
               ? CAD_OK
               : CAD_EHIP;
}

int cad_stack_accept_scan(const int32_t* draft, int with_current, const int32_t* draft_len, const int32_t* pred,
                          const int32_t* first_pred, int B, int W, int D, int mode, int32_t* accepted,
                          int32_t* best_w, int32_t* emitted, int32_t* n_emitted, int32_t* ctx, int64_t ctx_stride,
                          int32_t* ctx_len, int ctx_cap, const cad_kv_desc* kvs, int n_layers, hipStream_t stream) {
    if (!kvs || n_layers < 1 || n_layers > CAD_MAX_LAYERS) return CAD_EINVAL;
    const int st = accept_args_ok(draft, with_current, draft_len, pred, first_pred, B, W, D, mode, accepted, emitted,
                                  n_emitted, ctx, ctx_stride, ctx_len, ctx_cap, &kvs[0]);
    if (st != CAD_OK) return st;
    const bool block = mode == CAD_MASK_BLOCK_TRI && n_layers > 1;
    if (block) {
        if (!best_w) return CAD_EINVAL;
        for (int l = 1; l < n_layers; ++l) {
            const cad_kv_desc& k = kvs[l];
            if (!k.k || !k.v || k.B != B || k.cap != kvs[0].cap || k.n_kv_heads != kvs[0].n_kv_heads ||
                k.head_dim != kvs[0].head_dim || k.dtype != kvs[0].dtype)
                return CAD_EINVAL;
        }
    }
    if (launch_accept(draft, with_current, draft_len, pred, first_pred, B, W, D, mode, accepted, best_w, emitted,
                      n_emitted, ctx, ctx_stride, ctx_len, ctx_cap, &kvs[0], stream) != hipSuccess)
        return CAD_EHIP;
    if (block && launch_compact_layers(kvs, n_layers, B, D, accepted, best_w, n_emitted, stream) != hipSuccess)
        return CAD_EHIP;
    return CAD_OK;
}

}  // extern "C"
