// Host-side driver of the C ABI's argument handling, built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU (no GPU, no HIP runtime): the launchers the C-ABI file
// calls and the six HIP runtime calls it makes are replaced by stubs that count launches, so the
// whole host path (argument checks, shape planning, workspace carving, the launch sequence of a
// forward) runs with fake device pointers that are never dereferenced.
//
// Every argument-error case must return its status with no launch; every valid call must return
// CAD_OK and enqueue its launches.  Exit status 0 = all cases passed.
#include <cstdio>
#include <cstring>
#include <vector>

#include "cad_internal.h"

static int g_launches = 0;
static int g_fail = 0;

// ---- HIP runtime stubs (the only runtime calls of the C-ABI file) ----
extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) { static int pool[4096]; static int n = 0; *e = (hipEvent_t)&pool[n++ % 4096]; return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.001f; return hipSuccess; }
}

// ---- launcher and planner stubs ----
static hipError_t launched() { ++g_launches; return hipSuccess; }
hipError_t launch_embed_norm(const FwdDims&, const int32_t*, const void*, float, const RopeFreqs&, const int32_t*,
                             int32_t*, const FwdBufs&, hipStream_t) { return launched(); }
hipError_t launch_argmax_final(const FwdDims&, const FwdBufs&, bool, int32_t*, float*, int32_t*, hipStream_t) {
    return launched();
}
hipError_t launch_sample_final(const FwdDims&, const FwdBufs&, bool, const int32_t*, const SampleArgs&, int32_t*,
                               int32_t*, hipStream_t) { return launched(); }
hipError_t launch_allowed_argmax(const FwdDims&, const FwdBufs&, const void*, const int32_t*, int, bool, int32_t*,
                                 float*, int32_t*, hipStream_t) { return launched(); }
hipError_t launch_resid_norm(const FwdDims&, const float*, const float*, int, float*, void*, void*, bool, float,
                             const int32_t*, hipStream_t) { return launched(); }
hipError_t launch_gemm(int, int, const void*, const void*, int, int, int, int, EpiParams, hipStream_t) {
    return launched();
}
int gemm_partial_slices(int, int M, int, int K) { return M > 64 ? 4 : (K + 767) / 768; }
bool gemm_qkv_split(int dtype, int M, int) { return dtype == CAD_DTYPE_BF16 && M > 64; }
hipError_t launch_qkv_finish(const FwdDims&, const float*, int, int, int, const FwdBufs&, void*, void*, hipStream_t) {
    return launched();
}
int gemm_argmax_slots(int, int M, int, int, int) { return M > 32 ? 594 : 512; }
void attention_plan(FwdDims* fd, int) { fd->attn_splits = 8; fd->attn_chunk = 64; fd->attn_rows_per_wg = 64; fd->attn_row_tiles = 1; }
hipError_t launch_attention(const FwdDims&, const FwdBufs&, const void*, const void*, hipStream_t) { return launched(); }
hipError_t launch_attention_merge(const FwdDims&, const FwdBufs&, hipStream_t) { return launched(); }
bool attention_uses_merge(const FwdDims&) { return true; }
hipError_t launch_commit(const FwdDims&, const FwdBufs&, int32_t*, hipStream_t) { return launched(); }
hipError_t launch_ngram(const int32_t*, int64_t, const int32_t*, int, int, int, int, int, int, int32_t*, int32_t*,
                        int32_t*, int32_t*, hipStream_t) { return launched(); }
hipError_t launch_compact_layers(const cad_kv_desc*, int, int, int, const int32_t*, const int32_t*, const int32_t*,
                                 hipStream_t) { return launched(); }
hipError_t launch_accept(const int32_t*, int, const int32_t*, const int32_t*, const int32_t*, int, int, int, int,
                         int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, int64_t, int32_t*, int, const cad_kv_desc*,
                         hipStream_t) { return launched(); }

// ---- checks ----
#define EXPECT(call, want_status, want_launches)                                                              \
    do {                                                                                                       \
        const int before = g_launches;                                                                         \
        const int st = (call);                                                                                 \
        const int n = g_launches - before;                                                                     \
        const bool ok = st == (want_status) && ((want_launches) < 0 ? n > 0 : n == (want_launches));           \
        if (!ok) {                                                                                             \
            std::printf("FAIL line %d: %s -> status %d (want %d), launches %d\n", __LINE__, #call, st,          \
                        (int)(want_status), n);                                                                \
            ++g_fail;                                                                                          \
        }                                                                                                      \
    } while (0)

static void* P(uintptr_t v) { return (void*)v; }                 // fake device pointer, never dereferenced

static cad_layer_desc layer(int dtype = CAD_DTYPE_BF16, int head_dim = 64, int kv = 4) {
    cad_layer_desc d;
    std::memset(&d, 0, sizeof(d));
    d.hidden = 256; d.n_q_heads = 4; d.n_kv_heads = kv; d.head_dim = head_dim; d.ffn = 1024; d.vocab = 1024;
    d.dtype = dtype; d.rms_eps = 1e-6f; d.rope_base = 1e4;
    d.embed = d.w_qkv = d.w_o = d.w_gate_up = d.w_down = d.w_lm = P(0x1000);
    return d;
}

static cad_kv_desc cache(int B = 1, int cap = 160, int kv = 4, int head_dim = 64) {
    cad_kv_desc k;
    k.k = P(0x2000); k.v = P(0x3000); k.len = (int32_t*)P(0x4000); k.err = (int32_t*)P(0x5000);
    k.B = B; k.cap = cap; k.n_kv_heads = kv; k.head_dim = head_dim; k.dtype = CAD_DTYPE_BF16;
    return k;
}

int main() {
    const cad_layer_desc d = layer();
    const cad_kv_desc kv = cache();
    int32_t* tok = (int32_t*)P(0x6000);
    void* ws = P(0x100000);
    const size_t big = (size_t)1 << 30;

    // workspace queries
    const size_t full = cad_span_forward_workspace(&d, 1, 8, 0, 1, 1, 160, 0);
    const size_t kvo = cad_span_forward_workspace(&d, 1, 8, 0, 1, 1, 160, CAD_KV_ONLY);
    if (!(full > kvo && kvo > 0)) { std::printf("FAIL workspace sizes %zu %zu\n", full, kvo); ++g_fail; }
    if (cad_span_forward_workspace(&d, 1, 8, CAD_MASK_BLOCK_TRI, 3, 3, 160, 0) != 0) ++g_fail;
    cad_layer_desc bad_dtype = layer(); bad_dtype.dtype = 7;
    if (cad_span_forward_workspace(&bad_dtype, 1, 8, 0, 1, 1, 160, 0) != 0) ++g_fail;
    if (cad_span_forward_workspace(nullptr, 1, 8, 0, 1, 1, 160, 0) != 0) ++g_fail;
    if (cad_span_forward_workspace(&d, 1 << 20, 1 << 12, 0, 1, 1, 160, 0) != 0) ++g_fail;   // 2^32 rows: rejected
    if (cad_span_forward_workspace(&d, 1 << 12, 1 << 12, 0, 1, 1, 1 << 13, 0) == 0) ++g_fail;  // 2^24 rows: valid
    EXPECT(cad_span_forward(&d, &kv, tok, 1 << 20, 1 << 12, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);

    // span forward: argument errors (the cases of the ctypes ABI test)
    EXPECT(cad_span_forward(nullptr, &kv, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward(&d, &kv, nullptr, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    cad_kv_desc bad = cache(1, 160, 2);
    EXPECT(cad_span_forward(&d, &bad, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    cad_layer_desc d48 = layer(CAD_DTYPE_BF16, 48);
    cad_kv_desc kv48 = cache(1, 160, 4, 48);
    EXPECT(cad_span_forward(&d48, &kv48, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, P(256), 16, nullptr), CAD_EWORKSPACE, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, P(8), big, nullptr), CAD_EWORKSPACE, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, 8, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, 0, nullptr, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 0, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, CAD_MASK_BLOCK_TRI, 3, 4, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, CAD_MASK_BLOCK_TRI, 2, 4, CAD_LOGITS_LAST, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    cad_kv_desc odd = cache(1, 166);
    EXPECT(cad_span_forward(&d, &odd, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EUNSUPPORTED, 0);
    cad_kv_desc nolen = kv; nolen.len = nullptr;
    EXPECT(cad_span_forward(&d, &nolen, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    // valid forwards (host path only): causal, block, copy-commit, K/V-only, fp32, many rows
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, CAD_COMMIT_ALL, tok, P(0x7000), (float*)P(0x8000), (float*)P(0x9000), ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, CAD_MASK_BLOCK_TRI, 2, 4, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, CAD_COMMIT_ALL | CAD_LOGITS_LAST, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, CAD_COMMIT_ALL | CAD_KV_ONLY, nullptr, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    const cad_layer_desc d32 = layer(CAD_DTYPE_F32);
    cad_kv_desc kv32 = cache(); kv32.dtype = CAD_DTYPE_F32;
    EXPECT(cad_span_forward(&d32, &kv32, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    cad_kv_desc kvb = cache(4, 1024);
    EXPECT(cad_span_forward(&d, &kvb, tok, 4, 200, 0, 1, 1, CAD_COMMIT_ALL, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);

    // masked-decision and sampled forwards
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 1, 0, nullptr, 4, tok, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 1, 0, tok, 4, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 1, 0, tok, 0, tok, nullptr, nullptr, ws, big, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 1, 0, tok, CAD_MAX_ALLOWED + 1, tok, nullptr, nullptr, ws, big, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 1, CAD_KV_ONLY, tok, 4, tok, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward_allowed(&d, &kv, tok, 1, 3, CAD_COMMIT_ALL | CAD_LOGITS_LAST, tok, 4, tok, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_span_forward_sampled(&d, &kv, tok, 1, 8, 0, 0.f, 1, nullptr, tok, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward_sampled(&d, &kv, tok, 1, 8, 0, 1.f / 0.f, 1, nullptr, tok, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_span_forward_sampled(&d32, &kv32, tok, 1, 8, 0, 1.f, 1, nullptr, tok, nullptr, nullptr, ws, big, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_span_forward_sampled(&d, &kv, tok, 1, 8, CAD_COMMIT_ALL, 0.7f, 99, tok, tok, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);

    // stacks
    std::vector<cad_layer_desc> ls(3, d);
    std::vector<cad_kv_desc> ks(3, kv);
    ls[0].w_lm = nullptr; ls[1].embed = ls[1].w_lm = nullptr; ls[2].embed = nullptr;
    EXPECT(cad_stack_span_forward(ls.data(), 0, ks.data(), tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_stack_span_forward(ls.data(), CAD_MAX_LAYERS + 1, ks.data(), tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    std::vector<cad_layer_desc> mixed = ls;
    mixed[1].ffn = 512;
    EXPECT(cad_stack_span_forward(mixed.data(), 3, ks.data(), tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    std::vector<cad_kv_desc> kmixed = ks;
    kmixed[2].cap = 200;
    EXPECT(cad_stack_span_forward(ls.data(), 3, kmixed.data(), tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_stack_span_forward(ls.data(), 3, ks.data(), tok, 1, 8, 0, 1, 1, CAD_COMMIT_ALL, tok, nullptr, nullptr, (float*)P(0x9000), ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_stack_span_forward(ls.data(), 3, ks.data(), tok, 1, 8, 0, 1, 1, CAD_COMMIT_ALL | CAD_KV_ONLY, nullptr, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_stack_span_forward_allowed(ls.data(), 3, ks.data(), tok, 1, 2, 0, tok, 5, tok, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    EXPECT(cad_stack_span_forward_sampled(ls.data(), 3, ks.data(), tok, 1, 4, 0, 1.f, 5, nullptr, tok, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    if (cad_stack_span_forward_workspace(ls.data(), 3, 1, 8, 0, 1, 1, 160, 0) == 0) ++g_fail;
    if (cad_stack_span_forward_workspace(ls.data(), 0, 1, 8, 0, 1, 1, 160, 0) != 0) ++g_fail;

    // lookup
    EXPECT(cad_ngram_lookup(tok, 16, tok, 1, 0, 1, 4, 0, tok, tok, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_ngram_lookup(tok, 16, tok, 1, 3, 9, 4, 0, tok, tok, nullptr, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_ngram_lookup(tok, 16, tok, 1, 3, 1, 65, 0, tok, tok, nullptr, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_ngram_lookup(tok, 16, tok, 1, 3, 1, 8, 2, tok, tok, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_ngram_lookup(tok, (int64_t)1 << 32, tok, 1, 3, 1, 8, 0, tok, tok, nullptr, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_ngram_lookup(tok, 16, tok, 1, 3, 1, 8, 1, tok, tok, tok, nullptr), CAD_OK, 1);
    EXPECT(cad_ngram_lookup_longest(tok, 16, tok, 1, 2, 3, 1, 8, 0, tok, tok, nullptr, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_ngram_lookup_longest(tok, 16, tok, 1, 65, 1, 1, 8, 0, tok, tok, nullptr, nullptr, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_ngram_lookup_longest(tok, 16, tok, 1, 3, 1, 1, 8, 0, tok, tok, nullptr, tok, nullptr), CAD_OK, 1);

    // accept
    EXPECT(cad_accept_scan(tok, 1, tok, tok, nullptr, 1, 2, 4, CAD_MASK_CAUSAL_SPAN, tok, nullptr, tok, tok, nullptr, 0, nullptr, 0, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_accept_scan(tok, 0, tok, tok, nullptr, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, nullptr, tok, tok, nullptr, 0, nullptr, 0, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_accept_scan(tok, 1, tok, tok, nullptr, 1, 1, 4, CAD_MASK_CAUSAL_SPAN, tok, nullptr, tok, tok, tok, 16, nullptr, 16, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_accept_scan(tok, 1, tok, tok, nullptr, 1, 1, 4, CAD_MASK_CAUSAL_SPAN, tok, nullptr, tok, tok, tok, 16, tok, 32, nullptr, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_accept_scan(tok, 0, tok, tok, tok, 1, 9, 4, CAD_MASK_BLOCK_TRI, tok, nullptr, tok, tok, nullptr, 0, nullptr, 0, nullptr, nullptr), CAD_EUNSUPPORTED, 0);
    EXPECT(cad_accept_scan(tok, 1, tok, tok, nullptr, 1, 1, 4, CAD_MASK_CAUSAL_SPAN, tok, nullptr, tok, tok, tok, 16, tok, 16, &kv, nullptr), CAD_OK, 1);
    EXPECT(cad_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, tok, tok, tok, nullptr, 0, nullptr, 0, &kv, nullptr), CAD_OK, 1);

    // stack accept
    std::vector<cad_kv_desc> k2(2, kv);
    EXPECT(cad_stack_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, tok, tok, tok, nullptr, 0, nullptr, 0, nullptr, 2, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_stack_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, tok, tok, tok, nullptr, 0, nullptr, 0, k2.data(), 0, nullptr), CAD_EINVAL, 0);
    EXPECT(cad_stack_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, nullptr, tok, tok, nullptr, 0, nullptr, 0, k2.data(), 2, nullptr), CAD_EINVAL, 0);
    k2[1].head_dim = 32;
    EXPECT(cad_stack_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, tok, tok, tok, nullptr, 0, nullptr, 0, k2.data(), 2, nullptr), CAD_EINVAL, 0);
    k2[1].head_dim = 64;
    EXPECT(cad_stack_accept_scan(tok, 0, tok, tok, tok, 1, 2, 4, CAD_MASK_BLOCK_TRI, tok, tok, tok, tok, nullptr, 0, nullptr, 0, k2.data(), 2, nullptr), CAD_OK, 2);
    EXPECT(cad_stack_accept_scan(tok, 1, tok, tok, nullptr, 1, 1, 4, CAD_MASK_CAUSAL_SPAN, tok, nullptr, tok, tok, nullptr, 0, nullptr, 0, k2.data(), 2, nullptr), CAD_OK, 1);

    // diagnostics
    if (std::strcmp(cad_status_string(CAD_EWORKSPACE), "workspace missing or too small") != 0) ++g_fail;
    if (std::strcmp(cad_status_string(12345), "unknown status") != 0) ++g_fail;
    if (cad_version() < 100) ++g_fail;
    cad_profile_enable(1);
    EXPECT(cad_span_forward(&d, &kv, tok, 1, 8, 0, 1, 1, 0, tok, nullptr, nullptr, nullptr, ws, big, nullptr), CAD_OK, -1);
    double ms[32] = {0};
    int cnt[32] = {0};
    if (cad_profile_read(32, ms, cnt) <= 0 || cnt[0] != 1) { std::printf("FAIL profiler read\n"); ++g_fail; }
    if (cad_profile_read(0, ms, cnt) != CAD_EINVAL) ++g_fail;
    cad_profile_enable(0);
    if (std::strcmp(cad_profile_stage_name(-1), "unknown") != 0) ++g_fail;

    std::printf(g_fail ? "%d case(s) failed\n" : "all cases passed\n", g_fail);
    return g_fail ? 1 : 0;
}
