// The allocation-free span forward: cad_span_forward with its workspace taken from a static device
// array, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// Every device the library runs on holds its own copy of `scratch` from the code object's load
// until the process ends.  In host code the name `scratch` is a host-side stand-in, never a device
// address: the array's address on a device comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the first call there and kept in g_scratch_ptr[device]; only that
// pointer is ever handed to the kernels.
#include <mutex>

#include "cad_internal.h"

namespace {

constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[CAD_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices] = {nullptr};
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or nullptr on failure.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int cad_span_forward_noalloc(const cad_layer_desc* L, const cad_kv_desc* kv, const int32_t* tokens, int B,
                                        int Nq, int mode, int W, int D, int flags, int32_t* argmax_out,
                                        void* hidden_out, float* logits_out, float* top2_gap, hipStream_t stream) {
    if (!L || !kv) return CAD_EINVAL;
    FwdDims fd;
    if (!fwd_dims(L, B, Nq, mode, W, D, kv->cap, &fd)) return CAD_EINVAL;
    // the size this forward needs, as cad_span_forward_workspace reports it; nothing larger fits
    if (fwd_carve(fd, nullptr, (flags & CAD_KV_ONLY) != 0).total > (size_t)CAD_NOALLOC_SCRATCH_BYTES)
        return CAD_EWORKSPACE;
    void* ws = scratch_ptr();
    if (!ws) return CAD_EHIP;
    return span_forward_internal(L, kv, tokens, B, Nq, mode, W, D, flags, argmax_out, hidden_out, logits_out, top2_gap,
                                 ws, (size_t)CAD_NOALLOC_SCRATCH_BYTES, stream);
}
