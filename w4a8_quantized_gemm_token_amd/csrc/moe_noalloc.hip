// moe_noalloc.hip -- the MoE FFN layer for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// w4a8_moe_ffn takes its intermediates (routing tables, codes, gate/up and down
// outputs) in a caller workspace.  w4a8_moe_ffn_noalloc runs the same kernels over a
// file-scope device array instead: kNoAllocScratchBytes per GPU, held from the
// library's load until the process ends.  Host code never passes the array's name to
// a kernel (in host code it is a stand-in, not a device address): each device's
// address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is used.  Nothing in the layer needs the array
// cleared first (every part is written before it is read).  Calls that overlap on
// one GPU share the array and race; the caller orders them (one stream, or events).
#include <mutex>

#include "w4a8_internal.hpp"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (looked up once per device).
hipError_t scratch_for_current_device(void **ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t w4a8_moe_ffn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

w4a8_status w4a8_moe_ffn_noalloc(const float *x, const float *logits, int64_t T, int64_t H, int64_t I, int32_t E,
                                 int32_t topk, const uint8_t *gu_packed, const uint16_t *gu_scale,
                                 const uint16_t *gu_zp, const uint8_t *dn_packed, const uint16_t *dn_scale,
                                 const uint16_t *dn_zp, float *out, hipStream_t stream) {
    w4a8::clear_error();
    const int64_t need = w4a8::moe_ffn_ws_bytes(T, H, I, E, topk);
    if (need < 0)  // invalid sizes: the layer reports which
        return w4a8::moe_ffn_run(x, logits, T, H, I, E, topk, gu_packed, gu_scale, gu_zp, dn_packed, dn_scale, dn_zp,
                                 out, nullptr, 0, stream);
    if (need > (int64_t)kNoAllocScratchBytes) {
        w4a8::set_error("moe_ffn_noalloc: the layer needs %lld bytes of intermediates, the fixed scratch holds %zu "
                        "(use w4a8_moe_ffn with a workspace)",
                        (long long)need, kNoAllocScratchBytes);
        return W4A8_EWORKSPACE;
    }
    void *ws = nullptr;
    hipError_t err = scratch_for_current_device(&ws);
    if (err != hipSuccess) return w4a8::hip_status(err, "moe_ffn_noalloc: scratch address");
    return w4a8::moe_ffn_run(x, logits, T, H, I, E, topk, gu_packed, gu_scale, gu_zp, dn_packed, dn_scale, dn_zp, out,
                             ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
