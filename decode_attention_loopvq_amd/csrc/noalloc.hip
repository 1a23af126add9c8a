// lvq_decode_attn_noalloc: lvq_decode_attn with its workspace in library-held device memory, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace is a file-scope device array, one copy per GPU, alive until the process ends.  Its name
// is a host-side stand-in in host code, never a device address: the address each GPU gives it is asked
// for once per device, with that device current, and only that address reaches the kernels.
#include "common.h"

#include <mutex>

namespace lvq {
namespace {

constexpr size_t kScratchBytes = LVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call per device.
lvq_status device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    LVQ_REQUIRE(e == hipSuccess, LVQ_ERR_HIP, "lvq_decode_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    LVQ_REQUIRE(dev >= 0 && dev < kMaxDevices, LVQ_ERR_UNSUPPORTED, "lvq_decode_attn_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        LVQ_REQUIRE(e == hipSuccess && p, LVQ_ERR_HIP, "lvq_decode_attn_noalloc: hipGetSymbolAddress: %s",
                    hipGetErrorString(e));
        LVQ_REQUIRE(reinterpret_cast<uintptr_t>(p) % 256 == 0, LVQ_ERR_HIP,
                    "lvq_decode_attn_noalloc: scratch not 256-byte aligned");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LVQ_OK;
}

// Workspace of a valid call: the current device's scratch, if the call fits in it.
lvq_status scratch_workspace(size_t need, void** ws, size_t* ws_bytes) {
    LVQ_REQUIRE(need <= kScratchBytes, LVQ_ERR_WORKSPACE,
                "lvq_decode_attn_noalloc: the call needs %zu bytes of workspace, above the %zu bytes held per GPU",
                need, kScratchBytes);
    const lvq_status st = device_scratch(ws);
    if (st != LVQ_OK) return st;
    *ws_bytes = kScratchBytes;
    return LVQ_OK;
}

}  // namespace
}  // namespace lvq

extern "C" lvq_status lvq_decode_attn_noalloc(const lvq_geom* gp, int32_t step, const void* q, const uint8_t* pool,
                                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_len,
                                              int32_t max_len, const int32_t* order, const void* k_scales,
                                              const void* win_k, const void* win_v, const void* slices,
                                              const float* rope_cos, const float* rope_sin, const void* rope_f16,
                                              int32_t rope_len, float sm_scale, float* out, float* lse_out,
                                              int32_t num_splits, int32_t B, hipStream_t stream) {
    return lvq::decode_attn_impl("lvq_decode_attn_noalloc", gp, step, q, pool, page_table, pt_stride, seq_len, max_len,
                                 order, k_scales, win_k, win_v, slices, rope_cos, rope_sin, rope_f16, rope_len,
                                 sm_scale, out, lse_out, nullptr, 0, &lvq::scratch_workspace, num_splits, B, stream);
}
