// fd_decode_attn_noalloc: fd_decode_attn for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid hipMalloc).  The per-piece partials that fd_decode_attn keeps
// in the caller's workspace live here in one fixed array of this library,
// `scratch`, of FD_NOALLOC_MAX_WORKSPACE bytes.  Each GPU the library runs
// on holds its own copy of the array until the process ends; every call on
// one GPU uses that GPU's copy, so calls that overlap on one GPU race.
//
// The array's name is a host-side stand-in in host code; its device
// address comes from hipGetSymbolAddress, once per device (with that
// device current), and only that address is handed to the kernels.
#include "fd.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "fd_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[FD_NOALLOC_MAX_WORKSPACE];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;   // per device ordinal: device address of scratch

// Device address of this device's copy of `scratch`.
fd_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fd::set_error(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (dev >= int(g_scratch_ptr.size())) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fd::set_error(FD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                 hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FD_OK;
}

}  // namespace

extern "C" fd_status fd_decode_attn_noalloc(const void* q, const void* k, const void* v, const int32_t* lens,
                                            int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int64_t max_len, int32_t dtype, int32_t n_splits,
                                            void* out, int32_t out_dtype, float* lse_out, float scale,
                                            void* stream) {
    // Resolve the split count once, so the size checked here is the size
    // fd_decode_attn uses.
    int32_t ns = n_splits;
    if (ns <= 0) {
        int32_t cus = 0;
        const fd_status s = fd_device_cu_count(&cus);
        if (s != FD_OK) return s;
        ns = fd_plan_splits(batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, cus);
        if (ns <= 0) return fd::set_error(FD_ERR_INVALID_ARG, "invalid shapes for the split planner");
    }
    size_t need = 0;
    fd_status s = fd_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, ns,
                                                &need);
    if (s != FD_OK) return s;
    if (need > size_t(FD_NOALLOC_MAX_WORKSPACE))
        return fd::set_error(FD_ERR_WORKSPACE,
                             "%zu bytes of partials (%d pieces for %d x %d query rows) exceed the %zu bytes "
                             "the allocation-free entry point holds; use fd_decode_attn with a workspace",
                             need, ns, batch, num_q_heads, size_t(FD_NOALLOC_MAX_WORKSPACE));
    // The pointer checks fd_decode_attn makes, here too, so that they still
    // come before the first HIP call (the array's address lookup).
    auto misaligned = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; };
    if (!q || !k || !v || !out) return fd::set_error(FD_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16))
        return fd::set_error(FD_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (misaligned(lens, 4) || misaligned(lse_out, 4))
        return fd::set_error(FD_ERR_INVALID_ARG, "lens and lse_out must be 4-byte aligned");
    void* ws = nullptr;
    if (need > 0) {
        s = scratch_address(&ws);
        if (s != FD_OK) return s;
    }
    return fd_decode_attn(q, k, v, lens, batch, num_q_heads, num_kv_heads, head_dim, max_len, dtype, ns, out,
                          out_dtype, lse_out, scale, ws, need > 0 ? size_t(FD_NOALLOC_MAX_WORKSPACE) : 0, stream);
}
