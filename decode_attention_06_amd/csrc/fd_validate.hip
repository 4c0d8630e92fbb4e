// Optional device-side argument validation (FD_VALIDATE=1 in the
// environment when the library is first used, or fd_set_validation).
//
// The lengths and block tables an entry point reads live in device memory,
// so the host checks cannot see them without a synchronisation.  With
// validation on, each call first counts the out-of-range entries on the
// device, waits for the count and returns FD_ERR_INVALID_ARG (naming the
// first bad entry) before any attention kernel is launched.  This is a
// debugging aid: it synchronises the stream and therefore refuses to run
// under stream capture.
#include "fd.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "fd_internal.h"

namespace {

// [0]: number of bad entries, [1]: lowest bad index (per device).
__device__ __align__(16) int32_t check_word[2];

std::once_flag g_env_once;
int g_validate = 0;            // 1: validation on
std::mutex g_word_mutex;
std::vector<int32_t*> g_word;  // per device ordinal: device address of check_word

void read_env() {
    const char* e = std::getenv("FD_VALIDATE");
    g_validate = (e && std::strcmp(e, "0") != 0 && e[0] != '\0') ? 1 : 0;
}

fd_status word_address(int32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fd::set_error(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_word_mutex);
    if (dev >= int(g_word.size())) g_word.resize(dev + 1, nullptr);
    if (!g_word[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_word));
        if (e != hipSuccess || !p)
            return fd::set_error(FD_ERR_HIP, "hipGetSymbolAddress(check_word): %s", hipGetErrorString(e));
        g_word[dev] = static_cast<int32_t*>(p);
    }
    *out = g_word[dev];
    return FD_OK;
}

__global__ void reset_word(int32_t* w) {
    w[0] = 0;
    w[1] = INT32_MAX;
}

__device__ __forceinline__ void flag_bad(int32_t* w, int32_t i) {
    atomicAdd(&w[0], 1);
    atomicMin(&w[1], i);
}

__global__ void check_lens_kernel(const int32_t* lens, int32_t n, int64_t lo, int64_t hi, int32_t* w) {
    const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const int64_t v = lens[i];
        if (v < lo || v > hi) flag_bad(w, i);
    }
}

// Entry (b, j) of a [B, cols] table covers rows [j * page, (j + 1) * page);
// it is read when j * page < lens[b] (or < rows when lens is NULL).
__global__ void check_table_kernel(const int32_t* table, const int32_t* lens, int32_t B, int32_t cols,
                                   int64_t page, int64_t rows, int32_t n_pages, int32_t* w) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)B * cols) return;
    const int32_t b = (int32_t)(idx / cols), j = (int32_t)(idx % cols);
    const int64_t n = lens ? (int64_t)lens[b] : rows;
    if ((int64_t)j * page < n) {
        const int32_t id = table[idx];
        if (id < 0 || id >= n_pages) flag_bad(w, (int32_t)min(idx, (int64_t)INT32_MAX));
    }
}

// Waits for the count; returns FD_OK or FD_ERR_INVALID_ARG naming the first
// bad entry.
fd_status collect(int32_t* w, hipStream_t s, const char* what) {
    int32_t host[2] = {0, 0};
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(host, w, sizeof(host), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fd::set_error(FD_ERR_HIP, "validation of %s: %s", what, hipGetErrorString(e));
    if (host[0] != 0)
        return fd::set_error(FD_ERR_INVALID_ARG, "%s: %d entries out of range, the first at index %d (FD_VALIDATE)",
                             what, host[0], host[1]);
    return FD_OK;
}

fd_status begin(hipStream_t s, int32_t** w) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
        return fd::set_error(FD_ERR_UNSUPPORTED, "validation (FD_VALIDATE) synchronises the stream and cannot run "
                                                 "under stream capture");
    const fd_status st = word_address(w);
    if (st != FD_OK) return st;
    hipLaunchKernelGGL(reset_word, dim3(1), dim3(1), 0, s, *w);
    return FD_OK;
}

}  // namespace

namespace fd {

bool validation_on() {
    std::call_once(g_env_once, read_env);
    return __atomic_load_n(&g_validate, __ATOMIC_RELAXED) != 0;
}

fd_status validate_lens(const int32_t* lens, int64_t n, int64_t lo, int64_t hi, const char* what, hipStream_t s) {
    if (!lens || n <= 0 || !validation_on()) return FD_OK;
    int32_t* w = nullptr;
    const fd_status st = begin(s, &w);
    if (st != FD_OK) return st;
    hipLaunchKernelGGL(check_lens_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, lens, (int32_t)n, lo,
                       hi, w);
    return collect(w, s, what);
}

fd_status validate_table(const int32_t* table, const int32_t* lens, int32_t B, int32_t cols, int32_t page_size,
                         int64_t rows, int32_t n_pages, hipStream_t s) {
    if (!validation_on()) return FD_OK;
    int32_t* w = nullptr;
    const fd_status st = begin(s, &w);
    if (st != FD_OK) return st;
    const int64_t n = (int64_t)B * cols;
    hipLaunchKernelGGL(check_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, lens, B, cols,
                       (int64_t)page_size, rows, n_pages, w);
    return collect(w, s, "block_table (page ids of the rows in use)");
}

}  // namespace fd

extern "C" fd_status fd_set_validation(int32_t on) {
    std::call_once(g_env_once, read_env);
    __atomic_store_n(&g_validate, on ? 1 : 0, __ATOMIC_RELAXED);
    return FD_OK;
}

extern "C" int32_t fd_validation_enabled(void) { return fd::validation_on() ? 1 : 0; }
