// Device helpers shared by the kernels (bf16 bit conversions, exp2,
// output stores, DPP sums).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fd {

constexpr float kLn2f = 0.693147180559945309417f;
constexpr float kLog2ef = 1.4426950408889634074f;

// Hardware v_exp_f32 (2^x); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, int bf16) {
    if (bf16)
        static_cast<uint16_t*>(out)[idx] = to_bf16(v);
    else
        static_cast<float*>(out)[idx] = v;
}

// Loads of the KV cache.  Each cache row is read once per call, so the
// loads carry the non-temporal hint (the nt bit of the gfx950 load), which
// keeps streamed rows from displacing other lines on their way through the
// caches.  On MI355X it raised a cold 16-byte streaming read from about 6.1
// to 7.1 TB/s (1 GiB) and from 5.1 to 5.8 TB/s (64 MiB, 512 workgroups).
typedef uint32_t u32x4_stream_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_stream_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4_stream_t v = __builtin_nontemporal_load(static_cast<const u32x4_stream_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

}  // namespace fd
