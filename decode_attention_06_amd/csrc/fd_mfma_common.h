// Matrix-core helpers shared by the split-KV and bifurcated kernels
// (gfx950, bf16, head_dim 128, v_mfma_f32_16x16x32_bf16).  Internal.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16,
// i = l % 16): A holds row i, k = 8g .. 8g+7; B holds column i, the same k;
// the f32x4 result holds rows 4g .. 4g+3 of column i.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_device.h"

namespace fd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int MF_D = 128;
constexpr int MF_TILE = 32;   // tokens per wave tile
constexpr int MF_NW = 4;      // waves per workgroup (split-KV kernel)

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }


// KV cache loads with the non-temporal hint (see ld_stream16).
__device__ __forceinline__ u32x4_t ld16_kv(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x4_t ld16_kv(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x2_t ld8_kv(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Eight OCP E4M3 codes (two dwords, memory order) -> eight bf16 (four
// dwords), memory order kept (v_cvt_scalef32_pk_bf16_fp8 with scale 1:
// every E4M3 value is exact in bf16).
__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return r;
}

// Column e of the 8x8 bf16 block r[0..7] (row j = r[j], 8 elements each):
// {r[0][e], r[1][e], ..., r[7][e]}, packed two per dword.
template <int E>
__device__ __forceinline__ u32x4_t block_column(const u32x4_t (&r)[8]) {
    constexpr uint32_t sel = (E & 1) ? 0x07060302u : 0x05040100u;
    constexpr int dw = E >> 1;
    u32x4_t c;
    c[0] = __builtin_amdgcn_perm(r[1][dw], r[0][dw], sel);
    c[1] = __builtin_amdgcn_perm(r[3][dw], r[2][dw], sel);
    c[2] = __builtin_amdgcn_perm(r[5][dw], r[4][dw], sel);
    c[3] = __builtin_amdgcn_perm(r[7][dw], r[6][dw], sel);
    return c;
}

template <int E, int NRB>
__device__ __forceinline__ void pv_block(const u32x4_t (&vr)[8], const bf16x8_t (&pb)[NRB],
                                         f32x4_t (&acc)[NRB][8]) {
    const bf16x8_t va = as_bf16x8(block_column<E>(vr));
#pragma unroll
    for (int r = 0; r < NRB; ++r) acc[r][E] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[r], acc[r][E], 0, 0, 0);
}

// One 32-token tile of the online softmax for NRB blocks of 16 query rows,
// in three parts: scores S^T = K Q^T on the matrix cores (K in kr: token
// block blk, k-step s, lane (g, i) holds token 8*(i/4) + 4*blk + i%4,
// d = 32s + 8g .. +8); the softmax step (running max per query row m, log2
// domain; running sum lacc, every component holding the row's sum) giving
// the bf16 weights of this lane's tokens 8g .. 8g+7; and O^T += V^T P^T,
// where the V^T operand of output block e comes from the caller.  Tokens at
// or beyond t1 get weight 0.
// The running maximum m is a reference, not necessarily the exact maximum:
// it is raised only when a score exceeds it by more than MF_RESCALE_SLACK
// (log2 units), so weights stay below 2^MF_RESCALE_SLACK and the costly
// rescale of the accumulators is skipped for almost every tile.  Output
// (acc / l) and lse (m + log2 l) do not depend on the reference chosen.
constexpr float MF_RESCALE_SLACK = 8.0f;

template <int NRB>
__device__ __forceinline__ void tile_scores(const u32x4_t (&kr)[2][4], const bf16x8_t (&qb)[NRB][4],
                                            f32x4_t (&sc)[NRB][2]) {
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sc[r][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sc[r][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[blk][s]), qb[r][s], sc[r][blk], 0, 0, 0);
        }
}

// tmask (wave-uniform): no token below it is masked for any row of the
// wave; lim[r]: the lane's row of block r sees tokens below lim[r] only.
template <int NRB>
__device__ __forceinline__ void tile_softmax(const f32x4_t (&sc)[NRB][2], int tb, int tmask, const int (&lim)[NRB],
                                             int g, float sl2, float (&m)[NRB], f32x4_t (&lacc)[NRB],
                                             f32x4_t (&acc)[NRB][8], bf16x8_t (&pb)[NRB]) {
    // A block of bf16 ones: O^T rows of ones(16 x 32) P^T give the row sums of
    // the very weights used in P V, accumulated in fp32 by the matrix core.
    const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    // Raw scores q.k of this lane's query rows for tokens tb + 8g + j.
    float t[NRB][8];
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) t[r][j] = sc[r][j >> 2][j & 3];
    // Only tiles reaching tmask hold masked tokens (a piece's last tile, a
    // causal diagonal).  The empty asm statements keep this a branch: folded
    // into selects it would run on every tile.
    if (tb + MF_TILE > tmask) {
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (tb + 8 * g + j >= lim[r]) t[r][j] = -INFINITY;
                asm volatile("" : "+v"(t[r][j]));
            }
    }
    // This lane's maximum per row block, against the reference (log2
    // domain, scale * log2(e) folded in; sl2 > 0).
    float mx[NRB];
    bool raise = false;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        mx[r] = t[r][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx[r] = fmaxf(mx[r], t[r][j]);
        raise = raise || (mx[r] * sl2 > m[r] + MF_RESCALE_SLACK);
    }
    // Rare path: some score passed its row's reference by more than the
    // slack.  Form the row maxima over the four lane groups and raise every
    // row's reference, identically in all lanes of the row.
    if (__any(raise)) {
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            float x = fmaxf(mx[r], __shfl_xor(mx[r], 16));
            x = fmaxf(x, __shfl_xor(x, 32));
            const float mn = fmaxf(m[r], x * sl2);
            const float alpha = fast_exp2(m[r] - ((mn == -INFINITY) ? 0.f : mn));
            lacc[r] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
            m[r] = mn;
        }
    }
    // Weights exp2(s * sl2 - ref), rounded to bf16 for the matrix products.
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const float ref = (m[r] == -INFINITY) ? 0.f : m[r];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            bf16x2_t w2;
            w2.x = (__bf16)fast_exp2(fmaf(t[r][j], sl2, -ref));
            w2.y = (__bf16)fast_exp2(fmaf(t[r][j + 1], sl2, -ref));
            pb[r][j] = w2.x;
            pb[r][j + 1] = w2.y;
        }
        lacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[r], lacc[r], 0, 0, 0);
    }
}

// Whole tile with V held as the lane's 8x8 block (tokens 8g .. 8g+7,
// d = 8i .. 8i+7), transposed in registers: output row m of block e is
// d = 8m + e.
template <int NRB>
__device__ __forceinline__ void compute_tile(const u32x4_t (&kr)[2][4], const u32x4_t (&vr)[8],
                                             const bf16x8_t (&qb)[NRB][4], int tb, int t1, int g, float sl2,
                                             float (&m)[NRB], f32x4_t (&lacc)[NRB], f32x4_t (&acc)[NRB][8]) {
    f32x4_t sc[NRB][2];
    tile_scores<NRB>(kr, qb, sc);
    bf16x8_t pb[NRB];
    int lim[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) lim[r] = t1;
    tile_softmax<NRB>(sc, tb, t1, lim, g, sl2, m, lacc, acc, pb);
    pv_block<0>(vr, pb, acc);
    pv_block<1>(vr, pb, acc);
    pv_block<2>(vr, pb, acc);
    pv_block<3>(vr, pb, acc);
    pv_block<4>(vr, pb, acc);
    pv_block<5>(vr, pb, acc);
    pv_block<6>(vr, pb, acc);
    pv_block<7>(vr, pb, acc);
}

}  // namespace
}  // namespace fd
