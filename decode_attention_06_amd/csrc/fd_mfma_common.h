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

#include <type_traits>

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

// Output block E of O^T += V^T P^T for weights given as two bf16 parts,
// pb (rounded weight) and pl (rounded remainder): two products per block.
template <int E, int NRB>
__device__ __forceinline__ void pv_block(const u32x4_t (&vr)[8], const bf16x8_t (&pb)[NRB],
                                         const bf16x8_t (&pl)[NRB], f32x4_t (&acc)[NRB][8]) {
    const bf16x8_t va = as_bf16x8(block_column<E>(vr));
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        acc[r][E] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[r], acc[r][E], 0, 0, 0);
        acc[r][E] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[r], acc[r][E], 0, 0, 0);
    }
}

// Output block E for one B operand holding both weight parts (PACK below).
template <int E>
__device__ __forceinline__ void pv_packed(const u32x4_t (&vr)[8], const bf16x8_t& pp, f32x4_t (&acc)[8]) {
    acc[E] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(block_column<E>(vr)), pp, acc[E], 0, 0, 0);
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

// The k-steps run outermost, so consecutive products go to different
// accumulators (2 NRB independent chains) instead of one chain of four
// dependent products at a time.
template <int NRB>
__device__ __forceinline__ void tile_scores(const u32x4_t (&kr)[2][4], const bf16x8_t (&qb)[NRB][4],
                                            f32x4_t (&sc)[NRB][2]) {
#pragma unroll
    for (int r = 0; r < NRB; ++r)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) sc[r][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                sc[r][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[blk][s]), qb[r][s], sc[r][blk], 0, 0, 0);
}

// tmask (wave-uniform): no token below it is masked for any row of the
// wave; lim[r]: the lane's row of block r sees tokens below lim[r] only.
//
// SPLIT: each fp32 weight w leaves as two bf16 values, pb = w cut to its
// top 16 bits and pl = bf16(w - pb) (w - pb is exact in fp32).  pb + pl is
// within 2^-17 |w| of w, so the weights the products see are fp32-accurate
// and the output error no longer grows with the spread of V (one bf16 weight
// is off by up to 2^-9 |w|: about 2^-9 |v1 - v2| at the output).  The running sum
// then takes the fp32 weights themselves: `lsum` (a float per row) holds the
// sum over this lane's tokens only, and the caller adds the four lane
// groups of a row at the end.  Without SPLIT, `lsum` is an f32x4 whose
// every component holds the whole row's sum of the bf16 weights (a matrix
// product against a block of ones), so numerator and denominator use
// identical weights.  SPLIT doubles the P.V products, which the HBM-bound
// split-KV kernels have to spare; the kernels whose matrix cores are the
// bottleneck (many query rows per KV tile) keep one bf16 weight.
//
// PACK (see compute_tile): accumulator columns 8..15 hold the remainder
// shares of rows 0..7, so a rescale applies row i's factor to column i + 8;
// the running sum is then an f32x4 formed like the accumulators, by a
// product of a block of ones with the packed weights (compute_tile), and
// column i + 8 of it holds row i's remainder sum.
template <int NRB, bool SPLIT, typename SumT, bool PACK = false>
__device__ __forceinline__ void tile_softmax(const f32x4_t (&sc)[NRB][2], int tb, int tmask, const int (&lim)[NRB],
                                             int g, float sl2, float (&m)[NRB], SumT (&lsum)[NRB],
                                             f32x4_t (&acc)[NRB][8], bf16x8_t (&pb)[NRB], bf16x8_t (&pl)[NRB]) {
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
            float acc_alpha = alpha;
            if constexpr (PACK) {
                // row_shr:8 into banks 2 and 3: lane i + 8 of a 16-lane row
                // takes lane i's factor, lanes 0..7 keep their own
                acc_alpha = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(alpha), __float_as_int(alpha),
                                                                        0x118, 0xF, 0xC, false));
            }
            // PACK: the sums' columns 8..15 are rows 0..7's remainder sums too
            lsum[r] *= PACK ? acc_alpha : alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= acc_alpha;
            m[r] = mn;
        }
    }
    // Weights exp2(s * sl2 - ref), rounded to bf16 for the matrix products
    // (with SPLIT, the rounded remainder as well).
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const float ref = (m[r] == -INFINITY) ? 0.f : m[r];
        if constexpr (SPLIT) {
            // pb: w cut to its top 16 bits (a bf16 value, exact as a float);
            // pl: the exact remainder w - pb rounded to bf16.  Both parts
            // together are within 2^-17 w of w.
            u32x4_t hw, lw;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float w0 = fast_exp2(fmaf(t[r][j], sl2, -ref));
                const float w1 = fast_exp2(fmaf(t[r][j + 1], sl2, -ref));
                const uint32_t u0 = __float_as_uint(w0), u1 = __float_as_uint(w1);
                hw[j >> 1] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // top halves of w0, w1
                bf16x2_t r2;
                r2.x = (__bf16)(w0 - __uint_as_float(u0 & 0xffff0000u));
                r2.y = (__bf16)(w1 - __uint_as_float(u1 & 0xffff0000u));
                lw[j >> 1] = __builtin_bit_cast(uint32_t, r2);
                if constexpr (!PACK) lsum[r] += w0 + w1;
            }
            pb[r] = __builtin_bit_cast(bf16x8_t, hw);
            pl[r] = __builtin_bit_cast(bf16x8_t, lw);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                bf16x2_t w2;
                w2.x = (__bf16)fast_exp2(fmaf(t[r][j], sl2, -ref));
                w2.y = (__bf16)fast_exp2(fmaf(t[r][j + 1], sl2, -ref));
                pb[r][j] = w2.x;
                pb[r][j + 1] = w2.y;
            }
            lsum[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[r], lsum[r], 0, 0, 0);
        }
    }
}

// Whole tile with V held as the lane's 8x8 block (tokens 8g .. 8g+7,
// d = 8i .. 8i+7), transposed in registers: output row m of block e is
// d = 8m + e.  Split-KV kernels: weights in two bf16 parts (SPLIT above).
//
// PACK (one 16-row block holding at most 8 query rows, G <= 8): the
// B-operand columns of the padding rows 8..15 carry the remainders of rows
// 0..7 instead (moved over by 8 lanes within each 16-lane DPP row), so one
// product per output block takes both parts; column i + 8 of the result
// then holds row i's remainder share, which pack_fold() adds back once per
// piece.
template <bool PACK>
using SplitSum = typename std::conditional<PACK, f32x4_t, float>::type;

template <int NRB, bool PACK = false>
__device__ __forceinline__ void compute_tile(const u32x4_t (&kr)[2][4], const u32x4_t (&vr)[8],
                                             const bf16x8_t (&qb)[NRB][4], int tb, int t1, int g, float sl2,
                                             float (&m)[NRB], SplitSum<PACK> (&lsum)[NRB], f32x4_t (&acc)[NRB][8]) {
    static_assert(!PACK || NRB == 1, "packing needs one block with spare columns");
    f32x4_t sc[NRB][2];
    tile_scores<NRB>(kr, qb, sc);
    bf16x8_t pb[NRB], pl[NRB];
    int lim[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) lim[r] = t1;
    tile_softmax<NRB, true, SplitSum<PACK>, PACK>(sc, tb, t1, lim, g, sl2, m, lsum, acc, pb, pl);
    if constexpr (PACK) {
        const u32x4_t hi = __builtin_bit_cast(u32x4_t, pb[0]);
        const u32x4_t lo = __builtin_bit_cast(u32x4_t, pl[0]);
        u32x4_t pk;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // row_shr:8 written to banks 2 and 3 only (lanes 8..15 of each
            // 16-lane row take lane i's remainder); lanes 0..7 keep pb
            pk[k] = (uint32_t)__builtin_amdgcn_update_dpp((int)hi[k], (int)lo[k], 0x118, 0xF, 0xC, false);
        }
        const bf16x8_t pp = __builtin_bit_cast(bf16x8_t, pk);
        if constexpr (PACK) {
            const bf16x8_t ones = as_bf16x8(u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
            lsum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pp, lsum[0], 0, 0, 0);
        }
        pv_packed<0>(vr, pp, acc[0]);
        pv_packed<1>(vr, pp, acc[0]);
        pv_packed<2>(vr, pp, acc[0]);
        pv_packed<3>(vr, pp, acc[0]);
        pv_packed<4>(vr, pp, acc[0]);
        pv_packed<5>(vr, pp, acc[0]);
        pv_packed<6>(vr, pp, acc[0]);
        pv_packed<7>(vr, pp, acc[0]);
        return;
    }
    pv_block<0>(vr, pb, pl, acc);
    pv_block<1>(vr, pb, pl, acc);
    pv_block<2>(vr, pb, pl, acc);
    pv_block<3>(vr, pb, pl, acc);
    pv_block<4>(vr, pb, pl, acc);
    pv_block<5>(vr, pb, pl, acc);
    pv_block<6>(vr, pb, pl, acc);
    pv_block<7>(vr, pb, pl, acc);
}

// PACK: adds column i + 8 of every accumulator (row i's remainder share)
// into column i (row_shl:8 -- lane i of a 16-lane row reads lane i + 8).
// Columns 8..15 are meaningless afterwards.
__device__ __forceinline__ void pack_fold(f32x4_t (&acc)[1][8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[0][e][ii] += dpp<0x108>(acc[0][e][ii]);
}

}  // namespace
}  // namespace fd
