// Split-KV partial kernel on the MFMA matrix cores (gfx950, bf16, D = 128).
//
// Method: [FD] "¿Qué es Flash-Decoding y cuándo acelera los LLMs?"
// (slavadubrov.com), section "Por qué la decodificación necesita otra
// planificación" (pieces of the history -> partial output + log-sum-exp);
// [FA] "In che modo Flash Attention riduce il traffico di memoria durante
// l'inferenza locale?" (shop.zimaspace.com), sections on tiling and on the
// online softmax.  [BA] "Effiziente Verarbeitung ... bifurkierte
// Aufmerksamkeit ..." (linnk.ai), section "Tilastot": the G query heads of a
// KV head share its K/V rows, so the rows are read once and contracted
// against all G queries: a small dense product, which is what the matrix
// cores are for.
//
// Layout of one wave's 32-token tile (v_mfma_f32_16x16x32_bf16; lane l,
// g = l / 16, i = l % 16):
//  * Scores S^T = K Q^T, tokens on M, query rows on N, d on K.  A-operand
//    lane (g, i) of token block blk, k-step s holds K[token tau][32s + 8g ..
//    +8) with tau = 8*(i/4) + 4*blk + i%4; B-operand holds q[row i][same d].
//    The accumulator then gives lane (g, i) the scores of query row i for
//    tokens 8g .. 8g+7 (blk 0: +0..3, blk 1: +4..7).
//  * Those eight scores, as bf16 weights, are exactly the lane's B operand of
//    O^T += V^T P^T (k-slot 8g + j <-> token 8g + j).
//  * V^T A operand for output block e holds, in lane (g, i),
//    V[token 8g + j][8i + e] for j = 0..7: the lane loads V rows 8g .. 8g+7,
//    columns 8i .. 8i+7 (eight coalesced 16-byte loads) and transposes that
//    8x8 block in registers.  Output row m of block e is d = 8m + e.
//  No LDS is needed inside the token loop; each KV byte is loaded once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"

namespace fd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int MF_D = 128;
constexpr int MF_TILE = 32;   // tokens per wave tile
constexpr int MF_NW = 4;      // waves per workgroup

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

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

// Loads one 32-token tile starting at row tb (tb < t1): K in score
// A-operand layout, V as this lane's 8x8 block (rows 8g .. 8g+7, columns
// 8i .. 8i+7).  Every load is issued unconditionally; a row index at or
// beyond t1 is clamped to t1 - 1, a valid row, whose score is masked to -inf
// later, so no row past the sequence length is ever read.
__device__ __forceinline__ void load_tile(const uint16_t* kbase, const uint16_t* vbase, int tb, int t1,
                                          int ktok0, int g, int i, u32x4_t (&kr)[2][4], u32x4_t (&vr)[8]) {
    const int last = t1 - 1;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int t = min(tb + ktok0 + 4 * blk, last);
        const uint16_t* src = kbase + (int64_t)t * MF_D + 8 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[blk][s] = ld16(src + 32 * s);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = min(tb + 8 * g + j, last);
        vr[j] = ld16(vbase + (int64_t)t * MF_D + 8 * i);
    }
}

// One tile of the online softmax: scores on the matrix cores, running max /
// running sum update per query row, then O^T += V^T P^T.
template <int NRB>
__device__ __forceinline__ void compute_tile(const u32x4_t (&kr)[2][4], const u32x4_t (&vr)[8],
                                             const bf16x8_t (&qb)[NRB][4], int tb, int t1, int g, float sl2,
                                             float (&m)[NRB], float (&l)[NRB], f32x4_t (&acc)[NRB][8]) {
    const bool full = tb + MF_TILE <= t1;
    bf16x8_t pb[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        f32x4_t sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sc[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[blk][s]), qb[r][s], sc[blk], 0, 0, 0);
        }
        // Scores of this lane's query row for tokens tb + 8g + j, log2 domain.
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            t[j] = sc[j >> 2][j & 3] * sl2;
            if (!full && tb + 8 * g + j >= t1) t[j] = -INFINITY;
        }
        float mx = t[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, t[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[r], mx);
        const float ref = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m[r] - ref);
        // Weights rounded to bf16 for the matrix product; the running sum
        // adds the same rounded values, so numerator and denominator agree.
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            bf16x2_t w2;
            w2.x = (__bf16)fast_exp2(t[j] - ref);
            w2.y = (__bf16)fast_exp2(t[j + 1] - ref);
            pb[r][j] = w2.x;
            pb[r][j + 1] = w2.y;
            lsum += (float)w2.x + (float)w2.y;
        }
        l[r] = l[r] * alpha + lsum;
        m[r] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
    }
    pv_block<0>(vr, pb, acc);
    pv_block<1>(vr, pb, acc);
    pv_block<2>(vr, pb, acc);
    pv_block<3>(vr, pb, acc);
    pv_block<4>(vr, pb, acc);
    pv_block<5>(vr, pb, acc);
    pv_block<6>(vr, pb, acc);
    pv_block<7>(vr, pb, acc);
}

// NRB blocks of 16 query rows per work unit share every K/V load.
template <int NRB>
__global__ __launch_bounds__(256, (NRB == 1) ? 2 : 1) void partial_mfma_kernel(const PartialParams p) {
    constexpr int D = MF_D, NW = MF_NW, ROWS = 16 * NRB;
    __shared__ float s_acc[NW][ROWS][D];
    __shared__ float s_m[NW][ROWS];
    __shared__ float s_l[NW][ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
    const int g = lane >> 4, i = lane & 15;

    int idx = blockIdx.x;
    const int split = idx % p.n_splits;
    idx /= p.n_splits;
    const int rblk = idx % p.row_blocks;
    idx /= p.row_blocks;
    const int kvh = idx % p.Hkv;
    const int b = idx / p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int h0 = kvh * G + rblk * ROWS;
    const int nr = min(ROWS, G - rblk * ROWS);   // valid query rows in this unit

    int n = p.lens ? p.lens[b] : (int)p.Lmax;
    n = max(0, min(n, (int)p.Lmax));
    const int chunk = ((n + p.n_splits - 1) / p.n_splits + 15) & ~15;
    const int t0 = (int)min((int64_t)split * chunk, (int64_t)n);
    const int t1 = min(t0 + chunk, n);

    // Q^T fragments (B operand of the score product); rows >= nr are zero.
    bf16x8_t qb[NRB][4];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        const int row = r * 16 + i;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row < nr)
                v = ld16(static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h0 + row) * D + 32 * s + 8 * g);
            qb[r][s] = as_bf16x8(v);
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + (int64_t)b * p.kv_stride_b + (int64_t)kvh * p.kv_stride_h;
    const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + (int64_t)b * p.kv_stride_b + (int64_t)kvh * p.kv_stride_h;
    // Token offsets inside a tile for this lane's K rows (one per token block).
    const int ktok0 = 8 * (i >> 2) + (i & 3);
    const float sl2 = p.scale_log2;

    f32x4_t acc[NRB][8];
    float m[NRB], l[NRB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Two register buffers, alternating: the next tile's loads are in
    // flight while the current tile is computed.  The prefetch is issued
    // even past the piece's end (its rows clamp to t1 - 1, cache hits), so
    // every path leaves the same number of loads outstanding and the wait
    // before each tile covers only that tile's own loads.
    constexpr int STEP = NW * MF_TILE;
    u32x4_t ka[2][4], va[8], kb2[2][4], vb2[8];
    int tb = t0 + wave * MF_TILE;
    if (tb < t1) {
        load_tile(kbase, vbase, tb, t1, ktok0, g, i, ka, va);
        while (true) {
            load_tile(kbase, vbase, tb + STEP, t1, ktok0, g, i, kb2, vb2);
            compute_tile<NRB>(ka, va, qb, tb, t1, g, sl2, m, l, acc);
            tb += STEP;
            if (tb >= t1) break;
            load_tile(kbase, vbase, tb + STEP, t1, ktok0, g, i, ka, va);
            compute_tile<NRB>(kb2, vb2, qb, tb, t1, g, sl2, m, l, acc);
            tb += STEP;
            if (tb >= t1) break;
        }
    }

    // Row sums over the four lane groups, then hand the wave state to LDS.
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        l[r] += __shfl_xor(l[r], 16);
        l[r] += __shfl_xor(l[r], 32);
        const int row = r * 16 + i;
        if (row < nr) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s_acc[wave][row][8 * (4 * g + ii) + e] = acc[r][e][ii];
            if (g == 0) {
                s_m[wave][row] = m[r];
                s_l[wave][row] = l[r];
            }
        }
    }
    __syncthreads();

    for (int x = tid; x < nr * D; x += NW * 64) {
        const int row = x / D, d = x % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][row]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float a = fast_exp2(s_m[w][row] - M);
                L = fmaf(s_l[w][row], a, L);
                A = fmaf(s_acc[w][row][d], a, A);
            }
        }
        const float o = (L > 0.f) ? A / L : 0.f;
        const float lse = (L > 0.f) ? (M + __log2f(L)) * kLn2f : -INFINITY;
        const int64_t orow = (int64_t)b * p.Hq + h0 + row;
        if (p.direct) {
            store_out(p.out, orow * D + d, o, p.out_bf16);
            if (d == 0 && p.lse_out) p.lse_out[orow] = lse;
        } else {
            const int64_t slot = orow * p.part_stride + p.part_offset + split;
            p.o_part[slot * D + d] = o;
            if (d == 0) p.lse_part[slot] = lse;
        }
    }
}

}  // namespace

int mfma_rows_per_block(int G) { return G > 16 ? 32 : 16; }

hipError_t launch_partial_mfma(const PartialParams& p, hipStream_t stream) {
    const int G = p.Hq / p.Hkv;
    const int rows = mfma_rows_per_block(G);
    if (p.row_blocks != (G + rows - 1) / rows) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.row_blocks * p.n_splits));
    if (rows == 16)
        hipLaunchKernelGGL(partial_mfma_kernel<1>, grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(partial_mfma_kernel<2>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace fd
